"""The whole mixer (mono_mixer_forward) against the oracle's mixer, and the
whole path's determinism."""
import numpy as np
import pytest

from learned_sparse_causal_amd import binding, configs, synth
from parity import (NEAR_TIE, check_sel_invariants, dev, host, index_to_host, say, small_inputs,
                    torch)

pytestmark = pytest.mark.gpu


def run_mixer(cfg, inp):
    t = torch()
    cos, sin = binding.device_rope(cfg)
    delta, stats, ws = binding.mixer_forward(
        cfg, dev(inp["x"], cfg.dtype), dev(inp["w_qkv"], cfg.dtype), dev(inp["w_o"], cfg.dtype),
        t.from_numpy(inp["codebooks"]).cuda(), cos, sin)
    t.cuda.synchronize()
    views = binding.mixer_views(cfg, ws)
    res = dict(delta=host(delta), stats=host(stats), q=host(views["q"]), k=host(views["k"]),
               sel=host(views["sel"]), index=index_to_host(views["index"]))
    return res


@pytest.mark.parametrize("cfg", [configs.TINY, configs.SMALL, configs.ALL_ELIGIBLE],
                         ids=lambda c: c.name)
def test_mixer_parity(orc, cfg):
    say("[mixer] %s" % cfg.name)
    inp = synth.mixer_inputs(cfg)
    gpu = run_mixer(cfg, inp)
    c, s = orc.rope_table(cfg.T, cfg.d)
    ref = orc.mixer(orc.Shape.of(**cfg.shape_kw()), inp["x"], inp["w_qkv"], inp["w_o"],
                    inp["codebooks"], c, s, cfg.dtype)
    # projections: one rounding of the same product; accumulation order may
    # move a value by one unit in the last place
    for name in ("q", "k"):
        g, r = gpu[name], ref[name]
        rel = np.abs(g.astype(np.float64) - r) / np.maximum(np.abs(r), 1e-30)
        bound = 2.0 ** -7 if cfg.dtype == "bf16" else 1e-5
        assert rel.max() <= bound, (name, rel.max())
        frac = (g != r).mean()
        say("  %s elements differing from the oracle's rounding: %.2e" % (name, frac))
    # stats = total overflow and max load of the GPU's own index
    assert gpu["stats"][0] == gpu["index"]["overflow"].sum()
    assert gpu["stats"][1] == gpu["index"]["load"].max()
    check_sel_invariants(cfg, gpu["sel"], gpu["index"])
    # routes: equal unless a near-tie, or the route's own query row was
    # rounded differently by the projection
    g_sel = gpu["sel"].reshape(-1, cfg.R)
    o_sel = ref["sel"]
    qdiff = (gpu["q"] != ref["q"]).any(-1)                       # [B, T, Hq]
    qdiff = qdiff.transpose(0, 2, 1).reshape(-1)
    mism = (g_sel != o_sel).any(-1)
    tie = ref["gaps"].min(-1) < NEAR_TIE
    kdiff_bg = (gpu["k"] != ref["k"]).any(axis=(1, 3))          # [B, Hkv]
    route_bg = np.repeat(np.arange(cfg.B)[:, None] * cfg.Hkv + np.arange(cfg.Hq)[None, :] // cfg.G,
                         cfg.T, axis=1).reshape(-1)
    krounded = kdiff_bg.reshape(-1)[route_bg]
    unexplained = mism & ~tie & ~qdiff & ~krounded
    assert not unexplained.any(), np.nonzero(unexplained)[0][:10]
    frac = mism.mean()
    say("  routes differing: %d of %d (%.3g%%)" % (mism.sum(), mism.size, 100 * frac))
    assert frac <= (1e-4 if cfg.dtype == "f32" else 1e-3)
    # delta on the rows whose routes agree in every head
    row_ok = ~mism.reshape(cfg.B, cfg.Hq, cfg.T).any(1)        # [B, T]
    err = np.abs(gpu["delta"].astype(np.float64) - ref["delta"])
    if cfg.dtype == "f32":
        e = err[row_ok].max()
        say("  delta max abs error %.3g" % e)
        assert e <= 1e-4
    else:
        for b in range(cfg.B):
            e = err[b][row_ok[b]].max() / np.abs(ref["delta"][b]).max()
            say("  delta max relative error %.3g" % e)
            assert e <= 2e-2


def test_whole_path_deterministic():
    cfg = configs.SMALL
    say("[mixer] determinism")
    inp = synth.mixer_inputs(cfg)
    a = run_mixer(cfg, inp)
    b = run_mixer(cfg, inp)
    assert np.array_equal(a["delta"].view(np.uint32), b["delta"].view(np.uint32))
    assert np.array_equal(a["sel"], b["sel"])
