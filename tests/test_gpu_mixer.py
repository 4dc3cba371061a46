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
    # projections: the oracle rounds the exact product once; the GPU rounds an
    # fp32 accumulation, whose error is bounded by W * 2^-24 * sum|x_i w_i|
    # (forward error of a W-term dot product), so the two may differ by one
    # unit in the last place of the stored value (at most 2^-7 of it in bf16)
    # plus that bound
    x64 = np.abs(inp["x"].astype(np.float64)).reshape(-1, cfg.W)
    mag = x64 @ np.abs(inp["w_qkv"].astype(np.float64))
    nq, nk = cfg.Hq * cfg.d, cfg.Hkv * cfg.d
    unit = 2.0 ** -7 if cfg.dtype == "bf16" else 2.0 ** -23
    for name, cols in (("q", slice(0, nq)), ("k", slice(nq, nq + nk))):
        g, r = gpu[name].reshape(-1, cols.stop - cols.start), ref[name].reshape(
            -1, cols.stop - cols.start)
        bound = unit * np.maximum(np.abs(g), np.abs(r)) + cfg.W * 2.0 ** -24 * mag[:, cols]
        over = np.abs(g.astype(np.float64) - r) > bound
        assert not over.any(), "%s: %d elements beyond one ulp + accumulation bound" % (name, over.sum())
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
