"""The whole mixer (mono_mixer_forward) against the oracle, and the whole
path's determinism.

The projections are checked against the oracle's exact products within one
rounding plus the fp32 accumulation bound.  Routing is then compared stage
by stage on the GPU's own projected q and k (the oracle indexes and routes
exactly the bytes the GPU routed on), so routing parity is bit for bit with
the same near-tie rule and 0.01 % cap as the standalone calls; the delta is
compared with the oracle's attention on the GPU's q, k, v, projected by W_o
in fp64."""
import numpy as np
import pytest

from learned_sparse_causal_amd import binding, configs, synth
from parity import (BF16_RTOL, F32_ATOL, check_sel_invariants, compare_index, compare_sel, dev,
                    host, index_to_host, say, torch)

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
               v=host(views["v"]), sel=host(views["sel"]), index=index_to_host(views["index"]))
    return res


def exact_projections(cfg, inp):
    """x W_qkv in fp64, split into q, k, v."""
    x64 = inp["x"].astype(np.float64).reshape(-1, cfg.W)
    prod = x64 @ inp["w_qkv"].astype(np.float64)
    mag = np.abs(x64) @ np.abs(inp["w_qkv"].astype(np.float64))
    return prod, mag


@pytest.mark.parametrize("cfg", [configs.TINY, configs.SMALL, configs.ALL_ELIGIBLE],
                         ids=lambda c: c.name)
def test_mixer_parity(orc, cfg):
    say("[mixer] %s" % cfg.name)
    inp = synth.mixer_inputs(cfg)
    gpu = run_mixer(cfg, inp)
    # projections: the GPU rounds an fp32 accumulation of W products once to
    # the activation dtype.  Against the exact product that is at most one
    # unit in the last place of the stored value (2^-7 relative in bf16,
    # 2^-23 in fp32) plus the forward error bound of a W-term fp32 dot
    # product, about W * 2^-24 * sum |x_i w_i|.
    prod, mag = exact_projections(cfg, inp)
    nq, nk = cfg.Hq * cfg.d, cfg.Hkv * cfg.d
    unit = 2.0 ** -7 if cfg.dtype == "bf16" else 2.0 ** -23
    for name, cols in (("q", slice(0, nq)), ("k", slice(nq, nq + nk)),
                       ("v", slice(nq + nk, nq + 2 * nk))):
        g = gpu[name].reshape(-1, cols.stop - cols.start).astype(np.float64)
        r = prod[:, cols]
        bound = unit * np.abs(g) + 1.01 * cfg.W * 2.0 ** -24 * mag[:, cols]
        over = np.abs(g - r) > bound
        assert not over.any(), "%s: %d elements beyond the rounding bound" % (name, over.sum())
    # stats = total overflow and max load of the GPU's own index
    assert gpu["stats"][0] == gpu["index"]["overflow"].sum()
    assert gpu["stats"][1] == gpu["index"]["load"].max()
    check_sel_invariants(cfg, gpu["sel"], gpu["index"])

    # stage parity on the GPU's own projections
    c, s = orc.rope_table(cfg.T, cfg.d)
    sh = orc.Shape.of(**cfg.shape_kw())
    ref_idx = orc.build_index(sh, gpu["k"], c, s, inp["codebooks"])
    bad_bg = compare_index(cfg, gpu["index"], ref_idx)
    ref_sel, gaps = orc.route(sh, gpu["q"], c, s, inp["codebooks"], ref_idx)
    excused = compare_sel(cfg, gpu["sel"], ref_sel, gaps, bad_bg)
    say("  routes excused as near-ties: %d of %d" % (excused, cfg.routes))

    # delta: oracle attention on the GPU's q, k, v with the oracle's
    # selection, projected in fp64; rows with an excused route are skipped
    o = orc.attention(sh, gpu["q"], gpu["k"], gpu["v"], c, s, ref_sel)
    o = o.reshape(cfg.B, cfg.Hq, cfg.T, cfg.d).transpose(0, 2, 1, 3).reshape(cfg.B * cfg.T, -1)
    ref_delta = (o @ inp["w_o"].astype(np.float64)).reshape(cfg.B, cfg.T, cfg.W)
    mism = (gpu["sel"].reshape(-1, cfg.R) != ref_sel).any(-1)
    row_ok = ~mism.reshape(cfg.B, cfg.Hq, cfg.T).any(1)          # [B, T]
    err = np.abs(gpu["delta"].astype(np.float64) - ref_delta)
    if cfg.dtype == "f32":
        e = err[row_ok].max()
        say("  delta max abs error %.3g" % e)
        assert e <= F32_ATOL
    else:
        for b in range(cfg.B):
            e = err[b][row_ok[b]].max() / np.abs(ref_delta[b]).max()
            say("  delta max relative error %.3g" % e)
            assert e <= BF16_RTOL


def test_whole_path_deterministic():
    cfg = configs.SMALL
    say("[mixer] determinism")
    inp = synth.mixer_inputs(cfg)
    a = run_mixer(cfg, inp)
    b = run_mixer(cfg, inp)
    assert np.array_equal(a["delta"].view(np.uint32), b["delta"].view(np.uint32))
    assert np.array_equal(a["sel"], b["sel"])
