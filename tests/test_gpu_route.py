"""GPU routing (mono_route) against the oracle: selected block ids bit for
bit, with near-ties (oracle score gap < 1e-5 relative) counted and excused,
plus the stated invariants on every GPU selection."""
import numpy as np
import pytest

from learned_sparse_causal_amd import binding, configs, synth
from parity import (check_sel_invariants, compare_index, compare_sel, dev, host, index_to_host,
                    sample_routes, say, small_inputs, torch)

pytestmark = pytest.mark.gpu


def run_gpu(cfg, q_dev, k_dev, codebooks):
    t = torch()
    cos, sin = binding.device_rope(cfg)
    cb = t.from_numpy(codebooks).cuda()
    idx = binding.build_index(cfg, k_dev, cos, sin, cb)
    sel = binding.route(cfg, q_dev, cos, sin, cb, idx)
    t.cuda.synchronize()
    return index_to_host(idx), host(sel)


def run_oracle(orc, cfg, q, k, codebooks, route_ids=None):
    c, s = orc.rope_table(cfg.T, cfg.d)
    sh = orc.Shape.of(**cfg.shape_kw())
    idx = orc.build_index(sh, k, c, s, codebooks)
    sel, gaps = orc.route(sh, q, c, s, codebooks, idx, route_ids)
    return idx, sel, gaps


CFGS = [configs.TINY, configs.SMALL, configs.ALL_ELIGIBLE, configs.sweep(4096),
        configs.sweep(8192),
        configs.SMALL.with_(name="P1_K64", P=1, K=64, Hq=4, Hkv=2),
        configs.SMALL.with_(name="probes1_R1", n_probes=1, R=1, Hq=2, Hkv=2),
        configs.SMALL.with_(name="probes16_R16_L3", n_probes=16, R=16, L=3, Hq=2, Hkv=1),
        configs.SMALL.with_(name="probes8_R3_K5", n_probes=8, R=3, K=5, Hq=2, Hkv=2),
        configs.SMALL.with_(name="d128_beta128_f32", d=128, beta=128, T=8192, Hq=2, Hkv=1,
                            dtype="f32", n_probes=8, R=8),
        configs.SMALL.with_(name="cap1", cap=1, Hq=4, Hkv=4),
        # 65 blocks: the last route workgroup holds one wave of tokens
        configs.SMALL.with_(name="ragged_T4160_B2", T=4160, B=2, Hq=4, Hkv=2),
        configs.SMALL.with_(name="gqa4_T3136_L3_R3", T=3136, Hq=8, Hkv=2, L=3, R=3, n_probes=3),
        # 4096 addresses: the list offsets take several staging rounds
        configs.SMALL.with_(name="K64_P2_A4096", K=64, Hq=2, Hkv=2),
        # R in 3..8: the two-pass extension scan, with overflowed (unindexed)
        # eligible blocks, and at d 128 in bf16 with one component
        configs.SMALL.with_(name="cap2_R6_probes6", cap=2, R=6, n_probes=6, Hq=2, Hkv=2),
        configs.SMALL.with_(name="d128_bf16_P1_R5", d=128, P=1, K=32, Hq=2, Hkv=1,
                            n_probes=5, R=5),
        # sixteen slots, five of them sentinels
        configs.SMALL.with_(name="probes9_R11_L3", n_probes=9, R=11, L=3, Hq=2, Hkv=2)]


@pytest.mark.parametrize("cfg", CFGS, ids=lambda c: c.name)
def test_route_parity(orc, cfg):
    say("[route] %s" % cfg.name)
    inp, d = small_inputs(cfg)
    g_idx, g_sel = run_gpu(cfg, d["q"], d["k"], inp["codebooks"])
    o_idx, o_sel, gaps = run_oracle(orc, cfg, inp["q"], inp["k"], inp["codebooks"])
    bad = compare_index(cfg, g_idx, o_idx)
    check_sel_invariants(cfg, g_sel, g_idx)
    n = compare_sel(cfg, g_sel, o_sel, gaps, bad)
    say("  excused routes: %d of %d" % (n, cfg.routes))


def test_route_parity_32k_sampled(orc):
    cfg = configs.SWEEP_32K
    say("[route] %s sampled" % cfg.name)
    inp, d = small_inputs(cfg)
    g_idx, g_sel = run_gpu(cfg, d["q"], d["k"], inp["codebooks"])
    ids = sample_routes(cfg, 30000, seed=1, must=[(0, 0), (0, 15)])
    o_idx, o_sel, gaps = run_oracle(orc, cfg, inp["q"], inp["k"], inp["codebooks"], ids)
    bad = compare_index(cfg, g_idx, o_idx)
    check_sel_invariants(cfg, g_sel, g_idx)
    n = compare_sel(cfg, g_sel, o_sel, gaps, bad, route_ids=ids)
    say("  excused routes: %d of %d sampled" % (n, len(ids)))


def test_route_parity_large_sampled(orc):
    """Largest workload: the whole index, and routes of the (b, h) pairs
    (0, 0) and (7, 15) plus random routes (sampled scalar parity)."""
    cfg = configs.LARGE
    say("[route] %s sampled" % cfg.name)
    d = synth.qkv_device(cfg)
    g_idx, g_sel = run_gpu(cfg, d["q"], d["k"], d["codebooks"])
    ids = sample_routes(cfg, 30000, seed=2, must=[(0, 0), (7, 15)])
    q_h = host(d["q"])
    o_idx, o_sel, gaps = run_oracle(orc, cfg, q_h, host(d["k"]), d["codebooks"], ids)
    del q_h
    bad = compare_index(cfg, g_idx, o_idx)
    check_sel_invariants(cfg, g_sel, g_idx)
    n = compare_sel(cfg, g_sel, o_sel, gaps, bad, route_ids=ids)
    say("  excused routes: %d of %d sampled; overflow %d, max load %d" % (
        n, len(ids), g_idx["overflow"].sum(), g_idx["load"].max()))


@pytest.mark.parametrize("R", [2, 5])
def test_route_with_overflowed_eligible_blocks(orc, R):
    """Every block on one address, capacity 1: searched queries see one indexed
    block and pad the rest with -1; bypassed queries take every eligible block."""
    cfg = configs.SMALL.with_(name="one_address_cap1_R%d" % R, cap=1, R=R, L=1, Hq=2, Hkv=2)
    say("[route] %s" % cfg.name)
    k, cb = synth.stress_keys(cfg, "one_address")
    inp = synth.qkv(cfg)
    g_idx, g_sel = run_gpu(cfg, dev(inp["q"], cfg.dtype), dev(k, cfg.dtype), cb)
    o_idx, o_sel, gaps = run_oracle(orc, cfg, inp["q"], k, cb)
    compare_index(cfg, g_idx, o_idx, excuse=False)
    assert np.array_equal(g_sel.reshape(-1, cfg.R), o_sel)
    t = np.arange(cfg.T)
    searched = (t // cfg.beta - cfg.L + 1) > cfg.R
    assert (g_sel[:, :, searched] == np.array([0] + [-1] * (R - 1))).all()


def test_route_tied_extension(orc):
    """Two hot addresses (blocks alternate between them), one probe, R 5:
    the extension fills from blocks of equal sigma, which rank by block."""
    cfg = configs.SMALL.with_(name="two_clusters_R5_probes1", n_probes=1, R=5, L=1, Hq=2,
                              Hkv=2)
    say("[route] %s" % cfg.name)
    k, cb = synth.stress_keys(cfg, "two_clusters")
    inp = synth.qkv(cfg)
    g_idx, g_sel = run_gpu(cfg, dev(inp["q"], cfg.dtype), dev(k, cfg.dtype), cb)
    o_idx, o_sel, gaps = run_oracle(orc, cfg, inp["q"], k, cb)
    bad = compare_index(cfg, g_idx, o_idx, excuse=False)
    check_sel_invariants(cfg, g_sel, g_idx)
    n = compare_sel(cfg, g_sel, o_sel, gaps, bad)
    say("  excused routes: %d of %d" % (n, cfg.routes))


def test_route_deterministic():
    cfg = configs.sweep(8192)
    say("[route] determinism %s" % cfg.name)
    inp, d = small_inputs(cfg)
    a = run_gpu(cfg, d["q"], d["k"], inp["codebooks"])
    b = run_gpu(cfg, d["q"], d["k"], inp["codebooks"])
    for k in a[0]:
        assert np.array_equal(a[0][k], b[0][k]), k
    assert np.array_equal(a[1], b[1])


TIE_CFGS = [configs.SMALL.with_(name="ties_bf16_T4096"),
            configs.sweep(8192).with_(name="ties_sweep_T8192"),
            configs.SMALL.with_(name="ties_probes1_R1", n_probes=1, R=1, Hq=2, Hkv=2),
            configs.SMALL.with_(name="ties_d128_f32_R8", d=128, beta=128, T=8192, Hq=2, Hkv=1,
                                dtype="f32", n_probes=8, R=8),
            configs.SMALL.with_(name="ties_P1_K64_R3", P=1, K=64, Hq=4, Hkv=2, R=3)]


@pytest.mark.parametrize("cfg", TIE_CFGS, ids=lambda c: c.name)
def test_route_exact_ties(orc, cfg):
    """Exact score ties at every kind of decision, which the lowest-index
    rule decides: zeroed key blocks (summary 0, every code score 0: code 0,
    rerank score 0 for every query), zeroed query tokens (every address
    score and rerank score 0: addresses walked in ascending order, lowest
    blocks kept) and duplicated code rows (equal component scores).  The GPU
    must take every such decision as the oracle does: no route is excused."""
    say("[route] %s" % cfg.name)
    inp = synth.tied_inputs(cfg)
    g_idx, g_sel = run_gpu(cfg, dev(inp["q"], cfg.dtype), dev(inp["k"], cfg.dtype),
                           inp["codebooks"])
    o_idx, o_sel, gaps = run_oracle(orc, cfg, inp["q"], inp["k"], inp["codebooks"])
    compare_index(cfg, g_idx, o_idx, excuse=False)
    check_sel_invariants(cfg, g_sel, g_idx)
    tied = int((gaps.min(-1) == 0.0).sum())
    assert tied > 0, "the inputs produced no exact tie at a decision"
    diff = np.nonzero((g_sel.reshape(-1, cfg.R) != o_sel).any(-1))[0]
    assert len(diff) == 0, "%d routes differ (first %s: gpu %s oracle %s gaps %s)" % (
        len(diff), diff[:1], g_sel.reshape(-1, cfg.R)[diff[:1]], o_sel[diff[:1]], gaps[diff[:1]])
    say("  %d routes decided on an exact tie, all equal to the oracle" % tied)
