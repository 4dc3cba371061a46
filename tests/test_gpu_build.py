"""GPU index build (mono_build_index) against the oracle: block summaries,
addresses, posting lists, loads and overflow bit for bit."""
import numpy as np
import pytest

from learned_sparse_causal_amd import binding, configs, synth
from parity import compare_index, dev, host, index_to_host, say, small_inputs, torch

pytestmark = pytest.mark.gpu


def run_build(cfg, k_dev, codebooks):
    t = torch()
    cos, sin = binding.device_rope(cfg)
    idx = binding.build_index(cfg, k_dev, cos, sin, t.from_numpy(codebooks).cuda())
    t.cuda.synchronize()
    return index_to_host(idx)


def oracle_build(orc, cfg, k, codebooks):
    c, s = orc.rope_table(cfg.T, cfg.d)
    return orc.build_index(orc.Shape.of(**cfg.shape_kw()), k, c, s, codebooks)


CFGS = [configs.TINY, configs.SMALL, configs.ALL_ELIGIBLE, configs.sweep(4096),
        configs.SWEEP_32K,
        configs.SMALL.with_(name="d128_beta64_f32", d=128, Hq=4, Hkv=2, dtype="f32"),
        configs.SMALL.with_(name="d128_beta128_P1", d=128, beta=128, P=1, K=64, Hq=2, Hkv=2),
        configs.SMALL.with_(name="beta128_K3_ragged", beta=128, K=3, T=8192 + 128, Hq=2, Hkv=2)]


@pytest.mark.parametrize("cfg", CFGS, ids=lambda c: c.name)
def test_build_index_parity(orc, cfg):
    say("[build] %s" % cfg.name)
    inp, d = small_inputs(cfg)
    gpu = run_build(cfg, d["k"], inp["codebooks"])
    ref = oracle_build(orc, cfg, inp["k"], inp["codebooks"])
    bad = compare_index(cfg, gpu, ref)
    say("  excused (b, g) with a near-tie address: %d" % len(bad))


def test_build_index_parity_large(orc):
    cfg = configs.LARGE
    say("[build] %s" % cfg.name)
    d = synth.qkv_device(cfg)
    gpu = run_build(cfg, d["k"], d["codebooks"])
    ref = oracle_build(orc, cfg, host(d["k"]), d["codebooks"])
    bad = compare_index(cfg, gpu, ref)
    say("  overflow total %d, max load %d, excused %d" % (gpu["overflow"].sum(), gpu["load"].max(),
                                                          len(bad)))


@pytest.mark.parametrize("kind,cap", [("one_address", 8), ("one_address", 1), ("two_clusters", 4),
                                      ("two_clusters", 64)])
def test_build_index_overflow_stress(orc, kind, cap):
    cfg = configs.SMALL.with_(name="stress", T=4096, Hq=4, Hkv=4, cap=cap)
    say("[build stress] %s cap=%d" % (kind, cap))
    k, cb = synth.stress_keys(cfg, kind)
    gpu = run_build(cfg, dev(k, cfg.dtype), cb)
    ref = oracle_build(orc, cfg, k, cb)
    compare_index(cfg, gpu, ref)
    if kind == "one_address":
        assert (gpu["addr"] == 0).all()
        assert (gpu["overflow"] == cfg.NB - min(cap, cfg.NB)).all()
    else:
        assert (gpu["overflow"] == 2 * max(0, cfg.NB // 2 - cap)).all()


@pytest.mark.parametrize("cap", [1, 2, 10_000])
def test_build_index_capacity_extremes(orc, cap):
    cfg = configs.sweep(4096).with_(name="cap%d" % cap, cap=cap, K=4)   # 16 addresses, 64 blocks
    say("[build cap] %d" % cap)
    inp, d = small_inputs(cfg)
    gpu = run_build(cfg, d["k"], inp["codebooks"])
    ref = oracle_build(orc, cfg, inp["k"], inp["codebooks"])
    compare_index(cfg, gpu, ref)
    assert (np.minimum(gpu["load"], cap).sum(-1) + gpu["overflow"] == cfg.NB).all()
