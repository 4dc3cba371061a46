"""GPU spherical codebook calibration (mono_calibrate_codebooks) against the
oracle: calibrated codebooks bit for bit, and the held-out index built with
them equal to the oracle's, on concentrated and plain random keys."""
import numpy as np
import pytest

from learned_sparse_causal_amd import binding, configs, synth
from parity import compare_index, dev, host, index_to_host, say, torch

pytestmark = pytest.mark.gpu


def calibrate_both(orc, cfg, k_train, cb0, n_iter):
    """GPU: index of the training keys, then calibration; oracle: the same
    from the same host keys."""
    t = torch()
    cos, sin = binding.device_rope(cfg)
    idx = binding.build_index(cfg, dev(k_train, cfg.dtype), cos, sin, t.from_numpy(cb0).cuda())
    cb_g = t.from_numpy(cb0.copy()).cuda()
    binding.calibrate_codebooks(cfg, idx["kbar"], cb_g, n_iter)
    c, s = orc.rope_table(cfg.T, cfg.d)
    o_idx = orc.build_index(orc.Shape.of(**cfg.shape_kw()), k_train, c, s, cb0)
    assert np.array_equal(host(idx["kbar"]).view(np.uint32), o_idx["kbar"].view(np.uint32))
    cb_o = orc.calibrate(o_idx["kbar"], cb0, n_iter)
    return host(cb_g), cb_o


CASES = [
    # (name, cfg of the training split, key kind, rounds)
    ("concentrated_ds32_K8", configs.SMALL.with_(B=4, T=2048, Hq=2, Hkv=2, K=8, cap=8), "conc", 10),
    ("concentrated_f32_ds32_K16", configs.SMALL.with_(B=2, T=2048, Hq=2, Hkv=2, dtype="f32"),
     "conc", 6),
    ("random_ds64_P1_K64", configs.SMALL.with_(B=2, T=4096, Hq=4, Hkv=2, P=1, K=64), "rand", 8),
    ("random_ds64_d128_K32", configs.SMALL.with_(B=2, T=4096, d=128, beta=128, Hq=2, Hkv=1, K=32),
     "rand", 5),
    ("concentrated_ds128_P1_K16", configs.SMALL.with_(B=3, T=2048, d=128, Hq=2, Hkv=1, P=1, K=16),
     "conc", 7),
    ("capacity_shape_T8192", configs.ALL_ELIGIBLE.with_(B=4), "conc", 10),
]


def training_keys(cfg, kind):
    if kind == "conc":
        return synth.concentrated_keys(cfg, seed=51)
    inp = synth.qkv(cfg)
    return inp["k"], inp["codebooks"]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_calibration_parity(orc, case):
    name, cfg, kind, n_iter = case
    say("[calibrate] %s" % name)
    k_train, cb0 = training_keys(cfg, kind)
    cb_g, cb_o = calibrate_both(orc, cfg, k_train, cb0, n_iter)
    assert np.array_equal(cb_g.view(np.uint32), cb_o.view(np.uint32)), \
        "max abs %g" % np.abs(cb_g - cb_o).max()
    say("  %d codes moved" % int((np.abs(cb_g - cb0).max(-1) > 0).sum()))


def test_calibration_zero_rounds_and_determinism(orc):
    cfg = configs.SMALL.with_(B=2, T=2048, Hq=2, Hkv=2)
    k_train, cb0 = synth.concentrated_keys(cfg, seed=52)
    cb_g, _ = calibrate_both(orc, cfg, k_train, cb0, 0)
    assert np.array_equal(cb_g, cb0)
    a, _ = calibrate_both(orc, cfg, k_train, cb0, 4)
    b, _ = calibrate_both(orc, cfg, k_train, cb0, 4)
    assert np.array_equal(a, b)


def test_calibrated_held_out_index(orc):
    """Capacity workload: codebooks calibrated on four training sequences of
    8192 tokens; the held-out sequence's index built with them on the GPU
    equals the oracle's, and overflow and maximum load drop."""
    train_cfg = configs.ALL_ELIGIBLE.with_(B=4)
    cfg = configs.ALL_ELIGIBLE
    say("[calibrate] held-out index, %s" % cfg.name)
    t = torch()
    k_train, cb0 = synth.concentrated_keys(train_cfg, seed=53)
    k_test, _ = synth.concentrated_keys(cfg, seed=54)
    cb_g, cb_o = calibrate_both(orc, train_cfg, k_train, cb0, 10)
    cos, sin = binding.device_rope(cfg)
    kd = dev(k_test, cfg.dtype)
    before = index_to_host(binding.build_index(cfg, kd, cos, sin, t.from_numpy(cb0).cuda()))
    after = index_to_host(binding.build_index(cfg, kd, cos, sin, t.from_numpy(cb_g).cuda()))
    c, s = orc.rope_table(cfg.T, cfg.d)
    o_after = orc.build_index(orc.Shape.of(**cfg.shape_kw()), k_test, c, s, cb_o)
    compare_index(cfg, after, o_after, excuse=False)
    say("  overflow %d -> %d, max load %d -> %d" % (before["overflow"].sum(),
                                                    after["overflow"].sum(),
                                                    before["load"].max(), after["load"].max()))
    assert before["overflow"].sum() > 0 and after["overflow"].sum() < before["overflow"].sum()
    assert after["load"].max() < before["load"].max()
