"""GPU dense causal attention (mono_dense_attention) against the oracle's
textbook dense causal softmax (fp32 within 1e-4 max abs, bf16 within 2e-2 max
relative per (batch, head)), and against the routed path on the all-eligible
configuration, where both compute the same dense causal attention."""
import numpy as np
import pytest

from learned_sparse_causal_amd import binding, configs
from parity import check_attention, host, sample_routes, say, small_inputs, torch

pytestmark = pytest.mark.gpu


def dense_reference(orc, cfg, inp, route_ids):
    """fp64 dense causal attention for route ids (b*Hq + h)*T + t."""
    c, s = orc.rope_table(cfg.T, cfg.d)
    t = route_ids % cfg.T
    bh = route_ids // cfg.T
    ref = np.empty((len(route_ids), cfg.d))
    for x in np.unique(bh):
        b, h = divmod(int(x), cfg.Hq)
        g = h // cfg.G
        m = bh == x
        ref[m] = orc.dense_causal_attention(inp["q"][b, :, h], inp["k"][b, :, g],
                                            inp["v"][b, :, g], c, s, t[m])
    return ref


CFGS = [configs.TINY,
        configs.SMALL.with_(name="gqa_bf16_T2048", T=2048, Hq=6, Hkv=2),
        # T % 128 == 64: the last query tile holds 64 rows
        configs.SMALL.with_(name="ragged_bf16_T1088", T=1088, Hq=3, Hkv=1),
        configs.SMALL.with_(name="d128_bf16_T2048", d=128, beta=128, T=2048, Hq=4, Hkv=1),
        configs.SMALL.with_(name="d128_f32_T1024", d=128, T=1024, Hq=2, Hkv=2, dtype="f32"),
        configs.SMALL.with_(name="single_tile_f32_T64", T=64, Hq=2, Hkv=1, L=1, dtype="f32"),
        configs.SMALL.with_(name="batch2_bf16_T1024", B=2, T=1024, Hq=4, Hkv=2)]


@pytest.mark.parametrize("cfg", CFGS, ids=lambda c: c.name)
def test_dense_parity(orc, cfg):
    say("[dense] %s" % cfg.name)
    inp, d = small_inputs(cfg)
    cos, sin = binding.device_rope(cfg)
    out = host(binding.dense_attention(cfg, d["q"], d["k"], d["v"], cos, sin))
    ids = np.arange(cfg.routes) if cfg.routes <= 20000 else sample_routes(cfg, 20000, seed=7)
    ref = dense_reference(orc, cfg, inp, ids)
    say("  error %.3g" % check_attention(cfg, out, ref, ids))


def test_dense_parity_32k_sampled(orc):
    """The timed workload (T = 32768, 16 heads), in the launch configuration
    the benchmark times: sampled rows, the last tile of every head included."""
    cfg = configs.SWEEP_32K
    say("[dense] %s sampled" % cfg.name)
    inp, d = small_inputs(cfg)
    cos, sin = binding.device_rope(cfg)
    out = host(binding.dense_attention(cfg, d["q"], d["k"], d["v"], cos, sin))
    rng = np.random.default_rng(8)
    ids = []
    for h in range(cfg.Hq):
        t = np.concatenate([rng.choice(cfg.T, 24, replace=False), [0, 1, 63, 64, cfg.T - 1]])
        ids.append(h * cfg.T + t)
    ids = np.unique(np.concatenate(ids))
    ref = dense_reference(orc, cfg, inp, ids)
    say("  error %.3g" % check_attention(cfg, out, ref, ids))


def test_dense_equals_routed_all_eligible(orc):
    """All remote blocks eligible (R = NB - L): the routed path (index build,
    route, selected-set attention) and the dense kernel compute the same dense
    causal attention; both are checked against the oracle on sampled rows and
    against each other on every row."""
    cfg = configs.ALL_ELIGIBLE
    say("[dense] %s routed vs dense" % cfg.name)
    t = torch()
    inp, d = small_inputs(cfg)
    cos, sin = binding.device_rope(cfg)
    cb = t.from_numpy(inp["codebooks"]).cuda()
    idx = binding.build_index(cfg, d["k"], cos, sin, cb)
    sel = binding.route(cfg, d["q"], cos, sin, cb, idx)
    routed = host(binding.selected_attention(cfg, d["q"], d["k"], d["v"], cos, sin, sel))
    dense = host(binding.dense_attention(cfg, d["q"], d["k"], d["v"], cos, sin))
    ids = sample_routes(cfg, 3000, seed=9)
    ref = dense_reference(orc, cfg, inp, ids)
    e_dense = check_attention(cfg, dense, ref, ids)
    e_routed = check_attention(cfg, routed, ref, ids)
    worst = 0.0
    for h in range(cfg.Hq):
        diff = np.abs(routed[0, :, h].astype(np.float64) - dense[0, :, h]).max()
        worst = max(worst, diff / np.abs(dense[0, :, h]).max())
    say("  vs oracle: dense %.3g routed %.3g; routed vs dense max relative %.3g"
        % (e_dense, e_routed, worst))
    assert worst <= 2e-2


def test_dense_is_deterministic():
    cfg = configs.SMALL.with_(name="det", T=2048, Hq=4, Hkv=2)
    _, d = small_inputs(cfg)
    cos, sin = binding.device_rope(cfg)
    a = binding.dense_attention(cfg, d["q"], d["k"], d["v"], cos, sin)
    b = binding.dense_attention(cfg, d["q"], d["k"], d["v"], cos, sin)
    torch().cuda.synchronize()
    assert torch().equal(a, b)
