"""The whole step in one call (mono_routed_attention) against the three calls
it fuses (mono_build_index, mono_route, mono_selected_attention): index,
selection and output bitwise equal (the three calls are themselves checked
against the oracle in test_gpu_build, test_gpu_route and test_gpu_attention),
and the stage events it records bracket the stages."""
import numpy as np
import pytest

from learned_sparse_causal_amd import binding, configs, synth
from parity import index_to_host, host, say, small_inputs, torch

pytestmark = pytest.mark.gpu

CFGS = [configs.TINY, configs.SMALL, configs.sweep(4096),
        configs.SMALL.with_(name="gqa_L3_R5", Hq=6, Hkv=2, L=3, R=5),
        configs.SMALL.with_(name="d128_beta128", d=128, beta=128, T=4096, Hq=4, Hkv=1, R=8),
        configs.SMALL.with_(name="d128_beta64_f32", d=128, T=2048, Hq=2, Hkv=2, dtype="f32"),
        configs.SMALL.with_(name="P1_K64_B2", P=1, K=64, B=2, T=2048, Hq=4, Hkv=2),
        configs.ALL_ELIGIBLE]


@pytest.mark.parametrize("cfg", CFGS, ids=lambda c: c.name)
def test_step_equals_separate_calls(cfg):
    say("[step] %s" % cfg.name)
    t = torch()
    inp, d = small_inputs(cfg)
    cos, sin = binding.device_rope(cfg)
    cb = t.from_numpy(inp["codebooks"]).cuda()
    idx = binding.build_index(cfg, d["k"], cos, sin, cb)
    sel = binding.route(cfg, d["q"], cos, sin, cb, idx)
    out = binding.selected_attention(cfg, d["q"], d["k"], d["v"], cos, sin, sel)
    f_idx, f_sel, f_out = binding.routed_attention(cfg, d["q"], d["k"], d["v"], cos, sin, cb)
    a, b = index_to_host(idx), index_to_host(f_idx)
    for name in ("kbar", "addr", "offsets", "entries", "load", "overflow"):
        assert np.array_equal(a[name].view(np.uint32) if a[name].dtype == np.float32 else a[name],
                              b[name].view(np.uint32) if b[name].dtype == np.float32 else b[name]), name
    assert np.array_equal(host(sel), host(f_sel))
    t.cuda.synchronize()
    assert t.equal(out, f_out)


def test_step_stage_events():
    cfg = configs.sweep(8192)
    t = torch()
    d = synth.qkv_device(cfg)
    cos, sin = binding.device_rope(cfg)
    cb = t.from_numpy(d["codebooks"]).cuda()
    ev = [t.cuda.Event(enable_timing=True) for _ in range(4)]
    binding.routed_attention(cfg, d["q"], d["k"], d["v"], cos, sin, cb)   # warm-up
    binding.routed_attention(cfg, d["q"], d["k"], d["v"], cos, sin, cb, stage_events=ev)
    t.cuda.synchronize()
    stages = [ev[i].elapsed_time(ev[i + 1]) for i in range(3)]
    total = ev[0].elapsed_time(ev[3])
    say("  stages ms %s, total %.3f" % (["%.3f" % x for x in stages], total))
    assert all(x > 0 for x in stages)
    assert abs(sum(stages) - total) < 1e-3 * max(1.0, total)
