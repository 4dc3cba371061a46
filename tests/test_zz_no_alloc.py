"""The allocation-free whole step (mono_routed_attention_noalloc, for
callers that cannot allocate device memory) against the workspace entry
point it varies, mono_routed_attention: two calls in a row on the shared
static scratch, the second on a smaller workload, each equal to the
workspace call (index and selection bit for bit, attention output within
the attention tolerance); a workload too large for the scratch is refused
with MONO_ERR_SCRATCH and nothing written."""
import numpy as np
import pytest

from learned_sparse_causal_amd import binding, configs
from parity import BF16_RTOL, F32_ATOL, host, index_to_host, say, small_inputs, torch

pytestmark = pytest.mark.gpu


def both_calls(cfg):
    t = torch()
    inp, d = small_inputs(cfg)
    cos, sin = binding.device_rope(cfg)
    cb = t.from_numpy(inp["codebooks"]).cuda()
    need = binding.workspace_bytes(cfg, binding.WS_ATTENTION)
    assert need <= binding.NOALLOC_SCRATCH_BYTES
    n_idx, n_sel, n_out = binding.routed_attention_noalloc(cfg, d["q"], d["k"], d["v"], cos, sin, cb)
    w_idx, w_sel, w_out = binding.routed_attention(cfg, d["q"], d["k"], d["v"], cos, sin, cb)
    t.cuda.synchronize()
    return (index_to_host(n_idx), host(n_sel), host(n_out)), (index_to_host(w_idx), host(w_sel),
                                                            host(w_out)), need


def check_equal(cfg, got, want):
    g_idx, g_sel, g_out = got
    w_idx, w_sel, w_out = want
    for name in ("kbar", "addr", "offsets", "entries", "load", "overflow"):
        a, b = g_idx[name], w_idx[name]
        if a.dtype == np.float32:
            a, b = a.view(np.uint32), b.view(np.uint32)
        assert np.array_equal(a, b), name
    assert np.array_equal(g_sel, w_sel)
    err = np.abs(g_out.astype(np.float64) - w_out.astype(np.float64))
    if cfg.dtype == "f32":
        assert err.max() <= F32_ATOL
    else:
        assert err.max() <= BF16_RTOL * np.abs(w_out).max()
    return float(err.max())


def test_noalloc_step_twice_then_smaller():
    first = configs.sweep(8192)
    second = configs.SMALL.with_(name="bf16_T2048_gqa", T=2048, Hq=4, Hkv=2, R=3, L=2)
    for cfg in (first, second):
        say("[noalloc] %s" % cfg.name)
        got, want, need = both_calls(cfg)
        e = check_equal(cfg, got, want)
        say("  scratch used %.1f MiB of %d MiB; max |noalloc - workspace| %.3g"
            % (need / 2 ** 20, binding.NOALLOC_SCRATCH_BYTES >> 20, e))


def test_noalloc_refuses_a_workload_beyond_the_scratch():
    t = torch()
    cfg = configs.SWEEP_32K
    assert binding.workspace_bytes(cfg, binding.WS_ATTENTION) > binding.NOALLOC_SCRATCH_BYTES
    cos, sin = binding.device_rope(cfg)
    z = t.zeros((cfg.B, cfg.T, cfg.Hq, cfg.d), dtype=t.bfloat16, device="cuda")
    cb = t.zeros((cfg.Hkv, cfg.P, cfg.K, cfg.d // cfg.P), dtype=t.float32, device="cuda")
    out = t.full((cfg.B, cfg.T, cfg.Hq, cfg.d), 7.0, dtype=t.bfloat16, device="cuda")
    with pytest.raises(binding.MonoError) as e:
        binding.routed_attention_noalloc(cfg, z, z, z, cos, sin, cb, out=out)
    assert e.value.code == 6
    t.cuda.synchronize()
    assert bool((out == 7.0).all())
