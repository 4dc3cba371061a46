"""Host-only checks of the C ABI: the library loads, exports every function the
header declares, validates arguments on the host, and its rotary table equals
the oracle's bit for bit.  No GPU call is made here."""
import ctypes
import re

import numpy as np
import pytest

from learned_sparse_causal_amd import binding, configs


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def declared_functions():
    src = open(binding.HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mono_[a-z_]+)\s*\(", src)))


def test_header_symbols_exported(lib):
    names = declared_functions()
    assert "mono_build_index" in names and "mono_route" in names
    assert "mono_selected_attention" in names and "mono_mixer_forward" in names
    for n in names:
        assert hasattr(lib, n), n


def test_rope_table_matches_oracle(orc):
    for T, d in ((384, 64), (4096, 64), (1000, 128)):
        c1, s1 = binding.rope_table(T, d)
        c2, s2 = orc.rope_table(T, d)
        assert np.array_equal(c1.view(np.uint32), c2.view(np.uint32))
        assert np.array_equal(s1.view(np.uint32), s2.view(np.uint32))


def test_rope_table_argument_errors(lib):
    buf = np.zeros(8, np.float32)
    assert lib.mono_rope_table(4, 4, 10000.0, None, buf.ctypes.data) == 1
    assert lib.mono_rope_table(0, 4, 10000.0, buf.ctypes.data, buf.ctypes.data) == 2
    assert lib.mono_rope_table(4, 3, 10000.0, buf.ctypes.data, buf.ctypes.data) == 2


def cfg_status(lib, cfg, **over):
    c = binding.make_config(cfg)
    for k, v in over.items():
        setattr(c, k, v)
    # NULL data pointers: a valid shape reports MONO_ERR_NULL, an invalid one
    # its shape/support error, and nothing reaches the GPU either way.
    idx = binding.MonoIndex()
    return lib.mono_build_index(ctypes.byref(c), None, None, None, None, ctypes.byref(idx), None,
                                0, None)


def test_validation_codes(lib):
    cfg = configs.SMALL
    assert cfg_status(lib, cfg) == 1                                     # NULL pointers
    assert cfg_status(lib, cfg, seq_len=4000) == 2                       # T % beta
    assert cfg_status(lib, cfg, n_q_heads=6, n_kv_heads=4) == 2          # Hq % Hkv
    assert cfg_status(lib, cfg, n_components=3) == 2                     # d % P (64 % 3)
    assert cfg_status(lib, cfg, capacity=0) == 2
    assert cfg_status(lib, cfg, n_local=0) == 2
    assert cfg_status(lib, cfg, head_dim=96) == 3                        # unsupported d
    assert cfg_status(lib, cfg, block_size=32) == 3                      # unsupported beta
    assert cfg_status(lib, cfg, n_components=4) == 3                     # P > 2
    assert cfg_status(lib, cfg, codes_per_component=65) == 3
    assert cfg_status(lib, cfg, n_probes=17) == 3
    assert cfg_status(lib, cfg, n_remote=17) == 3                        # search with R > 16
    assert cfg_status(lib, cfg, dtype=7) == 3
    # R > 16 is fine when every query bypasses the search
    assert cfg_status(lib, configs.ALL_ELIGIBLE) == 1


def test_workspace_sizes(lib):
    for cfg in configs.ALL.values():
        c = binding.make_config(cfg)
        assert lib.mono_workspace_bytes(ctypes.byref(c), binding.WS_BUILD) == 0
        assert lib.mono_workspace_bytes(ctypes.byref(c), binding.WS_ROUTE) == 0
        attn = lib.mono_workspace_bytes(ctypes.byref(c), binding.WS_ATTENTION)
        es = 2 if cfg.dtype == "bf16" else 4
        nent = cfg.B * cfg.Hq * cfg.T * cfg.R
        # per (query, slot): its rank in its bin, its list row, and its
        # partial row (which carries the row's log-sum-exp in its low bits)
        assert attn >= nent * (cfg.d * es + 8)
        mix = lib.mono_workspace_bytes(ctypes.byref(c), binding.WS_MIXER)
        assert mix > attn
        cal = lib.mono_workspace_bytes(ctypes.byref(c), binding.WS_CALIBRATE)
        assert cal == cfg.Hkv * cfg.P * 2 * cfg.B * cfg.NB * 4
        dense = lib.mono_workspace_bytes(ctypes.byref(c), binding.WS_DENSE)
        assert dense >= cfg.B * cfg.T * (cfg.Hq + cfg.Hkv) * cfg.d * es
        off = binding.mixer_layout(cfg)
        assert off == sorted(off) and all(o % 256 == 0 for o in off)
    bad = binding.make_config(configs.SMALL)
    bad.seq_len = 100
    assert lib.mono_workspace_bytes(ctypes.byref(bad), binding.WS_ATTENTION) == 0


def test_attention_and_mixer_argument_errors(lib):
    cfg = configs.TINY
    c = binding.make_config(cfg)
    assert lib.mono_selected_attention(ctypes.byref(c), None, None, None, None, None, None, None,
                                       None, 0, None) == 1
    one = ctypes.c_void_p(256)   # never dereferenced: the size check fails first
    need = lib.mono_workspace_bytes(ctypes.byref(c), binding.WS_ATTENTION)
    assert lib.mono_selected_attention(ctypes.byref(c), one, one, one, one, one, one, one, one,
                                       need - 1, None) == 4
    m = binding.make_config(cfg)
    m.width = 100                                                         # Hq*d != W
    assert lib.mono_mixer_forward(ctypes.byref(m), one, one, one, one, one, one, one, None, one,
                                  1 << 40, None) == 2
    need = lib.mono_workspace_bytes(ctypes.byref(c), binding.WS_DENSE)
    assert lib.mono_dense_attention(ctypes.byref(c), one, one, one, one, one, None, one, need,
                                    None) == 1
    assert lib.mono_dense_attention(ctypes.byref(c), one, one, one, one, one, one, one, need - 1,
                                    None) == 4
    assert lib.mono_status_string(4) == b"workspace too small"


def test_calibrate_argument_errors(lib):
    cfg = configs.TINY
    c = binding.make_config(cfg)
    one = ctypes.c_void_p(256)   # never dereferenced: validation fails first
    need = lib.mono_workspace_bytes(ctypes.byref(c), binding.WS_CALIBRATE)
    assert lib.mono_calibrate_codebooks(ctypes.byref(c), None, one, 3, one, need, None) == 1
    assert lib.mono_calibrate_codebooks(ctypes.byref(c), one, one, -1, one, need, None) == 2
    assert lib.mono_calibrate_codebooks(ctypes.byref(c), one, one, 10001, one, need, None) == 2
    assert lib.mono_calibrate_codebooks(ctypes.byref(c), one, one, 3, one, need - 1, None) == 4


def test_decode_argument_errors(lib):
    cfg = configs.TINY
    c = binding.make_config(cfg)
    one = ctypes.c_void_p(256)   # never dereferenced: validation fails first
    idx = binding.MonoIndex(*(256,) * 6)
    # token count beyond the cache, indexed blocks beyond the token count
    assert lib.mono_decode_index(ctypes.byref(c), one, one, one, one, ctypes.byref(idx), 0,
                                 cfg.T + 1, None) == 2
    assert lib.mono_decode_index(ctypes.byref(c), one, one, one, one, ctypes.byref(idx), 3,
                                 2 * cfg.beta, None) == 2
    assert lib.mono_decode_index(ctypes.byref(c), one, one, one, one, ctypes.byref(idx), -1,
                                 2 * cfg.beta, None) == 2
    assert lib.mono_decode_index(ctypes.byref(c), None, one, one, one, ctypes.byref(idx), 0,
                                 cfg.T, None) == 1
    # position outside the cache, missing outputs
    assert lib.mono_decode_step(ctypes.byref(c), one, one, one, one, one, one, ctypes.byref(idx),
                                cfg.T, one, one, None) == 2
    assert lib.mono_decode_step(ctypes.byref(c), one, one, one, one, one, one, ctypes.byref(idx),
                                -1, one, one, None) == 2
    assert lib.mono_decode_step(ctypes.byref(c), one, one, one, one, one, one, ctypes.byref(idx),
                                0, None, one, None) == 1


def test_noalloc_argument_errors(lib):
    """mono_routed_attention_noalloc validates on the host before touching the
    device: NULL pointers, bad shapes, and a workload whose attention
    workspace exceeds the static scratch (MONO_ERR_SCRATCH)."""
    small = binding.make_config(configs.SMALL)
    big = binding.make_config(configs.SWEEP_32K)
    idx = binding.MonoIndex(*([1] * 6))
    p = ctypes.c_void_p(1)
    fn = lib.mono_routed_attention_noalloc
    assert fn(None, p, p, p, p, p, p, ctypes.byref(idx), p, p, None, None) == 1
    assert fn(ctypes.byref(small), None, p, p, p, p, p, ctypes.byref(idx), p, p, None, None) == 1
    assert fn(ctypes.byref(small), p, p, p, p, p, p, None, p, p, None, None) == 1
    bad = binding.make_config(configs.SMALL.with_(T=4100))
    assert fn(ctypes.byref(bad), p, p, p, p, p, p, ctypes.byref(idx), p, p, None, None) == 2
    assert lib.mono_workspace_bytes(ctypes.byref(big), binding.WS_ATTENTION) > \
        binding.NOALLOC_SCRATCH_BYTES
    assert fn(ctypes.byref(big), p, p, p, p, p, p, ctypes.byref(idx), p, p, None, None) == 6
    assert b"scratch" in lib.mono_status_string(6)
