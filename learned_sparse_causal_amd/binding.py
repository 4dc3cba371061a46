"""ctypes binding of libmono.so (include/mono.h), with the same call names.

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their device pointers and the current HIP stream are passed to
the C ABI, and a non-OK status raises MonoError.  Every step of the path runs
in the library's kernels; if the library is missing, loading raises.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmono.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "mono.h")

MONO_F32, MONO_BF16 = 0, 1
WS_BUILD, WS_ROUTE, WS_ATTENTION, WS_MIXER, WS_DENSE, WS_CALIBRATE = 0, 1, 2, 3, 4, 5
STATUS = {0: "MONO_OK", 1: "MONO_ERR_NULL", 2: "MONO_ERR_SHAPE", 3: "MONO_ERR_UNSUPPORTED",
          4: "MONO_ERR_WORKSPACE", 5: "MONO_ERR_HIP", 6: "MONO_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 128 << 20       # MONO_NOALLOC_SCRATCH_BYTES


class MonoError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("%s (%d): %s" % (STATUS.get(code, "?"), code, msg))
        self.code = code


class MonoConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "seq_len", "width", "n_q_heads", "n_kv_heads", "head_dim", "block_size",
        "n_components", "codes_per_component", "capacity", "n_probes", "n_remote", "n_local",
        "dtype")]


class MonoIndex(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("kbar", "addr", "offsets", "entries", "load", "overflow", "k_rot")]


_lib = None


def load_library(path=None):
    """Load libmono.so (the in-tree build, or the file the environment
    variable MONO_LIBRARY names); raises OSError if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("MONO_LIBRARY") or LIB_PATH
    if not os.path.exists(path):
        raise OSError("libmono.so is not built (run `python -m learned_sparse_causal_amd.build`)")
    # torch first: the library then binds to the HIP runtime torch loaded, so
    # its kernels and torch's memory and streams belong to one runtime
    _torch()
    lib = ctypes.CDLL(path)
    P, S, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    cfgp = ctypes.POINTER(MonoConfig)
    idxp = ctypes.POINTER(MonoIndex)
    lib.mono_workspace_bytes.argtypes = [cfgp, I]
    lib.mono_workspace_bytes.restype = S
    lib.mono_rope_table.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_double, P, P]
    lib.mono_build_index.argtypes = [cfgp, P, P, P, P, idxp, P, S, P]
    lib.mono_route.argtypes = [cfgp, P, P, P, P, idxp, P, P, S, P]
    lib.mono_selected_attention.argtypes = [cfgp, P, P, P, P, P, P, P, P, S, P]
    lib.mono_dense_attention.argtypes = [cfgp, P, P, P, P, P, P, P, S, P]
    lib.mono_routed_attention.argtypes = [cfgp, P, P, P, P, P, P, idxp, P, P, P, S, P, P]
    lib.mono_routed_attention_noalloc.argtypes = [cfgp, P, P, P, P, P, P, idxp, P, P, P, P]
    lib.mono_calibrate_codebooks.argtypes = [cfgp, P, P, ctypes.c_int32, P, S, P]
    lib.mono_decode_index.argtypes = [cfgp, P, P, P, P, idxp, ctypes.c_int32, ctypes.c_int32, P]
    lib.mono_decode_step.argtypes = [cfgp, P, P, P, P, P, P, idxp, ctypes.c_int32, P, P, P]
    lib.mono_mixer_forward.argtypes = [cfgp, P, P, P, P, P, P, P, P, P, S, P]
    lib.mono_mixer_layout.argtypes = [cfgp, ctypes.POINTER(ctypes.c_size_t)]
    lib.mono_status_string.argtypes = [I]
    lib.mono_status_string.restype = ctypes.c_char_p
    for f in ("mono_rope_table", "mono_build_index", "mono_route", "mono_selected_attention",
              "mono_dense_attention", "mono_routed_attention", "mono_routed_attention_noalloc",
              "mono_calibrate_codebooks",
              "mono_decode_index",
              "mono_decode_step",
              "mono_mixer_forward", "mono_mixer_layout"):
        getattr(lib, f).restype = I
    _lib = lib
    return lib


def _check(code):
    if code != 0:
        raise MonoError(code, load_library().mono_status_string(code).decode())


def make_config(cfg, dtype=None):
    """mono_config from a workload description (learned_sparse_causal_amd.configs.Config)."""
    dt = dtype or cfg.dtype
    return MonoConfig(cfg.B, cfg.T, cfg.W, cfg.Hq, cfg.Hkv, cfg.d, cfg.beta, cfg.P, cfg.K,
                      cfg.cap, cfg.n_probes, cfg.R, cfg.L, MONO_BF16 if dt == "bf16" else MONO_F32)


def workspace_bytes(cfg, which):
    c = make_config(cfg)
    return int(load_library().mono_workspace_bytes(ctypes.byref(c), which))


def rope_table(T, d, base=10000.0):
    """Host rotary tables (cos, sin) [T, d/2] float32 from mono_rope_table."""
    c = np.empty((T, d // 2), np.float32)
    s = np.empty((T, d // 2), np.float32)
    _check(load_library().mono_rope_table(T, d, base, c.ctypes.data, s.ctypes.data))
    return c, s


# ---------------------------------------------------------------- torch side
def _torch():
    import torch
    return torch


def _act_dtype(cfg):
    torch = _torch()
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def _need(t, shape, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a CUDA (HIP) tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


def _stream():
    return _torch().cuda.current_stream().cuda_stream


def device_rope(cfg, device="cuda", base=10000.0):
    torch = _torch()
    c, s = rope_table(cfg.T, cfg.d, base)
    return torch.from_numpy(c).to(device), torch.from_numpy(s).to(device)


def empty_index(cfg, device="cuda", rotated_keys=False):
    """Index arrays for cfg; with rotated_keys the optional k_rot copy
    [B, T, Hkv, d] (activation dtype) that the decode step reads."""
    torch = _torch()
    BG = (cfg.B, cfg.Hkv)
    i32 = torch.int32
    idx = dict(kbar=torch.empty(BG + (cfg.NB, cfg.d), dtype=torch.float32, device=device),
               addr=torch.empty(BG + (cfg.NB,), dtype=i32, device=device),
               offsets=torch.empty(BG + (cfg.A + 1,), dtype=i32, device=device),
               entries=torch.empty(BG + (cfg.NB,), dtype=i32, device=device),
               load=torch.empty(BG + (cfg.A,), dtype=i32, device=device),
               overflow=torch.empty(BG, dtype=i32, device=device))
    if rotated_keys:
        idx["k_rot"] = torch.empty((cfg.B, cfg.T, cfg.Hkv, cfg.d), dtype=_act_dtype(cfg),
                                   device=device)
    return idx


def _index_struct(cfg, idx):
    torch = _torch()
    BG = (cfg.B, cfg.Hkv)
    return MonoIndex(_need(idx["kbar"], BG + (cfg.NB, cfg.d), torch.float32, "kbar"),
                     _need(idx["addr"], BG + (cfg.NB,), torch.int32, "addr"),
                     _need(idx["offsets"], BG + (cfg.A + 1,), torch.int32, "offsets"),
                     _need(idx["entries"], BG + (cfg.NB,), torch.int32, "entries"),
                     _need(idx["load"], BG + (cfg.A,), torch.int32, "load"),
                     _need(idx["overflow"], BG, torch.int32, "overflow"),
                     _need(idx["k_rot"], (cfg.B, cfg.T, cfg.Hkv, cfg.d), _act_dtype(cfg), "k_rot")
                     if idx.get("k_rot") is not None else None)


def _workspace(cfg, which, ws):
    torch = _torch()
    n = workspace_bytes(cfg, which)
    if n == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    if ws.numel() < n:
        raise ValueError("workspace needs %d bytes" % n)
    return ws, ws.numel()


def build_index(cfg, k, rope_cos, rope_sin, codebooks, index=None, rotated_keys=False):
    """mono_build_index: returns the index dict (kbar, addr, offsets, entries, load,
    overflow, and k_rot when the index holds one or rotated_keys asks for it)."""
    torch = _torch()
    c = make_config(cfg)
    idx = index if index is not None else empty_index(cfg, rotated_keys=rotated_keys)
    st = _index_struct(cfg, idx)
    args = (_need(k, (cfg.B, cfg.T, cfg.Hkv, cfg.d), _act_dtype(cfg), "k"),
            _need(rope_cos, (cfg.T, cfg.d // 2), torch.float32, "rope_cos"),
            _need(rope_sin, (cfg.T, cfg.d // 2), torch.float32, "rope_sin"),
            _need(codebooks, (cfg.Hkv, cfg.P, cfg.K, cfg.d // cfg.P), torch.float32, "codebooks"))
    _check(load_library().mono_build_index(ctypes.byref(c), *args, ctypes.byref(st), None, 0,
                                           _stream()))
    return idx


def route(cfg, q, rope_cos, rope_sin, codebooks, index, sel=None):
    """mono_route: returns sel [B, Hq, T, R] int32."""
    torch = _torch()
    c = make_config(cfg)
    st = _index_struct(cfg, index)
    if sel is None:
        sel = torch.empty((cfg.B, cfg.Hq, cfg.T, cfg.R), dtype=torch.int32, device="cuda")
    args = (_need(q, (cfg.B, cfg.T, cfg.Hq, cfg.d), _act_dtype(cfg), "q"),
            _need(rope_cos, (cfg.T, cfg.d // 2), torch.float32, "rope_cos"),
            _need(rope_sin, (cfg.T, cfg.d // 2), torch.float32, "rope_sin"),
            _need(codebooks, (cfg.Hkv, cfg.P, cfg.K, cfg.d // cfg.P), torch.float32, "codebooks"))
    sp = _need(sel, (cfg.B, cfg.Hq, cfg.T, cfg.R), torch.int32, "sel")
    _check(load_library().mono_route(ctypes.byref(c), *args, ctypes.byref(st), sp, None, 0,
                                     _stream()))
    return sel


def selected_attention(cfg, q, k, v, rope_cos, rope_sin, sel, out=None, ws=None):
    """mono_selected_attention: returns out [B, T, Hq, d] in the activation dtype."""
    torch = _torch()
    c = make_config(cfg)
    dt = _act_dtype(cfg)
    if out is None:
        out = torch.empty((cfg.B, cfg.T, cfg.Hq, cfg.d), dtype=dt, device="cuda")
    ws, nws = _workspace(cfg, WS_ATTENTION, ws)
    args = (_need(q, (cfg.B, cfg.T, cfg.Hq, cfg.d), dt, "q"),
            _need(k, (cfg.B, cfg.T, cfg.Hkv, cfg.d), dt, "k"),
            _need(v, (cfg.B, cfg.T, cfg.Hkv, cfg.d), dt, "v"),
            _need(rope_cos, (cfg.T, cfg.d // 2), torch.float32, "rope_cos"),
            _need(rope_sin, (cfg.T, cfg.d // 2), torch.float32, "rope_sin"),
            _need(sel, (cfg.B, cfg.Hq, cfg.T, cfg.R), torch.int32, "sel"),
            _need(out, (cfg.B, cfg.T, cfg.Hq, cfg.d), dt, "out"))
    _check(load_library().mono_selected_attention(ctypes.byref(c), *args,
                                                  ws.data_ptr() if ws is not None else None,
                                                  nws, _stream()))
    return out


def _event_handles(events):
    """hipEvent_t handles of four torch.cuda.Event slots (None: not recorded)."""
    handles = []
    for e in events:
        if e is None:
            handles.append(None)
            continue
        if e.cuda_event == 0:       # created on first record
            e.record()
        handles.append(e.cuda_event)
    return handles


def routed_attention(cfg, q, k, v, rope_cos, rope_sin, codebooks, index=None, sel=None, out=None,
                     ws=None, stage_events=None):
    """mono_routed_attention: the whole step (index build, route, attention) in
    one call; returns (index, sel, out).  stage_events: None or four slots,
    each None or a torch.cuda.Event(enable_timing=True), recorded by the
    library before the build, after it, after the route and after the
    attention."""
    torch = _torch()
    c = make_config(cfg)
    dt = _act_dtype(cfg)
    idx = index if index is not None else empty_index(cfg)
    st = _index_struct(cfg, idx)
    if sel is None:
        sel = torch.empty((cfg.B, cfg.Hq, cfg.T, cfg.R), dtype=torch.int32, device="cuda")
    if out is None:
        out = torch.empty((cfg.B, cfg.T, cfg.Hq, cfg.d), dtype=dt, device="cuda")
    ws, nws = _workspace(cfg, WS_ATTENTION, ws)
    ev = None
    if stage_events is not None:
        ev = (ctypes.c_void_p * 4)(*_event_handles(stage_events))
    args = (_need(q, (cfg.B, cfg.T, cfg.Hq, cfg.d), dt, "q"),
            _need(k, (cfg.B, cfg.T, cfg.Hkv, cfg.d), dt, "k"),
            _need(v, (cfg.B, cfg.T, cfg.Hkv, cfg.d), dt, "v"),
            _need(rope_cos, (cfg.T, cfg.d // 2), torch.float32, "rope_cos"),
            _need(rope_sin, (cfg.T, cfg.d // 2), torch.float32, "rope_sin"),
            _need(codebooks, (cfg.Hkv, cfg.P, cfg.K, cfg.d // cfg.P), torch.float32, "codebooks"))
    _check(load_library().mono_routed_attention(
        ctypes.byref(c), *args, ctypes.byref(st),
        _need(sel, (cfg.B, cfg.Hq, cfg.T, cfg.R), torch.int32, "sel"),
        _need(out, (cfg.B, cfg.T, cfg.Hq, cfg.d), dt, "out"),
        ws.data_ptr() if ws is not None else None, nws, ev, _stream()))
    return idx, sel, out


def routed_attention_noalloc(cfg, q, k, v, rope_cos, rope_sin, codebooks, index=None, sel=None,
                             out=None, stage_events=None):
    """mono_routed_attention_noalloc: the whole step with the library's static
    scratch in place of a workspace; returns (index, sel, out).  Outputs not
    passed in are allocated here, by torch, before the call."""
    torch = _torch()
    c = make_config(cfg)
    dt = _act_dtype(cfg)
    idx = index if index is not None else empty_index(cfg)
    st = _index_struct(cfg, idx)
    if sel is None:
        sel = torch.empty((cfg.B, cfg.Hq, cfg.T, cfg.R), dtype=torch.int32, device="cuda")
    if out is None:
        out = torch.empty((cfg.B, cfg.T, cfg.Hq, cfg.d), dtype=dt, device="cuda")
    ev = None
    if stage_events is not None:
        ev = (ctypes.c_void_p * 4)(*_event_handles(stage_events))
    _check(load_library().mono_routed_attention_noalloc(
        ctypes.byref(c),
        _need(q, (cfg.B, cfg.T, cfg.Hq, cfg.d), dt, "q"),
        _need(k, (cfg.B, cfg.T, cfg.Hkv, cfg.d), dt, "k"),
        _need(v, (cfg.B, cfg.T, cfg.Hkv, cfg.d), dt, "v"),
        _need(rope_cos, (cfg.T, cfg.d // 2), torch.float32, "rope_cos"),
        _need(rope_sin, (cfg.T, cfg.d // 2), torch.float32, "rope_sin"),
        _need(codebooks, (cfg.Hkv, cfg.P, cfg.K, cfg.d // cfg.P), torch.float32, "codebooks"),
        ctypes.byref(st),
        _need(sel, (cfg.B, cfg.Hq, cfg.T, cfg.R), torch.int32, "sel"),
        _need(out, (cfg.B, cfg.T, cfg.Hq, cfg.d), dt, "out"),
        ev, _stream()))
    return idx, sel, out


def routed_attention_launcher(cfg, q, k, v, rope_cos, rope_sin, codebooks, index, sel, out, ws):
    """mono_routed_attention with the arguments checked and marshalled once:
    returns launch(stage_events=None), which only calls the library (on the
    stream current when the launcher was made).  For loops that repeat the
    same call, where per-call checks would cost host time."""
    torch = _torch()
    c = make_config(cfg)
    dt = _act_dtype(cfg)
    st = _index_struct(cfg, index)
    ws, nws = _workspace(cfg, WS_ATTENTION, ws)
    args = (ctypes.byref(c),
            _need(q, (cfg.B, cfg.T, cfg.Hq, cfg.d), dt, "q"),
            _need(k, (cfg.B, cfg.T, cfg.Hkv, cfg.d), dt, "k"),
            _need(v, (cfg.B, cfg.T, cfg.Hkv, cfg.d), dt, "v"),
            _need(rope_cos, (cfg.T, cfg.d // 2), torch.float32, "rope_cos"),
            _need(rope_sin, (cfg.T, cfg.d // 2), torch.float32, "rope_sin"),
            _need(codebooks, (cfg.Hkv, cfg.P, cfg.K, cfg.d // cfg.P), torch.float32, "codebooks"),
            ctypes.byref(st),
            _need(sel, (cfg.B, cfg.Hq, cfg.T, cfg.R), torch.int32, "sel"),
            _need(out, (cfg.B, cfg.T, cfg.Hq, cfg.d), dt, "out"),
            ws.data_ptr() if ws is not None else None, nws)
    stream = _stream()
    fn = load_library().mono_routed_attention
    keep = (c, st, ws)   # referenced by the closure so the marshalled memory stays alive

    def launch(stage_events=None):
        ev = None
        if stage_events is not None:
            ev = (ctypes.c_void_p * 4)(*_event_handles(stage_events))
        code = fn(*args, ev, stream)
        if code != 0:
            _check(code)
        return keep

    return launch


def dense_attention(cfg, q, k, v, rope_cos, rope_sin, out=None, ws=None):
    """mono_dense_attention: returns out [B, T, Hq, d] in the activation dtype."""
    torch = _torch()
    c = make_config(cfg)
    dt = _act_dtype(cfg)
    if out is None:
        out = torch.empty((cfg.B, cfg.T, cfg.Hq, cfg.d), dtype=dt, device="cuda")
    ws, nws = _workspace(cfg, WS_DENSE, ws)
    args = (_need(q, (cfg.B, cfg.T, cfg.Hq, cfg.d), dt, "q"),
            _need(k, (cfg.B, cfg.T, cfg.Hkv, cfg.d), dt, "k"),
            _need(v, (cfg.B, cfg.T, cfg.Hkv, cfg.d), dt, "v"),
            _need(rope_cos, (cfg.T, cfg.d // 2), torch.float32, "rope_cos"),
            _need(rope_sin, (cfg.T, cfg.d // 2), torch.float32, "rope_sin"),
            _need(out, (cfg.B, cfg.T, cfg.Hq, cfg.d), dt, "out"))
    _check(load_library().mono_dense_attention(ctypes.byref(c), *args,
                                               ws.data_ptr() if ws is not None else None,
                                               nws, _stream()))
    return out


def calibrate_codebooks(cfg, kbar, codebooks, n_iter, ws=None):
    """mono_calibrate_codebooks: calibrates codebooks [Hkv, P, K, d/P] in place on
    the training summaries kbar [B, Hkv, NB, d]; returns codebooks."""
    torch = _torch()
    c = make_config(cfg)
    ws, nws = _workspace(cfg, WS_CALIBRATE, ws)
    args = (_need(kbar, (cfg.B, cfg.Hkv, cfg.NB, cfg.d), torch.float32, "kbar"),
            _need(codebooks, (cfg.Hkv, cfg.P, cfg.K, cfg.d // cfg.P), torch.float32, "codebooks"))
    _check(load_library().mono_calibrate_codebooks(ctypes.byref(c), *args, int(n_iter),
                                                   ws.data_ptr() if ws is not None else None,
                                                   nws, _stream()))
    return codebooks


def decode_index(cfg, k_cache, rope_cos, rope_sin, codebooks, index, n_indexed, n_tokens):
    """mono_decode_index: index blocks n_indexed .. n_tokens // beta - 1 of the
    cache and rebuild the lists over the indexed prefix; returns the index."""
    torch = _torch()
    c = make_config(cfg)
    st = _index_struct(cfg, index)
    args = (_need(k_cache, (cfg.B, cfg.T, cfg.Hkv, cfg.d), _act_dtype(cfg), "k_cache"),
            _need(rope_cos, (cfg.T, cfg.d // 2), torch.float32, "rope_cos"),
            _need(rope_sin, (cfg.T, cfg.d // 2), torch.float32, "rope_sin"),
            _need(codebooks, (cfg.Hkv, cfg.P, cfg.K, cfg.d // cfg.P), torch.float32, "codebooks"))
    _check(load_library().mono_decode_index(ctypes.byref(c), *args, ctypes.byref(st),
                                            int(n_indexed), int(n_tokens), _stream()))
    return index


def decode_step(cfg, q, k_cache, v_cache, rope_cos, rope_sin, codebooks, index, pos, sel=None,
                out=None):
    """mono_decode_step: returns (sel [B, Hq, R] int32, out [B, Hq, d]) for the
    token at position pos."""
    torch = _torch()
    c = make_config(cfg)
    dt = _act_dtype(cfg)
    st = _index_struct(cfg, index)
    if sel is None:
        sel = torch.empty((cfg.B, cfg.Hq, cfg.R), dtype=torch.int32, device="cuda")
    if out is None:
        out = torch.empty((cfg.B, cfg.Hq, cfg.d), dtype=dt, device="cuda")
    args = (_need(q, (cfg.B, cfg.Hq, cfg.d), dt, "q"),
            _need(k_cache, (cfg.B, cfg.T, cfg.Hkv, cfg.d), dt, "k_cache"),
            _need(v_cache, (cfg.B, cfg.T, cfg.Hkv, cfg.d), dt, "v_cache"),
            _need(rope_cos, (cfg.T, cfg.d // 2), torch.float32, "rope_cos"),
            _need(rope_sin, (cfg.T, cfg.d // 2), torch.float32, "rope_sin"),
            _need(codebooks, (cfg.Hkv, cfg.P, cfg.K, cfg.d // cfg.P), torch.float32, "codebooks"))
    _check(load_library().mono_decode_step(ctypes.byref(c), *args, ctypes.byref(st), int(pos),
                                           _need(sel, (cfg.B, cfg.Hq, cfg.R), torch.int32, "sel"),
                                           _need(out, (cfg.B, cfg.Hq, cfg.d), dt, "out"),
                                           _stream()))
    return sel, out


def mixer_layout(cfg):
    c = make_config(cfg)
    off = (ctypes.c_size_t * 12)()
    _check(load_library().mono_mixer_layout(ctypes.byref(c), off))
    return list(off)


def mixer_forward(cfg, x, w_qkv, w_o, codebooks, rope_cos, rope_sin, delta=None, stats=None,
                  ws=None):
    """mono_mixer_forward: returns (delta [B, T, W], stats int32[2], workspace)."""
    torch = _torch()
    c = make_config(cfg)
    dt = _act_dtype(cfg)
    if delta is None:
        delta = torch.empty((cfg.B, cfg.T, cfg.W), dtype=dt, device="cuda")
    if stats is None:
        stats = torch.zeros(2, dtype=torch.int32, device="cuda")
    ws, nws = _workspace(cfg, WS_MIXER, ws)
    nqkv = (cfg.Hq + 2 * cfg.Hkv) * cfg.d
    args = (_need(x, (cfg.B, cfg.T, cfg.W), dt, "x"),
            _need(w_qkv, (cfg.W, nqkv), dt, "w_qkv"),
            _need(w_o, (cfg.Hq * cfg.d, cfg.W), dt, "w_o"),
            _need(codebooks, (cfg.Hkv, cfg.P, cfg.K, cfg.d // cfg.P), torch.float32, "codebooks"),
            _need(rope_cos, (cfg.T, cfg.d // 2), torch.float32, "rope_cos"),
            _need(rope_sin, (cfg.T, cfg.d // 2), torch.float32, "rope_sin"),
            _need(delta, (cfg.B, cfg.T, cfg.W), dt, "delta"),
            _need(stats, (2,), torch.int32, "stats"))
    _check(load_library().mono_mixer_forward(ctypes.byref(c), *args, ws.data_ptr(), nws,
                                              _stream()))
    return delta, stats, ws


def mixer_views(cfg, ws):
    """Views into a mixer workspace: q, k, v, the index, sel and the attention output."""
    torch = _torch()
    off = mixer_layout(cfg)
    dt = _act_dtype(cfg)
    es = 2 if cfg.dtype == "bf16" else 4

    def view(i, shape, dtype, esize):
        n = int(np.prod(shape))
        return ws[off[i]: off[i] + n * esize].view(dtype).view(shape)

    BG = (cfg.B, cfg.Hkv)
    return dict(
        q=view(0, (cfg.B, cfg.T, cfg.Hq, cfg.d), dt, es),
        k=view(1, (cfg.B, cfg.T, cfg.Hkv, cfg.d), dt, es),
        v=view(2, (cfg.B, cfg.T, cfg.Hkv, cfg.d), dt, es),
        index=dict(kbar=view(3, BG + (cfg.NB, cfg.d), torch.float32, 4),
                   addr=view(4, BG + (cfg.NB,), torch.int32, 4),
                   offsets=view(5, BG + (cfg.A + 1,), torch.int32, 4),
                   entries=view(6, BG + (cfg.NB,), torch.int32, 4),
                   load=view(7, BG + (cfg.A,), torch.int32, 4),
                   overflow=view(8, BG, torch.int32, 4)),
        sel=view(9, (cfg.B, cfg.Hq, cfg.T, cfg.R), torch.int32, 4),
        attn=view(10, (cfg.B, cfg.T, cfg.Hq, cfg.d), dt, es))
