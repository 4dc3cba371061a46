"""ctypes binding of oracle.c (test infrastructure; see the package docstring).

Arrays cross the boundary as numpy arrays: activations as float32 (bf16
inputs are widened exactly before they get here), codebooks and rotary tables
as float32, index arrays as int32.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# AddressSanitizer + UndefinedBehaviorSanitizer build of the same source, for
# the sanitizer run of the CPU tests: loaded instead of _LIB when the
# environment sets ORACLE_SANITIZED=1 (the process must then preload gcc's
# libasan, since the Python interpreter itself is not instrumented).
_LIB_SAN = os.path.join(_HERE, "liboracle_san.so")
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                  "-fno-omit-frame-pointer", "-g", "-O1"]
_lib = None


def _lib_path():
    return _LIB_SAN if os.environ.get("ORACLE_SANITIZED") == "1" else _LIB


def build_oracle(force=True, sanitize=None):
    """Compile oracle.c with gcc (fp contraction off, OpenMP); with
    sanitize=True (default: as ORACLE_SANITIZED asks) the instrumented
    library."""
    if sanitize is None:
        sanitize = os.environ.get("ORACLE_SANITIZED") == "1"
    lib = _LIB_SAN if sanitize else _LIB
    if not force and os.path.exists(lib) and os.path.getmtime(lib) >= os.path.getmtime(_SRC):
        return lib
    tmp = lib + ".tmp%d" % os.getpid()
    opt = SANITIZE_FLAGS if sanitize else ["-O2"]
    cmd = ["gcc", *opt, "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, lib)
    return lib


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in
                ("B", "T", "Hq", "Hkv", "d", "beta", "P", "K", "cap", "n_probes", "R", "L")]

    @classmethod
    def of(cls, **kw):
        return cls(*[int(kw[n]) for n, _ in cls._fields_])

    @property
    def NB(self):
        return self.T // self.beta


def load():
    global _lib
    if _lib is None:
        build_oracle(force=False)
        lib = ctypes.CDLL(_lib_path())
        P = ctypes.c_void_p
        I = ctypes.c_int
        L = ctypes.c_long
        lib.orc_rope_table.argtypes = [I, I, ctypes.c_double, P, P]
        lib.orc_block_addresses.argtypes = [P, P, P, P, P, P, P, P, I]
        lib.orc_posting_lists.argtypes = [I, I, I, P, P, P, P, P]
        lib.orc_build_index.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, I]
        lib.orc_route.argtypes = [P, P, P, P, P, P, P, P, P, L, P, P, I]
        lib.orc_attention.argtypes = [P, P, P, P, P, P, P, P, L, P, I]
        lib.orc_calibrate.argtypes = [I, I, I, I, I, I, P, P, I]
        lib.orc_max_threads.restype = I
        for f in ("orc_rope_table", "orc_block_addresses", "orc_posting_lists",
                  "orc_build_index", "orc_route", "orc_attention", "orc_calibrate"):
            getattr(lib, f).restype = None
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def max_threads():
    return load().orc_max_threads()


def num_addresses(sh):
    return int(sh.K) ** int(sh.P)


def rope_table(T, d, base=10000.0):
    """fp32 cos/sin tables [T, d/2] from fp64 angles."""
    c = np.empty((T, d // 2), np.float32)
    s = np.empty((T, d // 2), np.float32)
    load().orc_rope_table(int(T), int(d), float(base), _p(c), _p(s))
    return c, s


def block_addresses(sh, k, cos, sin, codebooks, nthreads=None):
    """Block summaries kbar [B,Hkv,NB,d], addresses [B,Hkv,NB] and the argmax
    gaps [B,Hkv,NB,P]."""
    k, cos, sin, codebooks = _f32(k), _f32(cos), _f32(sin), _f32(codebooks)
    NB = sh.T // sh.beta
    kbar = np.empty((sh.B, sh.Hkv, NB, sh.d), np.float32)
    addr = np.empty((sh.B, sh.Hkv, NB), np.int32)
    gap = np.empty((sh.B, sh.Hkv, NB, sh.P), np.float64)
    load().orc_block_addresses(ctypes.byref(sh), _p(k), _p(cos), _p(sin), _p(codebooks),
                               _p(kbar), _p(addr), _p(gap), int(nthreads or max_threads()))
    return kbar, addr, gap


def posting_lists(addr, A, cap):
    """Lists of one (batch, kv-head) from its address vector."""
    addr = _i32(addr)
    NB = addr.shape[0]
    offsets = np.empty(A + 1, np.int32)
    entries = np.empty(NB, np.int32)
    loadv = np.empty(A, np.int32)
    overflow = np.zeros(1, np.int32)
    load().orc_posting_lists(int(NB), int(A), int(cap), _p(addr), _p(offsets), _p(entries),
                             _p(loadv), _p(overflow))
    return offsets, entries, loadv, int(overflow[0])


def build_index(sh, k, cos, sin, codebooks, nthreads=None):
    """The whole index, as a dict of numpy arrays."""
    k, cos, sin, codebooks = _f32(k), _f32(cos), _f32(sin), _f32(codebooks)
    NB = sh.T // sh.beta
    A = num_addresses(sh)
    out = dict(
        kbar=np.empty((sh.B, sh.Hkv, NB, sh.d), np.float32),
        addr=np.empty((sh.B, sh.Hkv, NB), np.int32),
        offsets=np.empty((sh.B, sh.Hkv, A + 1), np.int32),
        entries=np.empty((sh.B, sh.Hkv, NB), np.int32),
        load=np.empty((sh.B, sh.Hkv, A), np.int32),
        overflow=np.empty((sh.B, sh.Hkv), np.int32),
        gap=np.empty((sh.B, sh.Hkv, NB, sh.P), np.float64),
    )
    load().orc_build_index(ctypes.byref(sh), _p(k), _p(cos), _p(sin), _p(codebooks),
                           _p(out["kbar"]), _p(out["addr"]), _p(out["offsets"]),
                           _p(out["entries"]), _p(out["load"]), _p(out["overflow"]),
                           _p(out["gap"]), int(nthreads or max_threads()))
    return out


def route(sh, q, cos, sin, codebooks, index, route_ids=None, nthreads=None):
    """Selected remote blocks for the listed routes (all routes if None).
    Returns (sel [n, R] int32, gaps [n, 2] float64)."""
    q, cos, sin, codebooks = _f32(q), _f32(cos), _f32(sin), _f32(codebooks)
    ids = None if route_ids is None else np.ascontiguousarray(route_ids, np.int64)
    n = sh.B * sh.Hq * sh.T if ids is None else ids.shape[0]
    sel = np.empty((n, sh.R), np.int32)
    gaps = np.empty((n, 2), np.float64)
    kbar = _f32(index["kbar"])
    offsets = _i32(index["offsets"])
    entries = _i32(index["entries"])
    load().orc_route(ctypes.byref(sh), _p(q), _p(cos), _p(sin), _p(codebooks), _p(kbar),
                     _p(offsets), _p(entries), _p(ids), int(n), _p(sel), _p(gaps),
                     int(nthreads or max_threads()))
    return sel, gaps


def calibrate(kbar, codebooks, n_iter):
    """Spherical k-means calibration of codebooks [Hkv, P, K, d/P] on block
    summaries kbar [B, Hkv, NB, d]; returns the calibrated codebooks."""
    kbar = _f32(kbar)
    B, Hkv, NB, d = kbar.shape
    cb = np.array(codebooks, np.float32, copy=True, order="C")
    _, P, K, _ = cb.shape
    load().orc_calibrate(B, Hkv, NB, d, P, K, _p(kbar), _p(cb), int(n_iter))
    return cb


def attention(sh, q, k, v, cos, sin, sel, route_ids=None, nthreads=None):
    """fp64 selected-set causal attention for the listed routes; sel holds
    the selection of each listed route ([n, R]).  Returns [n, d] float64."""
    q, k, v, cos, sin = _f32(q), _f32(k), _f32(v), _f32(cos), _f32(sin)
    ids = None if route_ids is None else np.ascontiguousarray(route_ids, np.int64)
    n = sh.B * sh.Hq * sh.T if ids is None else ids.shape[0]
    sel = _i32(sel).reshape(n, sh.R)
    out = np.empty((n, sh.d), np.float64)
    load().orc_attention(ctypes.byref(sh), _p(q), _p(k), _p(v), _p(cos), _p(sin), _p(sel),
                         _p(ids), int(n), _p(out), int(nthreads or max_threads()))
    return out


def _round_bf16(a):
    """Round values to the nearest bfloat16 (ties to even) straight from
    fp64 (one rounding), returned as float32 holding the bf16 value."""
    f = np.ascontiguousarray(a, dtype=np.float64)
    bits = f.view(np.uint64)
    drop = np.uint64(45)                      # 52 - 7 mantissa bits dropped
    half = np.uint64((1 << 44) - 1)
    odd = (bits >> drop) & np.uint64(1)
    rounded = ((bits + half + odd) >> drop) << drop
    return rounded.view(np.float64).astype(np.float32)


def mixer(sh, x, w_qkv, w_o, codebooks, cos, sin, dtype, nthreads=None):
    """The whole mixer: projections, index, route, attention, output
    projection ([TR] "Mixer", Figure 1: normalized stream in, attention delta
    of the same shape out).

    Projections are exact (fp64) products, rounded to the activation dtype
    because the routing decisions are taken on the stored q and k.  The
    attention output is kept in fp64 and projected in fp64.
    Returns dict(delta [B,T,W] fp64, q, k, v, index, sel, gaps)."""
    B, T = sh.B, sh.T
    W = x.shape[-1]
    Hq, Hkv, d = sh.Hq, sh.Hkv, sh.d
    x64 = np.asarray(x, np.float64).reshape(B * T, W)
    qkv = x64 @ np.asarray(w_qkv, np.float64)
    if dtype == "bf16":
        qkv = _round_bf16(qkv)
    else:
        qkv = qkv.astype(np.float32)
    q = qkv[:, : Hq * d].reshape(B, T, Hq, d)
    k = qkv[:, Hq * d: (Hq + Hkv) * d].reshape(B, T, Hkv, d)
    v = qkv[:, (Hq + Hkv) * d:].reshape(B, T, Hkv, d)
    idx = build_index(sh, k, cos, sin, codebooks, nthreads)
    sel, gaps = route(sh, q, cos, sin, codebooks, idx, None, nthreads)
    o = attention(sh, q, k, v, cos, sin, sel, None, nthreads)      # [(b,h,t), d]
    o = o.reshape(B, Hq, T, d).transpose(0, 2, 1, 3).reshape(B * T, Hq * d)
    delta = (o @ np.asarray(w_o, np.float64)).reshape(B, T, W)
    return dict(delta=delta, q=q, k=k, v=v, index=idx, sel=sel, gaps=gaps)
