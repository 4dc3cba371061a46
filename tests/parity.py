"""Helpers of the GPU parity tests (imported by tests/test_gpu_*.py).

The oracle never sees a value produced by the GPU path: both sides start
from the same seeded inputs and every comparison is made here.
"""
import sys

import numpy as np

from learned_sparse_causal_amd import configs, synth

NEAR_TIE = 1e-5          # relative score gap below which a routing decision may differ
MAX_EXCUSED = 1e-4       # excused routes must stay below 0.01 % of the routes
F32_ATOL = 1e-4          # fp32 attention: max abs error
BF16_RTOL = 2e-2         # bf16 attention: max |gpu - ref| / max |ref| per (batch, head)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch():
    import torch as _t
    return _t


def dev(a, dtype):
    """numpy float32 (bf16-representable for bf16) -> CUDA tensor of the workload dtype."""
    t = torch()
    x = t.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda")
    return x.to(t.bfloat16) if dtype == "bf16" else x


def host(x):
    """CUDA tensor -> numpy (float32 for floating point, int32 for integers)."""
    t = torch()
    if x.dtype in (t.bfloat16, t.float16):
        x = x.float()
    return x.cpu().numpy()


def small_inputs(cfg):
    inp = synth.qkv(cfg)
    return inp, {k: dev(inp[k], cfg.dtype) for k in ("q", "k", "v")}


def index_to_host(idx):
    return {k: host(v) for k, v in idx.items()}


def compare_index(cfg, gpu, orc, excuse=True):
    """Bit-exact index parity.  An address may differ only where the oracle's
    argmax gap is below NEAR_TIE; the (batch, kv-head) lists holding such a
    block are then checked for validity instead of equality.
    Returns the set of (b, g) with an excused address."""
    assert np.array_equal(gpu["kbar"].view(np.uint32), orc["kbar"].view(np.uint32)), \
        "block summaries differ: max abs %g" % np.abs(gpu["kbar"] - orc["kbar"]).max()
    diff = gpu["addr"] != orc["addr"]
    tie = (orc["gap"] < NEAR_TIE).any(-1)
    assert not (diff & ~tie).any(), "unexcused address mismatch at %s" % (np.argwhere(diff & ~tie)[:5],)
    bad_bg = set(map(tuple, np.argwhere(diff.any(-1))))
    if not excuse:
        assert not bad_bg
    for b in range(cfg.B):
        for g in range(cfg.Hkv):
            if (b, g) in bad_bg:
                check_lists_valid(cfg, gpu, b, g)
                continue
            for name in ("offsets", "entries", "load", "overflow"):
                assert np.array_equal(gpu[name][b, g], orc[name][b, g]), (name, b, g)
    return bad_bg


def check_lists_valid(cfg, idx, b, g):
    """Lists consistent with the GPU's own addresses."""
    addr, off, ent = idx["addr"][b, g], idx["offsets"][b, g], idx["entries"][b, g]
    ld = np.bincount(addr, minlength=cfg.A)
    assert np.array_equal(idx["load"][b, g], ld)
    assert idx["overflow"][b, g] == np.maximum(ld - cfg.cap, 0).sum()
    for a in range(cfg.A):
        want = np.nonzero(addr == a)[0][:cfg.cap]
        assert np.array_equal(ent[off[a]:off[a + 1]], want)


def check_sel_invariants(cfg, sel, index=None):
    """Causality, ascending unique ids, -1 padding, slot counts."""
    B, Hq, T, R = sel.shape
    t = np.arange(T)
    qb = t // cfg.beta
    E = np.maximum(0, qb - cfg.L + 1)
    valid = sel >= 0
    nvalid = valid.sum(-1)
    # padding only at the end
    assert (np.sort(~valid, axis=-1) == ~valid).all()
    # causality
    assert (np.where(valid, sel, -10**9) <= (qb - cfg.L)[None, None, :, None]).all()
    # ascending, unique
    d = np.diff(np.where(valid, sel, 10**9), axis=-1)
    assert (np.where(valid[..., 1:], d, 1) > 0).all()
    # bypass queries take every eligible block
    byp = E <= cfg.R
    if byp.any():
        want = np.where(np.arange(R)[None, :] < E[byp][:, None], np.arange(R)[None, :], -1)
        assert np.array_equal(sel[:, :, byp], np.broadcast_to(want, sel[:, :, byp].shape))
    # searched queries fill R slots when no eligible block overflowed
    if index is not None:
        nonbyp = ~byp
        for b in range(B):
            for h in range(Hq):
                g = h // cfg.G
                if index["overflow"][b, g] == 0:
                    assert (nvalid[b, h, nonbyp] == R).all()


def compare_sel(cfg, gpu_sel, orc_sel, gaps, bad_bg=(), route_ids=None):
    """sel parity: equal except near-ties (oracle gap < NEAR_TIE) and routes of a
    (batch, kv-head) whose index had an excused address.  Returns the excused count."""
    g_sel = gpu_sel.reshape(-1, cfg.R)
    o_sel = orc_sel.reshape(-1, cfg.R)
    if route_ids is not None:
        g_sel = g_sel[route_ids]
    mism = np.nonzero((g_sel != o_sel).any(-1))[0]
    excused = 0
    for i in mism:
        rid = int(route_ids[i]) if route_ids is not None else int(i)
        t = rid % cfg.T
        h = (rid // cfg.T) % cfg.Hq
        b = rid // (cfg.T * cfg.Hq)
        ok = gaps[i].min() < NEAR_TIE or (b, h // cfg.G) in bad_bg
        assert ok, "route %d (b=%d h=%d t=%d): gpu %s oracle %s gaps %s" % (
            rid, b, h, t, g_sel[i], o_sel[i], gaps[i])
        excused += 1
    n = len(o_sel)
    assert excused <= max(MAX_EXCUSED * n, 0), "%d excused of %d routes" % (excused, n)
    return excused


def attention_error(cfg, gpu_out, ref, route_ids):
    """gpu_out [B,T,Hq,d]; ref [n, d] fp64 for route ids (b*Hq + h)*T + t.
    fp32: max abs error.  bf16: max over (b, h) of max|err| / max|ref|."""
    t = route_ids % cfg.T
    h = (route_ids // cfg.T) % cfg.Hq
    b = route_ids // (cfg.T * cfg.Hq)
    got = gpu_out[b, t, h].astype(np.float64)
    err = np.abs(got - ref)
    if cfg.dtype == "f32":
        return err.max()
    worst = 0.0
    for bh in np.unique(b * cfg.Hq + h):
        m = (b * cfg.Hq + h) == bh
        worst = max(worst, err[m].max() / max(np.abs(ref[m]).max(), 1e-30))
    return worst


def check_attention(cfg, gpu_out, ref, route_ids):
    e = attention_error(cfg, gpu_out, ref, route_ids)
    tol = F32_ATOL if cfg.dtype == "f32" else BF16_RTOL
    assert e <= tol, "attention error %g > %g" % (e, tol)
    return e


def sample_routes(cfg, n, seed=0, must=()):
    """Route ids: every query of the (b, h) pairs in `must`, plus n random ones."""
    rng = np.random.default_rng(seed)
    ids = [rng.choice(cfg.routes, size=min(n, cfg.routes), replace=False)]
    for b, h in must:
        ids.append((b * cfg.Hq + h) * cfg.T + np.arange(cfg.T))
    return np.unique(np.concatenate(ids)).astype(np.int64)


ALL_CFGS = [configs.TINY, configs.SMALL, configs.ALL_ELIGIBLE,
            *[configs.sweep(t) for t in configs.SWEEP_T], configs.LARGE]
