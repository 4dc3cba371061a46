"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  Host arrays are float32 numpy arrays; for bf16
workloads they hold bf16-representable values (rounded to nearest, ties to
even), so the same bytes reach the GPU and the oracle.

Recipe (every workload): numpy PCG64 streams from SeedSequence(seed).spawn(9),
one stream each for x, W_q, W_k, W_v, W_o, codebooks, q, k, v.  Activations
and direct q/k/v draws are N(0, 1); weights are N(0, 1/W); each codebook row
is an N(0, I) draw scaled to unit norm, independently per kv-head.
"""
import numpy as np

from .configs import Config

_STREAMS = ("x", "wq", "wk", "wv", "wo", "codebooks", "q", "k", "v")


def _rngs(seed):
    kids = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return {n: np.random.Generator(np.random.PCG64(s)) for n, s in zip(_STREAMS, kids)}


def round_to_bf16(a):
    """Nearest bfloat16 (ties to even) of float32 values, as float32."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    rounded = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16) << 16
    return rounded.astype(np.uint32).view(np.float32)


def _cast(a, dtype):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return round_to_bf16(a) if dtype == "bf16" else a


def codebooks(cfg: Config, rng=None):
    """Unit-norm random codes [Hkv, P, K, d/P] (fp32)."""
    rng = rng or _rngs(cfg.seed)["codebooks"]
    c = rng.standard_normal((cfg.Hkv, cfg.P, cfg.K, cfg.d // cfg.P), dtype=np.float32)
    c /= np.linalg.norm(c, axis=-1, keepdims=True)
    return np.ascontiguousarray(c, dtype=np.float32)


def mixer_inputs(cfg: Config):
    """x [B,T,W], w_qkv [W, (Hq+2Hkv)d], w_o [Hq d, W], codebooks."""
    r = _rngs(cfg.seed)
    W, d = cfg.W, cfg.d
    std = 1.0 / np.sqrt(W)
    x = r["x"].standard_normal((cfg.B, cfg.T, W), dtype=np.float32)
    wq = r["wq"].standard_normal((W, cfg.Hq * d), dtype=np.float32) * std
    wk = r["wk"].standard_normal((W, cfg.Hkv * d), dtype=np.float32) * std
    wv = r["wv"].standard_normal((W, cfg.Hkv * d), dtype=np.float32) * std
    wo = r["wo"].standard_normal((cfg.Hq * d, W), dtype=np.float32) * std
    w_qkv = np.concatenate([wq, wk, wv], axis=1)
    return dict(x=_cast(x, cfg.dtype), w_qkv=_cast(w_qkv, cfg.dtype), w_o=_cast(wo, cfg.dtype),
                codebooks=codebooks(cfg, r["codebooks"]))


def qkv(cfg: Config):
    """Direct N(0,1) draws standing in for projected q [B,T,Hq,d], k and v
    [B,T,Hkv,d] (the projections of N(0,1) activations with N(0,1/W) weights
    have unit variance), plus the codebooks."""
    r = _rngs(cfg.seed)
    q = r["q"].standard_normal((cfg.B, cfg.T, cfg.Hq, cfg.d), dtype=np.float32)
    k = r["k"].standard_normal((cfg.B, cfg.T, cfg.Hkv, cfg.d), dtype=np.float32)
    v = r["v"].standard_normal((cfg.B, cfg.T, cfg.Hkv, cfg.d), dtype=np.float32)
    return dict(q=_cast(q, cfg.dtype), k=_cast(k, cfg.dtype), v=_cast(v, cfg.dtype),
                codebooks=codebooks(cfg, r["codebooks"]))


def qkv_device(cfg: Config, device="cuda"):
    """Large-workload variant of `qkv`: the draws are made by torch's seeded
    generator on `device` (same distribution, different stream), returned as
    torch tensors of the workload dtype, plus numpy codebooks."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(cfg.seed))
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    out = {}
    for name, heads in (("q", cfg.Hq), ("k", cfg.Hkv), ("v", cfg.Hkv)):
        out[name] = torch.randn((cfg.B, cfg.T, heads, cfg.d), generator=gen, device=device,
                                dtype=torch.float32).to(dt)
    out["codebooks"] = codebooks(cfg)
    return out


def random_selection(cfg: Config, seed, drop_prob=0.1):
    """A valid selection [B, Hq, T, R] for attention-only tests: for each
    query, min(R, E) distinct eligible remote blocks (E = qb - L + 1 blocks
    0..qb-L), ascending, -1 padded; with probability drop_prob a non-empty
    selection loses its last slot (exercising the padding path)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    B, Hq, T, R, L, beta = cfg.B, cfg.Hq, cfg.T, cfg.R, cfg.L, cfg.beta
    sel = np.full((B, Hq, T, R), -1, np.int32)
    for qb in range(cfg.NB):
        E = max(0, qb - L + 1)
        if E == 0:
            continue
        take = min(R, E)
        if E > 8 * R:
            # draws with replacement; a repeated block becomes an empty slot
            pick = np.sort(rng.integers(0, E, (B, Hq, beta, R)), axis=-1)
            dup = np.zeros(pick.shape, bool)
            dup[..., 1:] = pick[..., 1:] == pick[..., :-1]
            pick = np.sort(np.where(dup, np.iinfo(np.int32).max, pick), axis=-1)
            pick = np.where(pick == np.iinfo(np.int32).max, -1, pick).astype(np.int32)
        else:
            keys = rng.random((B, Hq, beta, E))
            pick = np.sort(np.argsort(keys, axis=-1)[..., :take], axis=-1).astype(np.int32)
        sel[:, :, qb * beta:(qb + 1) * beta, :take] = pick
    drop = rng.random((B, Hq, T)) < drop_prob
    nvalid = (sel >= 0).sum(-1)
    bb, hh, tt = np.nonzero(drop & (nvalid > 0))
    sel[bb, hh, tt, nvalid[bb, hh, tt] - 1] = -1
    return sel


def stress_keys(cfg: Config, kind, seed=7):
    """Adversarial keys and codebooks that drive posting-list overflow.

    "one_address": every key is the unit vector on the slowest-rotating
    dimension pair (d/2 - 1, d - 1) of the rotary embedding plus small noise,
    and code 0 of every component points along that pair's dimension in its
    sub-vector, so every block lands on address 0.
    "two_clusters": keys are +/- that vector by block parity (plus noise);
    codes 0 and 1 point along +/- the direction, giving two hot addresses.
    Returns (k [B,T,Hkv,d], codebooks [Hkv,P,K,d/P])."""
    rng = np.random.Generator(np.random.PCG64(seed))
    B, T, Hkv, d, P, K = cfg.B, cfg.T, cfg.Hkv, cfg.d, cfg.P, cfg.K
    ds = d // P
    k = 0.01 * rng.standard_normal((B, T, Hkv, d), dtype=np.float32)
    sign = np.ones(T, np.float32)
    if kind == "two_clusters":
        sign = np.where((np.arange(T) // cfg.beta) % 2 == 0, 1.0, -1.0).astype(np.float32)
    elif kind != "one_address":
        raise ValueError(kind)
    k[:, :, :, d // 2 - 1] += sign[None, :, None]
    k[:, :, :, d - 1] += 0.5 * sign[None, :, None]
    cb = codebooks(cfg, rng)
    for p in range(P):
        lo, hi = p * ds, (p + 1) * ds
        e = np.zeros(ds, np.float32)
        for dim in (d // 2 - 1, d - 1):
            if lo <= dim < hi:
                e[dim - lo] = 1.0
        if not e.any():
            continue
        cb[:, p, 0, :] = e
        if kind == "two_clusters" and K > 1:
            cb[:, p, 1, :] = -e
    return _cast(k, cfg.dtype), np.ascontiguousarray(cb, np.float32)


def concentrated_keys(cfg: Config, seed, model_seed=40, n_topics=8, shared=1.0, topic=0.5,
                      noise=0.3):
    """Keys whose block summaries crowd onto few addresses under random
    codebooks, standing in for the concentrated key distributions of real
    models (the capacity run of the report page).  Per kv-head, a shared
    direction and n_topics topic directions live on the slowest-rotating
    rotary pairs (so they survive the block mean); every block of a sequence
    takes one topic at random; each token adds N(0, noise^2) in every dim.
    The shared and topic directions and the codebooks depend on model_seed
    only, so sequences drawn with different `seed` come from one
    distribution (a training split and a held-out split).
    Returns (k [B,T,Hkv,d] in the workload dtype, codebooks [Hkv,P,K,d/P])."""
    mrng = np.random.Generator(np.random.PCG64(model_seed))
    srng = np.random.Generator(np.random.PCG64(seed))
    B, T, Hkv, d = cfg.B, cfg.T, cfg.Hkv, cfg.d
    h = d // 2
    slow = np.concatenate([np.arange(h - 4, h), np.arange(d - 4, d)])   # 4 slowest pairs
    mu = np.zeros((Hkv, d), np.float32)
    mu[:, h - 1] = shared
    mu[:, d - 1] = 0.5 * shared
    nu = np.zeros((Hkv, n_topics, d), np.float32)
    v = mrng.standard_normal((Hkv, n_topics, len(slow))).astype(np.float32)
    nu[:, :, slow] = topic * v / np.linalg.norm(v, axis=-1, keepdims=True)
    cb = codebooks(cfg, mrng)
    pick = srng.integers(0, n_topics, (B, cfg.NB, Hkv))
    k = noise * srng.standard_normal((B, T, Hkv, d), dtype=np.float32)
    for g in range(Hkv):
        blockwise = mu[g][None, None, :] + nu[g][pick[:, :, g]]          # [B, NB, d]
        k[:, :, g, :] += np.repeat(blockwise, cfg.beta, axis=1)
    return _cast(k, cfg.dtype), cb


def tied_inputs(cfg: Config, zero_key_every=5, zero_query_every=7):
    """The `qkv` draws rearranged so that routing meets exact score ties:
    every `zero_key_every`-th block of keys (blocks 1, 1 + every, ...) is
    zeroed in every kv-head, every `zero_query_every`-th query token is
    zeroed in every head, and in every component code 1 repeats code 0 and
    code K-1 repeats code 2 (K >= 4).  Layout only: rows are zeroed or
    copied, nothing is computed.  Returns dict(q, k, v, codebooks)."""
    inp = qkv(cfg)
    q, k, cb = inp["q"].copy(), inp["k"].copy(), inp["codebooks"].copy()
    for n in range(1, cfg.NB, zero_key_every):
        k[:, n * cfg.beta:(n + 1) * cfg.beta] = 0.0
    q[:, ::zero_query_every] = 0.0
    if cfg.K >= 4:
        cb[:, :, 1] = cb[:, :, 0]
        cb[:, :, cfg.K - 1] = cb[:, :, 2]
    return dict(q=q, k=k, v=inp["v"], codebooks=np.ascontiguousarray(cb))
