"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a worked
example computed by hand, a closed form, a library routine on a special case
that reduces to it, brute-force enumeration, or an invariant the pages state.
No test here needs a GPU.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

from learned_sparse_causal_amd import configs, synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
NEAR_TIE = 1e-5


def shape(orc, **kw):
    return orc.Shape.of(**kw)


def identity_table(T, d):
    return np.ones((T, d // 2), np.float32), np.zeros((T, d // 2), np.float32)


# ---------------------------------------------------------------- rotary ----
def test_rope_worked_example_rotate_half(orc):
    """d = 4, position 1: frequencies 1 and 10000^(-1/2) = 0.01.  Pairs are
    (0, 2) and (1, 3); each pair turns by +angle."""
    cos, sin = orc.rope_table(2, 4)
    assert cos[0].tolist() == [1.0, 1.0] and sin[0].tolist() == [0.0, 0.0]
    x = np.array([[1.0, 2.0, 3.0, 4.0], [1.0, 2.0, 3.0, 4.0]], np.float32)
    k = x.reshape(1, 2, 1, 4)
    sh = shape(orc, B=1, T=2, Hq=1, Hkv=1, d=4, beta=1, P=1, K=1, cap=1, n_probes=1, R=1, L=1)
    kbar, _, _ = orc.block_addresses(sh, k, cos, sin, np.ones((1, 1, 1, 4), np.float32) / 2)
    c1, s1, c2, s2 = math.cos(1.0), math.sin(1.0), math.cos(0.01), math.sin(0.01)
    want = [1 * c1 - 3 * s1, 2 * c2 - 4 * s2, 3 * c1 + 1 * s1, 4 * c2 + 2 * s2]
    np.testing.assert_allclose(kbar[0, 0, 1], want, rtol=0, atol=2e-6)
    np.testing.assert_array_equal(kbar[0, 0, 0], x[0])


def test_rope_table_frequencies_and_angle_addition(orc):
    T, d = 200, 64
    cos, sin = orc.rope_table(T, d)
    np.testing.assert_allclose(cos.astype(np.float64) ** 2 + sin.astype(np.float64) ** 2, 1.0,
                               atol=3e-7)
    theta = np.arctan2(sin[1].astype(np.float64), cos[1].astype(np.float64))
    assert abs(theta[0] - 1.0) < 1e-7
    ratio = theta[1:] / theta[:-1]
    np.testing.assert_allclose(ratio, 10000.0 ** (-2.0 / d), rtol=1e-6)
    # angle is linear in position: cos((a+b)w) = cos(aw)cos(bw) - sin(aw)sin(bw)
    a, b = 37, 121
    lhs = cos[a + b].astype(np.float64)
    rhs = cos[a].astype(np.float64) * cos[b] - sin[a].astype(np.float64) * sin[b]
    np.testing.assert_allclose(lhs, rhs, atol=2e-6)


def test_rope_preserves_norm_and_relative_position(orc):
    """||R(t)x|| = ||x||, and <R(m)q, R(n)k> depends only on m - n."""
    T, d = 64, 64
    cos, sin = orc.rope_table(T, d)
    rng = np.random.default_rng(3)
    vq = rng.standard_normal(d).astype(np.float32)
    vk = rng.standard_normal(d).astype(np.float32)
    rows = np.stack([vq, vk] * (T // 2)).reshape(1, T, 1, d)       # even: q, odd: k
    sh = shape(orc, B=1, T=T, Hq=1, Hkv=1, d=d, beta=1, P=1, K=1, cap=1, n_probes=1, R=1, L=1)
    rot, _, _ = orc.block_addresses(sh, rows, cos, sin, np.ones((1, 1, 1, d), np.float32) / 8)
    rot = rot[0, 0].astype(np.float64)
    np.testing.assert_allclose(np.linalg.norm(rot[0::2], axis=1), np.linalg.norm(vq), rtol=2e-6)
    # pairs (m, n) with m - n = 5: q at even m, k at odd n
    dots = [rot[m] @ rot[m - 5] for m in range(6, T, 2)]
    np.testing.assert_allclose(dots, dots[0], atol=5e-5)


# ---------------------------------------------------- summaries, addresses --
def test_block_summary_is_block_mean(orc):
    """With the identity rotation the summary is the mean of the block's keys."""
    B, T, Hkv, d, beta = 2, 48, 3, 8, 4
    rng = np.random.default_rng(5)
    k = rng.standard_normal((B, T, Hkv, d)).astype(np.float32)
    cos, sin = identity_table(T, d)
    sh = shape(orc, B=B, T=T, Hq=Hkv, Hkv=Hkv, d=d, beta=beta, P=2, K=3, cap=4, n_probes=1,
               R=1, L=1)
    cb = synth.codebooks(configs.TINY.with_(Hkv=Hkv, d=d, K=3))
    kbar, _, _ = orc.block_addresses(sh, k, cos, sin, cb)
    want = k.astype(np.float64).reshape(B, T // beta, beta, Hkv, d).mean(axis=2).transpose(0, 2, 1, 3)
    np.testing.assert_allclose(kbar, want, rtol=0, atol=1e-6)


@pytest.mark.parametrize("P,K", [(1, 16), (2, 8), (2, 5)])
def test_address_is_nearest_unit_code_per_component(orc, P, K):
    """Spherical product quantization: with unit-norm codes the argmax inner
    product is the nearest code in Euclidean distance; the address is the
    mixed-radix number of the component codes, component 0 most significant."""
    B, T, Hkv, d, beta = 1, 512, 2, 16, 8
    rng = np.random.default_rng(11 + P * K)
    k = rng.standard_normal((B, T, Hkv, d)).astype(np.float32)
    cos, sin = identity_table(T, d)
    cb = synth.codebooks(configs.TINY.with_(Hkv=Hkv, d=d, P=P, K=K, seed=99))
    sh = shape(orc, B=B, T=T, Hq=Hkv, Hkv=Hkv, d=d, beta=beta, P=P, K=K, cap=4, n_probes=1,
               R=1, L=1)
    kbar, addr, gap = orc.block_addresses(sh, k, cos, sin, cb)
    ds = d // P
    want = np.zeros(addr.shape, np.int64)
    for p in range(P):
        sub = kbar[..., p * ds:(p + 1) * ds].astype(np.float64)          # [B,Hkv,NB,ds]
        codes = cb[:, p].astype(np.float64)                               # [Hkv,K,ds]
        dist = ((sub[:, :, :, None, :] - codes[None, :, None, :, :]) ** 2).sum(-1)
        want = want * K + dist.argmin(-1)
    tie = (gap < NEAR_TIE).any(-1)
    assert (addr[~tie] == want[~tie]).all()
    assert tie.mean() < 1e-2


def test_address_axis_aligned_worked_example(orc):
    """d = 4, P = 2, K = 2; codes are +/- unit axes of each 2-dim sub-vector.
    Block means (+a, -b) choose code 0 in component 0 and code 1 in
    component 1: address 0*2 + 1 = 1."""
    d, T = 4, 4
    cb = np.zeros((1, 2, 2, 2), np.float32)
    cb[0, 0, 0] = [1, 0]
    cb[0, 0, 1] = [-1, 0]
    cb[0, 1, 0] = [0, 1]
    cb[0, 1, 1] = [0, -1]
    k = np.zeros((1, T, 1, d), np.float32)
    k[0, :2, 0] = [0.9, 0.1, 0.2, -0.7]        # block 0 -> (0, 1) -> 1
    k[0, 2:, 0] = [-0.5, 0.0, 0.1, 0.4]        # block 1 -> (1, 0) -> 2
    cos, sin = identity_table(T, d)
    sh = shape(orc, B=1, T=T, Hq=1, Hkv=1, d=d, beta=2, P=2, K=2, cap=2, n_probes=1, R=1, L=1)
    _, addr, _ = orc.block_addresses(sh, k, cos, sin, cb)
    assert addr.ravel().tolist() == [1, 2]


def test_argmax_ties_go_to_lowest_code(orc):
    d, T = 4, 2
    cb = np.zeros((1, 1, 3, 4), np.float32)
    cb[0, 0, 0] = [0, 0, 0, 1]
    cb[0, 0, 1] = [1, 0, 0, 0]
    cb[0, 0, 2] = [1, 0, 0, 0]                  # duplicate of code 1
    k = np.zeros((1, T, 1, d), np.float32)
    k[0, :, 0, 0] = 1.0
    cos, sin = identity_table(T, d)
    sh = shape(orc, B=1, T=T, Hq=1, Hkv=1, d=d, beta=2, P=1, K=3, cap=1, n_probes=1, R=1, L=1)
    _, addr, gap = orc.block_addresses(sh, k, cos, sin, cb)
    assert addr.ravel().tolist() == [1] and gap.ravel()[0] == 0.0


# ------------------------------------------------------------ posting lists --
def characterize_lists(addr, A, cap):
    """What the lists must be, stated directly: each address keeps the first
    `cap` of its blocks in source order."""
    groups = {a: sorted(n for n, x in enumerate(addr) if x == a) for a in range(A)}
    loadv = [len(groups[a]) for a in range(A)]
    kept = [groups[a][:cap] for a in range(A)]
    offsets = [0]
    for a in range(A):
        offsets.append(offsets[-1] + len(kept[a]))
    entries = [n for a in range(A) for n in kept[a]]
    entries += [-1] * (len(addr) - len(entries))
    overflow = sum(max(0, x - cap) for x in loadv)
    return offsets, entries, loadv, overflow


def test_posting_lists_brute_force_enumeration(orc):
    """Every address assignment of NB <= 4 blocks over A <= 3 addresses
    (and NB = 5 over A = 2), every capacity."""
    for NB, A in ((1, 3), (2, 3), (3, 3), (4, 3), (5, 2)):
        for addr in itertools.product(range(A), repeat=NB):
            for cap in range(1, NB + 1):
                off, ent, ld, ov = orc.posting_lists(np.array(addr), A, cap)
                w_off, w_ent, w_ld, w_ov = characterize_lists(addr, A, cap)
                assert off.tolist() == w_off and ent.tolist() == w_ent
                assert ld.tolist() == w_ld and ov == w_ov


def test_posting_lists_equal_stable_sort_when_uncapped(orc):
    rng = np.random.default_rng(2)
    for _ in range(20):
        NB, A = 300, 37
        addr = rng.integers(0, A, NB)
        off, ent, ld, ov = orc.posting_lists(addr, A, NB)
        order = sorted(range(NB), key=lambda n: addr[n])      # Python's sort is stable
        assert ent.tolist() == order and ov == 0
        assert ld.tolist() == np.bincount(addr, minlength=A).tolist()
        assert off.tolist() == [0] + np.cumsum(np.bincount(addr, minlength=A)).tolist()


def test_counter_conservation_and_identical_addresses(orc):
    rng = np.random.default_rng(4)
    for cap in (1, 2, 3, 8):
        addr = rng.integers(0, 16, 200)
        off, ent, ld, ov = orc.posting_lists(addr, 16, cap)
        assert np.minimum(ld, cap).sum() + ov == 200
        assert (np.diff(off) <= cap).all()
    NB, cap = 64, 8
    off, ent, ld, ov = orc.posting_lists(np.full(NB, 5), 16, cap)
    assert ld[5] == NB and ov == NB - cap and ld.sum() == NB
    assert ent[:cap].tolist() == list(range(cap)) and (ent[cap:] == -1).all()


def test_stress_keys_drive_one_address(orc):
    cfg = configs.SMALL.with_(T=1024, Hq=2, Hkv=2, dtype="f32")
    k, cb = synth.stress_keys(cfg, "one_address")
    cos, sin = orc.rope_table(cfg.T, cfg.d)
    sh = orc.Shape.of(**cfg.shape_kw())
    idx = orc.build_index(sh, k, cos, sin, cb)
    assert (idx["addr"] == 0).all()
    assert (idx["overflow"] == cfg.NB - min(cfg.cap, cfg.NB)).all()
    k2, cb2 = synth.stress_keys(cfg.with_(cap=4), "two_clusters")
    idx2 = orc.build_index(orc.Shape.of(**cfg.with_(cap=4).shape_kw()), k2, cos, sin, cb2)
    assert set(np.unique(idx2["addr"]).tolist()) == {0, cfg.K + 1}
    assert (idx2["overflow"] == cfg.NB - 8).all()


# ----------------------------------------------------------------- routing --
def route_setup(orc, cfg, seed_shift=0):
    cfg = cfg.with_(seed=cfg.seed + seed_shift)
    inp = synth.qkv(cfg)
    cos, sin = orc.rope_table(cfg.T, cfg.d)
    sh = orc.Shape.of(**cfg.shape_kw())
    idx = orc.build_index(sh, inp["k"], cos, sin, inp["codebooks"])
    return cfg, sh, inp, cos, sin, idx


def test_six_blocks_five_eligible(orc):
    """Technical report, 'Learned sparse route': six blocks, one local block,
    five eligible remote blocks at the latest queries."""
    g = json.load(open(os.path.join(GOLDEN, "six_blocks.json")))
    cfg = configs.TINY
    assert cfg.NB == g["n_blocks"] and cfg.L == g["local_blocks"]
    # with R >= NB the search is bypassed and the selection is the eligible set
    cfg_all = cfg.with_(R=cfg.NB)
    _, sh, inp, cos, sin, idx = route_setup(orc, cfg_all)
    sel, _ = orc.route(sh, inp["q"], cos, sin, inp["codebooks"], idx)
    sel = sel.reshape(cfg.B, cfg.Hq, cfg.T, cfg.NB)
    latest = sel[:, :, -1]
    assert ((latest >= 0).sum(-1) == g["eligible_remote_blocks_at_latest_query"]).all()
    for t in range(cfg.T):
        qb = t // cfg.beta
        E = max(0, qb - cfg.L + 1)
        assert (sel[:, :, t, :E] == np.arange(E)).all() and (sel[:, :, t, E:] == -1).all()
    # with R = 2 the latest queries select two of the five
    _, sh2, inp2, cos2, sin2, idx2 = route_setup(orc, cfg)
    sel2, _ = orc.route(sh2, inp2["q"], cos2, sin2, inp2["codebooks"], idx2)
    sel2 = sel2.reshape(cfg.B, cfg.Hq, cfg.T, cfg.R)[:, :, -1]
    assert ((sel2 >= 0) & (sel2 <= 4)).all() and g["selected_remote_blocks"] == cfg.R


def rotate64(x, cos, sin):
    h = x.shape[-1] // 2
    a, b = x[..., :h].astype(np.float64), x[..., h:].astype(np.float64)
    c, s = cos.astype(np.float64), sin.astype(np.float64)
    return np.concatenate([a * c - b * s, b * c + a * s], -1)


def rel_gap(best, second):
    """Relative gap of a decision: (best - runner-up) / max(|best|, |runner-up|, 1e-30)."""
    return (best - second) / max(abs(best), abs(second), 1e-30)


def dual_form_selection(cfg, q_row_rot, scores, idx, b, g, qb):
    """The selection written as a threshold on address rank (the dual of the
    walk): pool = indexed eligible blocks whose address rank is <= m, with
    m = max(n_probes, first rank where the eligible count reaches R) (or all
    addresses); then the R best by rerank score.  Scores here are fp64.
    Also returns the two decision gaps: the pool boundary (rank m against
    rank m + 1; +inf when every address is probed) and the rerank boundary
    (R-th kept against the best dropped; +inf when the pool holds <= R)."""
    K, P, A, R, L = cfg.K, cfg.P, cfg.A, cfg.R, cfg.L
    sig = np.zeros(A)
    for a in range(A):
        digits = [(a // K ** (P - 1 - p)) % K for p in range(P)]
        sig[a] = sum(scores[p * K + digits[p]] for p in range(P))
    order = sorted(range(A), key=lambda a: (-sig[a], a))
    rank = {a: i + 1 for i, a in enumerate(order)}
    off, ent = idx["offsets"][b, g], idx["entries"][b, g]
    elig = []
    for a in range(A):
        for n in ent[off[a]:off[a + 1]]:
            if n <= qb - L:
                elig.append((rank[a], int(n)))
    elig.sort()
    if len(elig) >= R:
        m = min(max(cfg.n_probes, elig[R - 1][0]), A)
    else:
        m = A
    pool = [n for r, n in elig if r <= m]
    kbar = idx["kbar"][b, g].astype(np.float64)
    rho = {n: float(q_row_rot @ kbar[n]) for n in pool}
    ranked = sorted(pool, key=lambda n: (-rho[n], n))
    best = ranked[:R]
    gap_pool = math.inf if m >= A else rel_gap(sig[order[m - 1]], sig[order[m]])
    gap_rerank = math.inf if len(pool) <= R else rel_gap(rho[ranked[R - 1]], rho[ranked[R]])
    return sorted(best) + [-1] * (R - len(best)), (gap_pool, gap_rerank)


@pytest.mark.parametrize("cfg_name,n_probes", [("tiny", None), ("small", None), ("small", 1),
                                               ("small_exhaustive", None)])
def test_route_equals_dual_form_brute_force(orc, cfg_name, n_probes):
    """The walk against its dual form, both selections and both decision
    gaps.  The gaps are recomputed here from fp64 scores, so they are
    compared loosely (the oracle takes them from its fp32 scores); a gap
    taken at the wrong boundary, or not at all, is off by far more."""
    if cfg_name == "tiny":
        cfg = configs.TINY
    else:
        cfg = configs.SMALL.with_(T=1024, Hq=2, Hkv=2, K=8, cap=3, dtype="f32")
    if cfg_name == "small_exhaustive":
        cfg = cfg.with_(n_probes=cfg.A)            # probe everything: exhaustive top-R
    if n_probes is not None:
        cfg = cfg.with_(n_probes=n_probes)
    cfg, sh, inp, cos, sin, idx = route_setup(orc, cfg)
    rng = np.random.default_rng(0)
    ids = rng.choice(cfg.routes, size=min(cfg.routes, 300), replace=False)
    sel, gaps = orc.route(sh, inp["q"], cos, sin, inp["codebooks"], idx, ids)
    mism = 0
    n_gaps = [0, 0]
    for i, rid in enumerate(ids):
        t = rid % cfg.T
        h = (rid // cfg.T) % cfg.Hq
        b = rid // (cfg.T * cfg.Hq)
        g, qb = h // cfg.G, t // cfg.beta
        E = max(0, qb - cfg.L + 1)
        if E <= cfg.R:
            want, want_gaps = list(range(E)) + [-1] * (cfg.R - E), (math.inf, math.inf)
        else:
            qr = rotate64(inp["q"][b, t, h], cos[t], sin[t])
            ds = cfg.d // cfg.P
            scores = [qr[p * ds:(p + 1) * ds] @ inp["codebooks"][g, p, c].astype(np.float64)
                      for p in range(cfg.P) for c in range(cfg.K)]
            want, want_gaps = dual_form_selection(cfg, qr, scores, idx, b, g, qb)
        for j in range(2):
            got_g, want_g = gaps[i][j], want_gaps[j]
            if math.isinf(want_g) or math.isinf(got_g):
                assert got_g == want_g, (rid, j, got_g, want_g)
            else:
                assert abs(got_g - want_g) <= 1e-4 * max(1.0, abs(want_g)), (rid, j, got_g, want_g)
                n_gaps[j] += 1
        if sel[i].tolist() != want:
            assert gaps[i].min() < NEAR_TIE, (rid, sel[i], want, gaps[i])
            mism += 1
    assert mism <= 2
    # finite gaps were compared: the pool boundary wherever not every address
    # is probed, the rerank boundary wherever the pool outgrows R (rare in the
    # six-block case, whose lists hold 6 blocks over 64 addresses)
    assert n_gaps[0] > 0 or cfg.n_probes >= cfg.A
    assert n_gaps[1] > 0 or cfg_name == "tiny"


# ------------------------------------------------ routing ties and gaps ----
# Hand-built one-head cases with the identity rotation (cos = 1, sin = 0) and
# one token per block, so every summary, code score, address score and rerank
# score below is an exact small dyadic number and each decision can be
# checked by hand.  Ties break toward the lowest index (the lowest address in
# the walk, the lowest block in the rerank), as the routing rule states.
def hand_route(orc, keys, query, cb, *, R=1, n_probes=1, L=1, cap=4):
    """Index T blocks of one token (keys [T, d]) and route the last token
    (query [d]).  cb is [P, K, d/P].  Returns (addr, sel, gaps)."""
    keys = np.asarray(keys, np.float32)
    T, d = keys.shape
    P, K = cb.shape[0], cb.shape[1]
    cos, sin = identity_table(T, d)
    sh = shape(orc, B=1, T=T, Hq=1, Hkv=1, d=d, beta=1, P=P, K=K, cap=cap,
               n_probes=n_probes, R=R, L=L)
    cb4 = np.asarray(cb, np.float32).reshape(1, P, K, d // P)
    idx = orc.build_index(sh, keys.reshape(1, T, 1, d), cos, sin, cb4)
    q = np.zeros((1, T, 1, d), np.float32)
    q[0, T - 1, 0] = query
    sel, gaps = orc.route(sh, q, cos, sin, cb4, idx, np.array([T - 1]))
    return idx["addr"].ravel().tolist(), sel[0].tolist(), gaps[0].tolist()


# two components of two codes each: +x and +y of a 2-dim sub-vector
AXES2 = np.array([[[1, 0], [0, 1]], [[1, 0], [0, 1]]], np.float32)


def test_address_score_tie_goes_to_lower_address(orc):
    """Blocks 0 and 1 sit at addresses 2 = (1, 0) and 1 = (0, 1); the query
    (1, 0 | 1, 0) scores component codes (1, 0) and (1, 0), so
    sigma = 2, 1, 1, 0 for addresses 0..3.  Address 0 holds no block; the
    next two addresses tie at sigma 1 and the walk takes address 1 first:
    with one probe and R = 1 the pool is its block 1, the selection [1].
    Taking the tie toward the higher address would select block 0.  The
    pool boundary (address 1 against address 2) has gap 0; the pool holds R
    blocks, so no rerank decision is taken (+inf)."""
    keys = [[0, 1, 1, 0],      # block 0 -> codes (1, 0) -> address 2
            [1, 0, 0, 1],      # block 1 -> codes (0, 1) -> address 1
            [0, 1, 0, 1]]      # block 2 (the query's own) -> address 3
    addr, sel, gaps = hand_route(orc, keys, [1, 0, 1, 0], AXES2)
    assert addr == [2, 1, 3]
    assert sel == [1]
    assert gaps[0] == 0.0 and gaps[1] == math.inf


def test_address_score_clear_decision_and_its_gap(orc):
    """The case above with the query (1, 0 | 0.75, 0.25): sigma = 1.75,
    1.25, 0.75, 0.25.  Address 1 is now strictly ahead of address 2, the
    selection is again [1], and the pool boundary gap is
    (1.25 - 0.75) / 1.25 = 0.4, far above the near-tie bound."""
    keys = [[0, 1, 1, 0], [1, 0, 0, 1], [0, 1, 0, 1]]
    addr, sel, gaps = hand_route(orc, keys, [1, 0, 0.75, 0.25], AXES2)
    assert addr == [2, 1, 3] and sel == [1]
    assert gaps[0] == 0.4 and gaps[1] == math.inf
    # the query (0, 1 | 1, 0) puts address 2 = (1, 0) first: sigma 2; then
    # addresses 0 and 3 tie at 1 (both empty or ineligible) and address 1 is
    # last.  Block 0 is taken at the first probe; boundary gap (2 - 1) / 2.
    addr, sel, gaps = hand_route(orc, keys, [0, 1, 1, 0], AXES2)
    assert sel == [0] and gaps[0] == 0.5


# one component of two codes, +x and -x of the 4-dim key: every key with a
# positive first coordinate (and every zero key: a tie, code 0) is address 0
PLUS_MINUS_X = np.array([[[1, 0, 0, 0], [-1, 0, 0, 0]]], np.float32)


def test_rerank_tie_on_zero_keys_goes_to_lower_blocks(orc):
    """Zero keys give zero summaries, address 0 (both codes score 0; the tie
    takes code 0) and a rerank score of exactly 0 for every block.  The
    query block is 4 and L = 1, so blocks 0..3 are eligible and all four sit
    in the one list probed.  R = 2 keeps the two lowest blocks, [0, 1]
    (toward the highest would give [2, 3]); the rerank boundary gap is 0;
    the pool boundary (address 0 at sigma 0.5 against address 1 at -0.5)
    has gap 2."""
    keys = np.zeros((5, 4), np.float32)
    addr, sel, gaps = hand_route(orc, keys, [0.5, 1, 2, 3], PLUS_MINUS_X, R=2)
    assert addr == [0] * 5
    assert sel == [0, 1]
    assert gaps == [2.0, 0.0]


def test_rerank_duplicate_keys_and_clear_gap(orc):
    """Blocks 1 and 3 carry the same key, the best rerank score (1.5) for
    the query (1, 1, 1, 1): with R = 1 the tie keeps block 1 (gap 0).  With
    R = 2 both are kept and the boundary against the next best (block 0,
    score 0.5) has gap (1.5 - 0.5) / 1.5 = 2/3."""
    keys = [[0.25, 0.25, 0, 0],     # rho 0.5
            [0.5, 0.5, 0.25, 0.25],  # rho 1.5
            [0.125, 0, 0, 0],        # rho 0.125
            [0.5, 0.5, 0.25, 0.25],  # rho 1.5 (duplicate of block 1)
            [1, 0, 0, 0]]            # the query's own block
    addr, sel, gaps = hand_route(orc, keys, [1, 1, 1, 1], PLUS_MINUS_X, R=1)
    assert addr == [0] * 5 and sel == [1] and gaps[1] == 0.0
    addr, sel, gaps = hand_route(orc, keys, [1, 1, 1, 1], PLUS_MINUS_X, R=2)
    assert sel == [1, 3] and gaps[1] == (1.5 - 0.5) / 1.5
    # three slots: blocks 1, 3 and 0; the dropped block 2 (0.125) against
    # block 0 (0.5): gap 0.75
    addr, sel, gaps = hand_route(orc, keys, [1, 1, 1, 1], PLUS_MINUS_X, R=3)
    assert sel == [0, 1, 3] and gaps[1] == 0.75


def test_zero_query_walks_addresses_in_order(orc):
    """A zero query scores every address 0: the walk visits addresses in
    ascending order and every rerank score is 0.  Blocks 0..5 sit at
    addresses 3, 1, 1, 2, 0, 3 (query block 6, L = 1).  With two probes and
    R = 3 the walk takes address 0 (block 4), address 1 (blocks 1, 2): the
    pool reaches 3 at the second address.  The rerank ties keep the lowest
    three blocks of the pool, all of it: [1, 2, 4]."""
    keys = [[0, 1, 0, 1],      # (1, 1) -> 3
            [1, 0, 0, 1],      # (0, 1) -> 1
            [1, 0, 0, 1],      # (0, 1) -> 1
            [0, 1, 1, 0],      # (1, 0) -> 2
            [1, 0, 1, 0],      # (0, 0) -> 0
            [0, 1, 0, 1],      # (1, 1) -> 3
            [1, 0, 1, 0]]      # the query's own block
    addr, sel, gaps = hand_route(orc, keys, [0, 0, 0, 0], AXES2, R=3, n_probes=2)
    assert addr == [3, 1, 1, 2, 0, 3, 0]
    assert sel == [1, 2, 4]
    assert gaps == [0.0, math.inf]
    # R = 2: the pool is still blocks 4, 1, 2 (whole lists); the tie keeps 1, 2
    addr, sel, gaps = hand_route(orc, keys, [0, 0, 0, 0], AXES2, R=2, n_probes=1)
    assert sel == [1, 2] and gaps == [0.0, 0.0]


@pytest.mark.parametrize("cfg", [configs.TINY,
                                 configs.SMALL.with_(T=2048, Hq=4, Hkv=2, dtype="f32"),
                                 configs.SMALL.with_(T=2048, Hq=4, Hkv=4, cap=1, dtype="f32")])
def test_route_invariants(orc, cfg):
    """Causality, slot counts, ascending unique ids, bounded lists."""
    cfg, sh, inp, cos, sin, idx = route_setup(orc, cfg)
    sel, gaps = orc.route(sh, inp["q"], cos, sin, inp["codebooks"], idx)
    sel = sel.reshape(cfg.B, cfg.Hq, cfg.T, cfg.R)
    assert (np.diff(idx["offsets"], axis=-1) <= cfg.cap).all()
    for b in range(cfg.B):
        for h in range(cfg.Hq):
            g = h // cfg.G
            ld = idx["load"][b, g]
            addr = idx["addr"][b, g]
            rank_in_addr = np.zeros(cfg.NB, np.int64)
            seen = {}
            for n in range(cfg.NB):
                rank_in_addr[n] = seen.get(addr[n], 0)
                seen[addr[n]] = rank_in_addr[n] + 1
            indexed = rank_in_addr < cfg.cap
            for t in range(cfg.T):
                qb = t // cfg.beta
                E = max(0, qb - cfg.L + 1)
                s = sel[b, h, t]
                valid = s[s >= 0]
                assert (s[len(valid):] == -1).all()
                assert (np.diff(valid) > 0).all()
                assert (valid <= qb - cfg.L).all()                  # causality
                if E <= cfg.R:
                    assert len(valid) == E
                else:
                    assert indexed[valid].all()
                    n_indexed_eligible = int(indexed[:E].sum())
                    assert len(valid) == min(cfg.R, n_indexed_eligible)
                    if indexed[:E].all():
                        assert len(valid) == cfg.R                  # fixed R slots
    assert ld.sum() == cfg.NB


# --------------------------------------------------------------- attention --
def test_all_eligible_equals_dense_causal(orc):
    """Bypass everywhere (R >= eligible blocks) reduces selected-set attention
    to dense causal softmax; the report's bound is 1.91e-6."""
    bound = json.load(open(os.path.join(GOLDEN, "selected_mask_error.json")))["max_abs_error"]
    cfg = configs.ALL_ELIGIBLE.with_(T=1024, Hq=3, Hkv=1, R=15, dtype="f32")
    inp = synth.qkv(cfg)
    cos, sin = orc.rope_table(cfg.T, cfg.d)
    sh = orc.Shape.of(**cfg.shape_kw())
    idx = orc.build_index(sh, inp["k"], cos, sin, inp["codebooks"])
    sel, _ = orc.route(sh, inp["q"], cos, sin, inp["codebooks"], idx)
    out = orc.attention(sh, inp["q"], inp["k"], inp["v"], cos, sin, sel)
    out = out.reshape(cfg.B, cfg.Hq, cfg.T, cfg.d)
    worst = 0.0
    for h in range(cfg.Hq):
        g = h // cfg.G
        dense = orc.dense_causal_attention(inp["q"][0, :, h], inp["k"][0, :, g],
                                           inp["v"][0, :, g], cos, sin)
        worst = max(worst, np.abs(out[0, h] - dense).max())
    assert worst < 1e-12 and worst < bound


@pytest.mark.parametrize("L", [1, 2, 3])
def test_gathered_attention_equals_dense_mask_twin(orc, L):
    cfg = configs.SMALL.with_(T=640, Hq=4, Hkv=2, R=3, L=L, dtype="f32", beta=64)
    inp = synth.qkv(cfg)
    cos, sin = orc.rope_table(cfg.T, cfg.d)
    sel = synth.random_selection(cfg, seed=L)
    sh = orc.Shape.of(**cfg.shape_kw())
    out = orc.attention(sh, inp["q"], inp["k"], inp["v"], cos, sin, sel.reshape(-1, cfg.R))
    out = out.reshape(cfg.B, cfg.Hq, cfg.T, cfg.d)
    for h in range(cfg.Hq):
        g = h // cfg.G
        twin = orc.dense_masked_attention(inp["q"][0, :, h], inp["k"][0, :, g], inp["v"][0, :, g],
                                          cos, sin, sel[0, h], cfg.beta, cfg.L)
        assert np.abs(out[0, h] - twin).max() < 1e-12


def test_attention_is_convex_combination_of_selected_values(orc):
    cfg = configs.SMALL.with_(T=512, Hq=2, Hkv=1, R=2, L=2, dtype="f32")
    inp = synth.qkv(cfg)
    cos, sin = orc.rope_table(cfg.T, cfg.d)
    sel = synth.random_selection(cfg, seed=9)
    sh = orc.Shape.of(**cfg.shape_kw())
    out = orc.attention(sh, inp["q"], inp["k"], inp["v"], cos, sin, sel.reshape(-1, cfg.R))
    out = out.reshape(cfg.Hq, cfg.T, cfg.d)
    for h in range(cfg.Hq):
        for t in range(0, cfg.T, 7):
            qb = t // cfg.beta
            blocks = set(sel[0, h, t][sel[0, h, t] >= 0].tolist())
            blocks.update(range(max(0, qb - cfg.L + 1), qb + 1))
            toks = [s for s in range(t + 1) if s // cfg.beta in blocks]
            vals = inp["v"][0, toks, 0].astype(np.float64)
            assert (out[h, t] >= vals.min(0) - 1e-12).all()
            assert (out[h, t] <= vals.max(0) + 1e-12).all()
    # the first query of the sequence sees only itself
    np.testing.assert_allclose(out[:, 0], np.broadcast_to(inp["v"][0, 0, 0], (cfg.Hq, cfg.d)),
                               rtol=0, atol=1e-15)


def test_local_window_covering_sequence_is_dense(orc):
    cfg = configs.SMALL.with_(T=384, Hq=2, Hkv=2, R=1, L=6, dtype="f32")
    inp = synth.qkv(cfg)
    cos, sin = orc.rope_table(cfg.T, cfg.d)
    sh = orc.Shape.of(**cfg.shape_kw())
    sel = np.full((cfg.routes, cfg.R), -1, np.int32)
    out = orc.attention(sh, inp["q"], inp["k"], inp["v"], cos, sin, sel).reshape(cfg.Hq, cfg.T, -1)
    for h in range(cfg.Hq):
        dense = orc.dense_causal_attention(inp["q"][0, :, h], inp["k"][0, :, h], inp["v"][0, :, h],
                                           cos, sin)
        assert np.abs(out[h] - dense).max() < 1e-12


def test_mixer_output_projection_and_rounding(orc):
    """With W_o = identity the delta is the concatenated head outputs; the
    stored projections are the exact products rounded once to bf16."""
    cfg = configs.TINY.with_(dtype="bf16")
    inp = synth.mixer_inputs(cfg)
    cos, sin = orc.rope_table(cfg.T, cfg.d)
    sh = orc.Shape.of(**cfg.shape_kw())
    eye = np.eye(cfg.Hq * cfg.d, cfg.W, dtype=np.float32)
    res = orc.mixer(sh, inp["x"], inp["w_qkv"], eye, inp["codebooks"], cos, sin, "bf16")
    o = orc.attention(sh, res["q"], res["k"], res["v"], cos, sin, res["sel"])
    o = o.reshape(cfg.B, cfg.Hq, cfg.T, cfg.d).transpose(0, 2, 1, 3).reshape(cfg.B, cfg.T, -1)
    np.testing.assert_array_equal(res["delta"], o)
    exact = inp["x"].astype(np.float64).reshape(-1, cfg.W) @ inp["w_qkv"].astype(np.float64)
    q = res["q"].reshape(-1, cfg.Hq * cfg.d).astype(np.float64)
    err = np.abs(q - exact[:, :cfg.Hq * cfg.d]) / np.maximum(np.abs(exact[:, :cfg.Hq * cfg.d]), 1e-30)
    assert err.max() <= 2.0 ** -8 + 1e-12
    # bf16 values: the low 16 bits of every stored float32 are zero
    assert (res["q"].view(np.uint32) & 0xFFFF == 0).all()


def test_bypass_boundary_with_overflowed_blocks(orc):
    """All blocks on one address with capacity 1: only block 0 is indexed.
    With E <= R the search is bypassed and the eligible blocks are taken
    as they are (E = R = 2 gives [0, 1]); above that the pool holds only
    indexed blocks, so the selection is [0, -1]."""
    cfg = configs.SMALL.with_(T=512, Hq=2, Hkv=2, cap=1, R=2, L=1, dtype="f32")
    k, cb = synth.stress_keys(cfg, "one_address")
    inp = synth.qkv(cfg)
    cos, sin = orc.rope_table(cfg.T, cfg.d)
    sh = orc.Shape.of(**cfg.shape_kw())
    idx = orc.build_index(sh, k, cos, sin, cb)
    assert (idx["addr"] == 0).all() and (idx["overflow"] == cfg.NB - 1).all()
    sel, _ = orc.route(sh, inp["q"], cos, sin, cb, idx)
    sel = sel.reshape(cfg.B, cfg.Hq, cfg.T, cfg.R)
    for t in range(cfg.T):
        qb = t // cfg.beta
        E = max(0, qb - cfg.L + 1)
        want = ([0, 1] if E == 2 else [0, -1] if E == 1 else [-1, -1]) if E <= 2 else [0, -1]
        assert sel[:, :, t].tolist() == [[want] * cfg.Hq] * cfg.B, (t, sel[:, :, t])


# ------------------------------------------------------ codebook calibration ----
def unit(x):
    x = np.asarray(x, np.float64)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def test_calibrate_single_code_is_normalized_sum(orc):
    """K = 1: every point joins the one code, so one round leaves the
    normalized sum of all points (closed form), whatever the start."""
    rng = np.random.default_rng(31)
    kbar = rng.standard_normal((2, 3, 5, 8)).astype(np.float32)   # B, Hkv, NB, d
    cb0 = unit(rng.standard_normal((3, 2, 1, 4))).astype(np.float32)
    cb = orc.calibrate(kbar, cb0, 1)
    for g in range(3):
        for p in range(2):
            pts = kbar[:, g, :, 4 * p:4 * p + 4].reshape(-1, 4).astype(np.float64)
            want = unit(pts.sum(0))
            np.testing.assert_allclose(cb[g, p, 0], want, atol=2e-6)


def test_calibrate_zero_rounds_is_identity(orc):
    rng = np.random.default_rng(32)
    kbar = rng.standard_normal((1, 2, 6, 8)).astype(np.float32)
    cb0 = unit(rng.standard_normal((2, 2, 3, 4))).astype(np.float32)
    assert np.array_equal(orc.calibrate(kbar, cb0, 0), cb0)


def clustered_points(rng, dirs, n_per, noise):
    pts, lab = [], []
    for c, u in enumerate(dirs):
        pts.append(u[None, :] + noise * rng.standard_normal((n_per, len(u))))
        lab += [c] * n_per
    pts = np.concatenate(pts)
    perm = rng.permutation(len(pts))
    return pts[perm].astype(np.float32), np.array(lab)[perm]


def test_calibrate_recovers_separated_clusters(orc):
    """Points around four orthogonal directions, codes started as rotated
    guesses: calibration assigns every point to its own cluster and ends at a
    fixed point where each code is the normalized mean of its members
    (recomputed here in fp64) and each point takes its nearest code."""
    rng = np.random.default_rng(33)
    ds, K = 8, 4
    dirs = np.eye(ds)[:K]
    pts, lab = clustered_points(rng, dirs, 40, 0.05)          # 160 points
    kbar = pts.reshape(1, 1, -1, ds)                          # B=1, Hkv=1, NB=160, d=ds, P=1
    start = unit(dirs + 0.6 * rng.standard_normal((K, ds)))
    cb = orc.calibrate(kbar, start.reshape(1, 1, K, ds).astype(np.float32), 20)[0, 0]
    scores = pts.astype(np.float64) @ cb.T.astype(np.float64)
    asg = scores.argmax(1)
    # every cluster maps to one code, one to one
    mapping = {c: set(asg[lab == c]) for c in range(K)}
    assert all(len(v) == 1 for v in mapping.values())
    assert len(set.union(*mapping.values())) == K
    cluster_of = {next(iter(v)): k for k, v in mapping.items()}
    for c in range(K):
        members = pts[asg == c].astype(np.float64)
        np.testing.assert_allclose(cb[c], unit(members.sum(0)), atol=3e-6)
        assert float(cb[c] @ dirs[cluster_of[c]]) > 0.99


def test_calibrate_objective_never_decreases_and_codes_stay_unit(orc):
    """Spherical k-means: neither the assignment nor the normalized-mean
    update lowers sum_x max_c <x, c>; every code with members has unit norm;
    a code that no point is nearest to keeps its value."""
    rng = np.random.default_rng(34)
    B, Hkv, NB, d, P, K = 2, 2, 64, 16, 2, 6
    kbar = (rng.standard_normal((B, Hkv, NB, d)) + 0.8).astype(np.float32)   # skewed cloud
    cb0 = unit(rng.standard_normal((Hkv, P, K, d // P)))
    cb0[1, 0, K - 1] = -unit(np.ones(d // P))      # points away from every point
    cb0 = cb0.astype(np.float32)
    ds = d // P

    def objective(cb):
        tot = 0.0
        for g in range(Hkv):
            for p in range(P):
                x = kbar[:, g, :, p * ds:(p + 1) * ds].reshape(-1, ds).astype(np.float64)
                tot += (x @ cb[g, p].T.astype(np.float64)).max(1).sum()
        return tot

    prev = objective(cb0)
    for it in range(1, 9):
        cb = orc.calibrate(kbar, cb0, it)
        cur = objective(cb)
        assert cur >= prev - 1e-4 * abs(prev), (it, prev, cur)
        prev = cur
        norms = np.linalg.norm(cb.astype(np.float64), axis=-1)
        moved = np.abs(cb - cb0).max(-1) > 0
        assert np.abs(norms[moved] - 1.0).max() < 2e-6
    assert np.array_equal(cb[1, 0, K - 1], cb0[1, 0, K - 1])


def test_calibrate_lowers_overflow_on_concentrated_keys(orc):
    """The effect the report page shows (section "Capacity", Figure 3), on
    synthetic concentrated keys: with random codebooks almost every block of
    a held-out sequence lands on one address and overflows; codebooks
    calibrated on separate training sequences spread the same blocks."""
    cfg = configs.SMALL.with_(T=2048, Hq=2, Hkv=2, K=8, cap=8, dtype="f32")
    train_k, cb0 = synth.concentrated_keys(cfg.with_(B=4), seed=41)
    test_k, _ = synth.concentrated_keys(cfg, seed=42)
    c, s = orc.rope_table(cfg.T, cfg.d)
    sh = orc.Shape.of(**cfg.shape_kw())
    before = orc.build_index(sh, test_k, c, s, cb0)
    train_idx = orc.build_index(orc.Shape.of(**cfg.with_(B=4).shape_kw()), train_k, c, s, cb0)
    cb = orc.calibrate(train_idx["kbar"], cb0, 10)
    after = orc.build_index(sh, test_k, c, s, cb)
    assert before["overflow"].sum() > 0
    assert after["overflow"].sum() < before["overflow"].sum()
    assert after["load"].max() < before["load"].max()
