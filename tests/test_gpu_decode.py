"""GPU incremental decode (mono_decode_index, mono_decode_step) against the
oracle.

- The index grown block by block equals the oracle's whole-sequence build of
  the same block prefix, bit for bit (summaries, addresses, lists, loads,
  overflow), for ragged token counts, several blocks at once, and capacity
  overflow.
- A decode step at position t equals row t of the oracle's whole-sequence
  route (selected ids bit for bit, near-ties excused as for mono_route) and
  attention (fp32 within 1e-4 max abs, bf16 within 2e-2 max relative per
  (batch, head)), with the index grown by mono_decode_index or built by
  mono_build_index over the same layout, with and without the index's
  rotated-key copy (which the step then reads for the selected blocks).
- That copy holds, for every indexed block and no other, the keys rotated in
  fp32 (products rounded before the add) and rounded to the activation dtype.
"""
import numpy as np
import pytest

from learned_sparse_causal_amd import binding, configs, synth
from parity import (BF16_RTOL, F32_ATOL, MAX_EXCUSED, NEAR_TIE, compare_index, dev, host,
                    index_to_host, say, small_inputs, torch)

pytestmark = pytest.mark.gpu


def oracle_prefix_index(orc, cfg, k, codebooks, nb):
    """The oracle's whole-sequence build over the first nb blocks."""
    T = nb * cfg.beta
    c, s = orc.rope_table(T, cfg.d)
    sh = orc.Shape.of(**cfg.with_(T=T).shape_kw())
    return orc.build_index(sh, np.ascontiguousarray(k[:, :T]), c, s, codebooks)


def check_prefix_index(orc, cfg, gpu, k, codebooks, nb):
    if nb == 0:
        assert (gpu["offsets"] == 0).all() and (gpu["entries"] == -1).all()
        assert (gpu["load"] == 0).all() and (gpu["overflow"] == 0).all()
        return set()
    ref = oracle_prefix_index(orc, cfg, k, codebooks, nb)
    pre = dict(gpu)
    for name in ("kbar", "addr", "entries"):
        pre[name] = np.ascontiguousarray(gpu[name][:, :, :nb])
    assert (gpu["entries"][:, :, nb:] == -1).all()
    return compare_index(cfg.with_(T=nb * cfg.beta), pre, ref)


INDEX_CFGS = [configs.TINY,
              configs.SMALL.with_(name="gqa_T2048", T=2048, Hq=6, Hkv=2),
              # 16 addresses, capacity 2: lists overflow as blocks arrive
              configs.SMALL.with_(name="cap2_A16", T=2048, K=4, cap=2, Hq=2, Hkv=2),
              configs.SMALL.with_(name="d128_beta128", d=128, beta=128, T=4096, Hq=4, Hkv=1,
                                  R=8)]


@pytest.mark.parametrize("cfg", INDEX_CFGS, ids=lambda c: c.name)
def test_decode_index_grows_like_prefix_builds(orc, cfg):
    say("[decode index] %s" % cfg.name)
    t = torch()
    inp, d = small_inputs(cfg)
    cos, sin = binding.device_rope(cfg)
    cb = t.from_numpy(inp["codebooks"]).cuda()
    idx = binding.empty_index(cfg)
    beta = cfg.beta
    # token counts: empty, a partial block, one block, one more token, several
    # blocks in one call, blocks one at a time, the whole cache
    steps = [0, beta // 2, beta, beta + 1, 5 * beta + 3, 6 * beta, 7 * beta - 1, 7 * beta,
             cfg.T - beta, cfg.T]
    steps = sorted(set(x for x in steps if x <= cfg.T))
    done = 0
    for n_tok in steps:
        binding.decode_index(cfg, d["k"], cos, sin, cb, idx, done, n_tok)
        done = n_tok // beta
        check_prefix_index(orc, cfg, index_to_host(idx), inp["k"], inp["codebooks"], done)
    g = index_to_host(idx)
    say("  %d steps, final overflow %d, max load %d" % (len(steps), g["overflow"].sum(),
                                                       g["load"].max()))
    if cfg.cap == 2:
        assert g["overflow"].sum() > 0


def expected_rotated_keys(cfg, k, cos, sin):
    """Keys [B, T, Hkv, d] rotated in fp32 (each product rounded before the
    add), rounded to the activation dtype (round to nearest even)."""
    t = torch()
    x = t.from_numpy(np.ascontiguousarray(k, dtype=np.float32))
    c = t.from_numpy(cos)[None, :, None, :]
    s = t.from_numpy(sin)[None, :, None, :]
    h = cfg.d // 2
    x0, x1 = x[..., :h], x[..., h:]
    r = t.cat([x0 * c - x1 * s, x1 * c + x0 * s], dim=-1)
    return r.to(t.bfloat16).float().numpy() if cfg.dtype == "bf16" else r.numpy()


ROT_CFGS = [configs.SMALL.with_(name="gqa_T2048", T=2048, Hq=6, Hkv=2),
            configs.SMALL.with_(name="d128_beta128_f32", d=128, beta=128, T=4096, Hq=4, Hkv=1,
                                R=8, dtype="f32")]


@pytest.mark.parametrize("cfg", ROT_CFGS, ids=lambda c: c.name)
def test_decode_index_writes_rotated_keys(cfg):
    say("[decode index, rotated keys] %s" % cfg.name)
    t = torch()
    inp, d = small_inputs(cfg)
    cos, sin = binding.device_rope(cfg)
    cb = t.from_numpy(inp["codebooks"]).cuda()
    idx = binding.empty_index(cfg, rotated_keys=True)
    idx["k_rot"].fill_(7.0)                          # sentinel for rows not indexed
    want = expected_rotated_keys(cfg, inp["k"], host(cos), host(sin))
    done = 0
    for n_tok in (3 * cfg.beta + 5, 8 * cfg.beta, cfg.T):
        binding.decode_index(cfg, d["k"], cos, sin, cb, idx, done, n_tok)
        done = n_tok // cfg.beta
        got = host(idx["k_rot"])
        T_ix = done * cfg.beta
        assert np.array_equal(got[:, :T_ix], want[:, :T_ix])
        assert (got[:, T_ix:] == 7.0).all()
    full = binding.build_index(cfg, d["k"], cos, sin, cb, rotated_keys=True)
    assert np.array_equal(host(full["k_rot"]), want)


def decode_positions(cfg, rng, n_random):
    beta, L, R = cfg.beta, cfg.L, cfg.R
    first_search = (R + L) * beta                     # first position with E > R
    fixed = [0, 1, beta - 1, beta, first_search - 1, first_search, first_search + beta - 1,
             cfg.T // 2, cfg.T - beta, cfg.T - 1]
    extra = rng.choice(cfg.T, n_random, replace=False)
    return np.array(sorted(set(int(x) for x in [*fixed, *extra] if 0 <= x < cfg.T)))


def oracle_rows(orc, cfg, inp, positions):
    c, s = orc.rope_table(cfg.T, cfg.d)
    sh = orc.Shape.of(**cfg.shape_kw())
    idx = orc.build_index(sh, inp["k"], c, s, inp["codebooks"])
    bh = np.arange(cfg.B * cfg.Hq)
    ids = (bh[:, None] * cfg.T + positions[None, :]).reshape(-1).astype(np.int64)
    sel, gaps = orc.route(sh, inp["q"], c, s, inp["codebooks"], idx, ids)
    out = orc.attention(sh, inp["q"], inp["k"], inp["v"], c, s, sel, ids)
    return idx, ids, sel, gaps, out


def compare_decode(cfg, orc_idx, ids, o_sel, gaps, o_out, g_sel, g_out):
    """g_sel [n, R] and g_out [n, d] in the order of ids.  Routes whose GPU
    selection differs must be oracle near-ties (or belong to a (b, kv-head)
    with a near-tie address), and such excused routes stay below 0.01 % of
    the rows compared, as for mono_route; attention is compared where
    selections agree."""
    tie_bg = (orc_idx["gap"] < NEAR_TIE).any(-1).any(-1)       # [B, Hkv]
    diff = (g_sel != o_sel).any(-1)
    for i in np.nonzero(diff)[0]:
        rid = int(ids[i])
        b, h = divmod(rid // cfg.T, cfg.Hq)
        assert gaps[i].min() < NEAR_TIE or tie_bg[b, h // cfg.G], \
            "route (b=%d h=%d t=%d): gpu %s oracle %s" % (b, h, rid % cfg.T, g_sel[i], o_sel[i])
    assert diff.sum() <= MAX_EXCUSED * len(ids), "%d excused of %d rows" % (diff.sum(), len(ids))
    keep = ~diff
    err = np.abs(g_out[keep].astype(np.float64) - o_out[keep])
    if cfg.dtype == "f32":
        worst = err.max()
        assert worst <= F32_ATOL, worst
    else:
        worst = 0.0
        bh = ids[keep] // cfg.T
        for x in np.unique(bh):
            m = bh == x
            worst = max(worst, err[m].max() / np.abs(o_out[keep][m]).max())
        assert worst <= BF16_RTOL, worst
    return int(diff.sum()), worst


STEP_CFGS = [configs.TINY,
             configs.SMALL.with_(name="gqa_T2048", T=2048, Hq=6, Hkv=2),
             configs.SMALL.with_(name="L3_R5_probes8", T=2048, Hq=4, Hkv=2, L=3, R=5,
                                 n_probes=8),
             configs.SMALL.with_(name="cap2_A16", T=2048, K=4, cap=2, Hq=2, Hkv=2),
             configs.SMALL.with_(name="d128_beta128_f32", d=128, beta=128, T=4096, Hq=4, Hkv=1,
                                 R=8, n_probes=8, dtype="f32"),
             configs.SMALL.with_(name="P1_K64", T=2048, P=1, K=64, Hq=4, Hkv=2)]


@pytest.mark.parametrize("rotated", [False, True], ids=["raw_keys", "rotated_keys"])
@pytest.mark.parametrize("cfg", STEP_CFGS, ids=lambda c: c.name)
def test_decode_steps_match_whole_sequence_rows(orc, cfg, rotated):
    say("[decode step] %s %s" % (cfg.name, "rotated keys" if rotated else "raw keys"))
    t = torch()
    inp, d = small_inputs(cfg)
    positions = decode_positions(cfg, np.random.default_rng(21), 12)
    o_idx, ids, o_sel, gaps, o_out = oracle_rows(orc, cfg, inp, positions)
    cos, sin = binding.device_rope(cfg)
    cb = t.from_numpy(inp["codebooks"]).cuda()
    idx = binding.empty_index(cfg, rotated_keys=rotated)
    g_sel = np.empty((cfg.B, cfg.Hq, len(positions), cfg.R), np.int32)
    g_out = np.empty((cfg.B, cfg.Hq, len(positions), cfg.d), np.float32)
    done = 0
    for i, pos in enumerate(positions):
        binding.decode_index(cfg, d["k"], cos, sin, cb, idx, done, pos + 1)
        done = (pos + 1) // cfg.beta
        sel, out = binding.decode_step(cfg, d["q"][:, pos].contiguous(), d["k"], d["v"], cos, sin,
                                       cb, idx, pos)
        g_sel[:, :, i] = host(sel)
        g_out[:, :, i] = host(out)
    n, worst = compare_decode(cfg, o_idx, ids, o_sel, gaps, o_out, g_sel.reshape(-1, cfg.R),
                              g_out.reshape(-1, cfg.d))
    say("  %d positions x %d heads: %d excused routes, attention error %.3g"
        % (len(positions), cfg.B * cfg.Hq, n, worst))


def test_decode_step_all_eligible(orc):
    """Every remote block eligible within R: decode takes every block and
    equals the dense causal row."""
    cfg = configs.ALL_ELIGIBLE
    say("[decode step] %s" % cfg.name)
    t = torch()
    inp, d = small_inputs(cfg)
    positions = np.array([0, 63, 64, 4095, cfg.T - 1])
    cos, sin = binding.device_rope(cfg)
    cb = t.from_numpy(inp["codebooks"]).cuda()
    idx = binding.build_index(cfg, d["k"], cos, sin, cb)
    c, s = orc.rope_table(cfg.T, cfg.d)
    worst = 0.0
    for pos in positions:
        sel, out = binding.decode_step(cfg, d["q"][:, pos].contiguous(), d["k"], d["v"], cos, sin,
                                       cb, idx, int(pos))
        qb = pos // cfg.beta
        want = np.where(np.arange(cfg.R) < qb, np.arange(cfg.R), -1)
        assert (host(sel) == want).all()
        o = host(out)
        for h in (0, 7, 14):
            ref = orc.dense_causal_attention(inp["q"][0, :, h], inp["k"][0, :, h // cfg.G],
                                             inp["v"][0, :, h // cfg.G], c, s, [pos])[0]
            worst = max(worst, np.abs(o[0, h] - ref).max() / np.abs(ref).max())
    say("  max relative error vs dense %.3g" % worst)
    assert worst <= BF16_RTOL


def test_decode_step_large_with_prefill_index(orc):
    """Largest workload (batch 8, 64K-token cache, d 128): the index built by
    mono_build_index over the whole cache (with and without its rotated-key
    copy), decode steps at the last position and two others, every
    (batch, head), against the oracle's rows."""
    cfg = configs.LARGE
    say("[decode step] %s" % cfg.name)
    t = torch()
    d = synth.qkv_device(cfg)
    cos, sin = binding.device_rope(cfg)
    cb = t.from_numpy(d["codebooks"]).cuda()
    positions = np.array([cfg.T // 2 + 77, cfg.T - cfg.beta, cfg.T - 1])
    results = {}
    for rotated in (False, True):
        idx = binding.build_index(cfg, d["k"], cos, sin, cb, rotated_keys=rotated)
        g_sel = np.empty((cfg.B, cfg.Hq, len(positions), cfg.R), np.int32)
        g_out = np.empty((cfg.B, cfg.Hq, len(positions), cfg.d), np.float32)
        for i, pos in enumerate(positions):
            sel, out = binding.decode_step(cfg, d["q"][:, pos].contiguous(), d["k"], d["v"], cos,
                                           sin, cb, idx, int(pos))
            g_sel[:, :, i] = host(sel)
            g_out[:, :, i] = host(out)
        results[rotated] = (g_sel, g_out)
        del idx
    inp = {k: host(d[k]) for k in ("q", "k", "v")}
    inp["codebooks"] = d["codebooks"]
    o_idx, ids, o_sel, gaps, o_out = oracle_rows(orc, cfg, inp, positions)
    for rotated, (g_sel, g_out) in results.items():
        n, worst = compare_decode(cfg, o_idx, ids, o_sel, gaps, o_out, g_sel.reshape(-1, cfg.R),
                                  g_out.reshape(-1, cfg.d))
        say("  %s: %d routes, %d excused, attention error %.3g"
            % ("rotated keys" if rotated else "raw keys", len(ids), n, worst))


def test_decode_overflowed_lists():
    """Every block on one address with capacity 1: searched decode queries see
    one indexed block (block 0) and pad with -1."""
    cfg = configs.SMALL.with_(name="one_address_cap1", T=2048, cap=1, R=2, L=1, Hq=2, Hkv=2)
    say("[decode step] %s" % cfg.name)
    t = torch()
    k, cb_np = synth.stress_keys(cfg, "one_address")
    inp = synth.qkv(cfg)
    kd, qd, vd = dev(k, cfg.dtype), dev(inp["q"], cfg.dtype), dev(inp["v"], cfg.dtype)
    cos, sin = binding.device_rope(cfg)
    cb = t.from_numpy(cb_np).cuda()
    idx = binding.empty_index(cfg)
    binding.decode_index(cfg, kd, cos, sin, cb, idx, 0, cfg.T)
    g = index_to_host(idx)
    assert (g["overflow"] == cfg.NB - 1).all()
    for pos in (3 * cfg.beta, cfg.T - 1):
        sel, _ = binding.decode_step(cfg, qd[:, pos].contiguous(), kd, vd, cos, sin, cb, idx, pos)
        assert (host(sel) == np.array([0, -1])).all()


def test_decode_is_deterministic():
    cfg = configs.SMALL.with_(name="det", T=2048, Hq=4, Hkv=2)
    t = torch()
    inp, d = small_inputs(cfg)
    cos, sin = binding.device_rope(cfg)
    cb = t.from_numpy(inp["codebooks"]).cuda()
    idx = binding.build_index(cfg, d["k"], cos, sin, cb)
    q = d["q"][:, cfg.T - 1].contiguous()
    a = binding.decode_step(cfg, q, d["k"], d["v"], cos, sin, cb, idx, cfg.T - 1)
    b = binding.decode_step(cfg, q, d["k"], d["v"], cos, sin, cb, idx, cfg.T - 1)
    t.cuda.synchronize()
    assert t.equal(a[0], b[0]) and t.equal(a[1], b[1])
