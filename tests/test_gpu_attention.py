"""GPU selected-set attention (mono_selected_attention) against the oracle:
fp32 within 1e-4 max abs, bf16 within 2e-2 max relative per (batch, head);
the all-eligible configuration against textbook dense causal attention."""
import numpy as np
import pytest

from learned_sparse_causal_amd import binding, configs, synth
from parity import check_attention, dev, host, sample_routes, say, small_inputs, torch

pytestmark = pytest.mark.gpu


def gpu_attention(cfg, d, sel_np):
    t = torch()
    cos, sin = binding.device_rope(cfg)
    sel = t.from_numpy(np.ascontiguousarray(sel_np, np.int32)).cuda()
    out = binding.selected_attention(cfg, d["q"], d["k"], d["v"], cos, sin, sel)
    t.cuda.synchronize()
    return host(out)


def oracle_attention(orc, cfg, inp, sel_np, ids):
    c, s = orc.rope_table(cfg.T, cfg.d)
    sh = orc.Shape.of(**cfg.shape_kw())
    return orc.attention(sh, inp["q"], inp["k"], inp["v"], c, s,
                         sel_np.reshape(-1, cfg.R)[ids], ids)


CFGS = [configs.TINY, configs.SMALL, configs.sweep(4096),
        configs.SMALL.with_(name="gqa_L3_R5", Hq=6, Hkv=2, L=3, R=5),
        configs.SMALL.with_(name="d128_beta128", d=128, beta=128, T=4096, Hq=4, Hkv=1, R=8),
        configs.SMALL.with_(name="d128_beta64_f32", d=128, T=2048, Hq=2, Hkv=2, dtype="f32"),
        configs.SMALL.with_(name="d64_beta128_f32", beta=128, T=2048, Hq=2, Hkv=1, dtype="f32",
                            R=3),
        # T not a multiple of the 1024-token prep segment or 256-row chunks; batch 2
        configs.SMALL.with_(name="ragged_T4160_B2", T=4160, B=2, Hq=4, Hkv=2, R=3)]


@pytest.mark.parametrize("cfg", CFGS, ids=lambda c: c.name)
def test_attention_parity(orc, cfg):
    say("[attn] %s" % cfg.name)
    inp, d = small_inputs(cfg)
    sel = synth.random_selection(cfg, seed=11)
    out = gpu_attention(cfg, d, sel)
    ids = np.arange(cfg.routes) if cfg.routes <= 40000 else sample_routes(cfg, 40000, seed=3)
    ref = oracle_attention(orc, cfg, inp, sel, ids)
    e = check_attention(cfg, out, ref, ids)
    say("  error %.3g" % e)


def test_attention_invalid_and_duplicate_ids_are_ignored(orc):
    cfg = configs.SMALL.with_(name="dirty_sel", Hq=2, Hkv=2, R=4, L=2)
    say("[attn] %s" % cfg.name)
    inp, d = small_inputs(cfg)
    sel = synth.random_selection(cfg, seed=5)
    rng = np.random.default_rng(6)
    dirty = sel.copy()
    qb = np.arange(cfg.T) // cfg.beta
    pick = rng.random(dirty.shape[:3]) < 0.3
    dirty[..., 3] = np.where(pick, dirty[..., 0], dirty[..., 3])                 # duplicate
    late = rng.random(dirty.shape[:3]) < 0.2
    dirty[..., 2] = np.where(late, (qb + 1)[None, None, :], dirty[..., 2])     # future block
    clean = dirty.copy()
    for b in range(cfg.B):
        for h in range(cfg.Hq):
            for t in range(cfg.T):
                row, seen = clean[b, h, t], set()
                for r in range(cfg.R):
                    x = row[r]
                    if x < 0 or x > qb[t] - cfg.L or x in seen:
                        row[r] = -1
                    else:
                        seen.add(x)
    out = gpu_attention(cfg, d, dirty)
    ids = np.arange(cfg.routes)
    ref = oracle_attention(orc, cfg, inp, clean, ids)
    check_attention(cfg, out, ref, ids)


def test_attention_parity_32k_sampled(orc):
    cfg = configs.SWEEP_32K
    say("[attn] %s sampled" % cfg.name)
    inp, d = small_inputs(cfg)
    sel = synth.random_selection(cfg, seed=12)
    out = gpu_attention(cfg, d, sel)
    ids = sample_routes(cfg, 30000, seed=4, must=[(0, 7)])
    ref = oracle_attention(orc, cfg, inp, sel, ids)
    say("  error %.3g" % check_attention(cfg, out, ref, ids))


def test_attention_parity_large_sampled(orc):
    cfg = configs.LARGE
    say("[attn] %s sampled" % cfg.name)
    d = synth.qkv_device(cfg)
    sel = synth.random_selection(cfg, seed=13, drop_prob=0.02)
    out = gpu_attention(cfg, d, sel)
    ids = sample_routes(cfg, 6000, seed=5)
    inp = {k: host(d[k]) for k in ("q", "k", "v")}
    ref = oracle_attention(orc, cfg, inp, sel, ids)
    say("  error %.3g" % check_attention(cfg, out, ref, ids))


def test_all_eligible_equals_dense_causal(orc):
    """Configuration with every remote block eligible within R: the route is the
    bypass everywhere and the result must equal dense causal softmax."""
    cfg = configs.ALL_ELIGIBLE
    say("[attn] %s dense equivalence" % cfg.name)
    t = torch()
    inp, d = small_inputs(cfg)
    cos, sin = binding.device_rope(cfg)
    cb = t.from_numpy(inp["codebooks"]).cuda()
    idx = binding.build_index(cfg, d["k"], cos, sin, cb)
    sel = binding.route(cfg, d["q"], cos, sin, cb, idx)
    out = host(binding.selected_attention(cfg, d["q"], d["k"], d["v"], cos, sin, sel))
    assert host(idx["overflow"]).sum() == 0
    c, s = orc.rope_table(cfg.T, cfg.d)
    rows = np.unique(np.concatenate([np.arange(0, cfg.T, 37), np.arange(cfg.T - 64, cfg.T)]))
    worst = 0.0
    for h in (0, 7, 14):
        g = h // cfg.G
        ref = orc.dense_causal_attention(inp["q"][0, :, h], inp["k"][0, :, g], inp["v"][0, :, g],
                                         c, s, rows)
        err = np.abs(out[0, rows, h] - ref).max() / np.abs(ref).max()
        worst = max(worst, err)
    say("  max relative error vs dense %.3g" % worst)
    assert worst <= 2e-2
