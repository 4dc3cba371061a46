"""Every point of the scaling sweep (4K, 8K, 16K and 32K tokens), run as the
whole step in one call (mono_routed_attention, the call the benchmark times)
and checked against the oracle, as the technical report's section
"Finite-range scaling" checks each of its lengths (and at 64K tokens): the whole index (block
summaries, addresses, lists, loads and counters) bit for bit with zero
overflow; sampled routes bit for bit (near-ties excused under the 0.01 %
cap) with the causality and fixed-slot checks on every route; sampled
attention rows within 2e-2 max relative per (batch, head)."""
import numpy as np
import pytest

from learned_sparse_causal_amd import binding, configs
from parity import (check_attention, check_sel_invariants, compare_index, compare_sel, host,
                    index_to_host, sample_routes, say, small_inputs, torch)

pytestmark = pytest.mark.gpu


# the four sweep lengths, and 64K tokens (the comparison's longest length;
# late query blocks there leave few lanes needing the extension, so the
# router's wave-cooperative extension runs)
@pytest.mark.parametrize("T", configs.SWEEP_T + (65536,))
def test_sweep_point_whole_step(orc, T):
    cfg = configs.sweep(T)
    say("[sweep] %s" % cfg.name)
    t = torch()
    inp, d = small_inputs(cfg)
    cos, sin = binding.device_rope(cfg)
    cb = t.from_numpy(inp["codebooks"]).cuda()
    idx, sel, out = binding.routed_attention(cfg, d["q"], d["k"], d["v"], cos, sin, cb)
    t.cuda.synchronize()
    g_idx, g_sel, g_out = index_to_host(idx), host(sel), host(out)

    c, s = orc.rope_table(cfg.T, cfg.d)
    sh = orc.Shape.of(**cfg.shape_kw())
    o_idx = orc.build_index(sh, inp["k"], c, s, inp["codebooks"])
    bad = compare_index(cfg, g_idx, o_idx)
    assert g_idx["overflow"].sum() == 0, "the sweep's balanced configuration overflowed"
    # causality, ascending ids, bypass rows, and R slots filled on every
    # searched route (no eligible block overflowed)
    check_sel_invariants(cfg, g_sel, g_idx)

    ids = sample_routes(cfg, 20000, seed=T, must=[(0, 0), (0, cfg.Hq - 1)])
    o_sel, gaps = orc.route(sh, inp["q"], c, s, inp["codebooks"], o_idx, ids)
    n = compare_sel(cfg, g_sel, o_sel, gaps, bad, route_ids=ids)
    keep = ~(g_sel.reshape(-1, cfg.R)[ids] != o_sel).any(-1)
    ref = orc.attention(sh, inp["q"], inp["k"], inp["v"], c, s, o_sel[keep], ids[keep])
    e = check_attention(cfg, g_out, ref, ids[keep])
    say("  %d routes sampled, %d excused; max load %d; attention error %.3g"
        % (len(ids), n, g_idx["load"].max(), e))
