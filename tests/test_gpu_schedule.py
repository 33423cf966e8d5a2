"""GPU parity of the V4.1 CSA2 layer schedule ("DeepSeek-V4.1 架构解析" §02): three encoder groups
of a Full layer and five Reuse layers, then the decoder group (a Full layer
that builds the block pool, three Reuse layers, and four times a Reindex
layer and three Reuse layers), every group with its own global KV and every
layer with its own window, one decode step through all 38 layers.

Every group is checked against the oracle with the rules of the layer tests:
all queries of a small schedule, sampled queries of the 1M-context, batch-32
schedule the benchmark times.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from compressed_sparse_attention_04_amd.step import from_schedule
from helpers import OracleStep, check_queries, np_

pytestmark = pytest.mark.gpu


def run_schedule(cfgs):
    wls = [W.make_workload(c, device="cuda") for c in cfgs]
    sch = from_schedule(wls)
    sch.setup()
    sch.step()
    torch.cuda.synchronize()
    return wls, sch


def test_v41_schedule_small_all_queries():
    cfgs = W.v41_schedule("decode", n_seq=2, ctx_tokens=4 * 3000 + 4, cid=210)
    wls, sch = run_schedule(cfgs)
    assert sum(len(c.layers) for c in cfgs) == 38
    for wl, st in zip(wls, sch.groups):
        r = check_queries(wl, st, range(wl.cfg.n_queries))
        n_out = wl.cfg.n_queries * len(wl.cfg.layers)
        assert r["swaps"] <= 1 and r["compared"] == n_out, (wl.cfg.name, r)
    # every layer's own window ring, bit-exact
    for wl, st in zip(wls, sch.groups):
        ref = OracleStep(wl)
        for s in range(wl.cfg.n_seq):
            p = int(wl.tensors["q_pos"][s])
            rows = oracle.window_positions(p) % st.win_cap
            for li in range(len(wl.cfg.layers)):
                assert np.array_equal(np_(st.wins[li][s])[rows], ref.window(s, p, li)), (wl.cfg.name, s, li)


def test_v41_schedule_layers_differ():
    """Layers with their own windows and queries give different outputs (no
    buffer is shared by mistake), and Reuse layers keep their group's indices."""
    cfgs = W.v41_schedule("decode", n_seq=1, ctx_tokens=4 * 1500, cid=230)
    wls, sch = run_schedule(cfgs)
    dec = sch.groups[3]
    outs = [np_(o) for o in dec.outs]
    for a in range(len(outs)):
        for b in range(a + 1, len(outs)):
            assert not np.array_equal(outs[a], outs[b]), (a, b)
    modes = wls[3].cfg.layers
    for li, m in enumerate(modes):
        if m == "U":
            src = max(j for j in range(li) if modes[j] in ("F", "I"))
            assert dec.idxs[li] is dec.idxs[src]


def test_v41_schedule_1m_decode_sampled():
    """The 1M-context, batch-32 schedule: every query's pool and Top-K in each
    group, attention on 16 sampled queries (every layer) per group."""
    name = "decode_b32_1m_v41_38layers"
    cfgs = W.v41_schedule(**W.SCHEDULES[name])
    wls, sch = run_schedule(cfgs)
    for g, (wl, st) in enumerate(zip(wls, sch.groups)):
        qa = sorted(np.random.default_rng(g).choice(wl.cfg.n_queries, 16, replace=False).tolist())
        r = check_queries(wl, st, range(wl.cfg.n_queries), attn_queries=qa)
        print(f"[parity] {wl.cfg.name}: {r}", flush=True)
        n_sel = wl.cfg.n_queries * sum(m in ("F", "I") for m in wl.cfg.layers)
        assert r["swaps"] <= max(1, n_sel // 50) and r["compared"] == 16 * len(wl.cfg.layers), (wl.cfg.name, r)
    del sch, wls
    torch.cuda.empty_cache()
