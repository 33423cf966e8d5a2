"""A layer-group step captured in a HIP graph gives the eager step's results.

Before every replay the state the step writes (the window rings and the
stored entries) is put back as it was before the step, where the rows of the
step's tokens and entries are still empty: a replay that skipped or misordered
the window append or the compression would leave them empty.  Every replay
must reproduce the eager outputs bit for bit.  Eager work and a
synchronisation separate the replays.
"""

import pytest
import torch

import workloads as W
from compressed_sparse_attention_04_amd.step import from_schedule, from_workload

pytestmark = pytest.mark.gpu

CASES = [
    W.small_config("decode", n_seq=3, ctx_tokens=4 * 3000, layers=("F", "U", "I"), build_pool=True, cid=401),
    W.small_config("prefill", n_seq=1, ctx_tokens=4 * 2000, chunk=192, layers=("F", "U", "I"), build_pool=True,
                   cid=402),
]


def snapshot(st):
    outs = [o.clone() for o in st.outs]
    idxs = [i.clone() for i in st.idxs]
    rows = slice(st.prior, st.prior + st.new)
    return outs, idxs, st.codes[:, rows].clone(), st.scales[:, rows].clone(), st.win_all.clone()


def restore(st, pre):
    st.codes.copy_(pre[0])
    st.scales.copy_(pre[1])
    st.win_all.copy_(pre[2])
    for o in st.outs:
        o.zero_()


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_graph_replay_matches_eager(cfg):
    wl = W.make_workload(cfg, device="cuda")
    st = from_workload(wl)
    st.setup()
    rows = slice(st.prior, st.prior + st.new)
    st.codes[:, rows].zero_()
    st.scales[:, rows].zero_()
    torch.cuda.synchronize()
    pre = (st.codes.clone(), st.scales.clone(), st.win_all.clone())
    st.step()
    torch.cuda.synchronize()
    ref = snapshot(st)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.step()
    torch.cuda.synchronize()
    for rep in range(3):
        restore(st, pre)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot(st)
        for a, b in zip(ref[0], got[0]):
            assert torch.equal(a, b), (cfg.name, rep, "attention output")
        for a, b in zip(ref[1], got[1]):
            assert torch.equal(a, b), (cfg.name, rep, "indices")
        assert torch.equal(ref[2], got[2]) and torch.equal(ref[3], got[3]), (cfg.name, rep, "new entries")
        assert torch.equal(ref[4], got[4]), (cfg.name, rep, "window rings")
        _ = torch.randn(1 << 20, device="cuda").sum().item()     # eager work between replays
    del g
    torch.cuda.synchronize()


def test_graph_replay_schedule_matches_eager():
    """The 38-layer schedule (four groups, each with its own global KV and
    windows) captured as one graph: every replay from the pre-step state
    matches the eager step bit for bit."""
    cfgs = W.v41_schedule("decode", n_seq=2, ctx_tokens=4 * 1500, cid=420)
    wls = [W.make_workload(c, device="cuda") for c in cfgs]
    sch = from_schedule(wls)
    sch.setup()
    for st in sch.groups:
        rows = slice(st.prior, st.prior + st.new)
        st.codes[:, rows].zero_()
        st.scales[:, rows].zero_()
    torch.cuda.synchronize()
    pres = [(st.codes.clone(), st.scales.clone(), st.win_all.clone()) for st in sch.groups]
    sch.step()
    torch.cuda.synchronize()
    refs = [snapshot(st) for st in sch.groups]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sch.step()
    torch.cuda.synchronize()
    for rep in range(2):
        for st, pre in zip(sch.groups, pres):
            restore(st, pre)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for gi, (st, ref) in enumerate(zip(sch.groups, refs)):
            got = snapshot(st)
            assert all(torch.equal(a, b) for a, b in zip(ref[0], got[0])), (gi, rep, "attention output")
            assert all(torch.equal(a, b) for a, b in zip(ref[1], got[1])), (gi, rep, "indices")
            assert torch.equal(ref[4], got[4]), (gi, rep, "window rings")
    del g
    torch.cuda.synchronize()
