"""A layer-group step that compresses its new entries on a second stream
beside the first layer's scoring and selection (the prefill default) leaves the same
bytes as the same step run in order: every layer's output and ids, the pool,
the new cache rows and the window.  Checked eagerly and on several replays
of a captured HIP graph, with eager work and synchronisation between them."""

import pytest
import torch

import workloads as W
from compressed_sparse_attention_04_amd.step import from_workload

pytestmark = pytest.mark.gpu

CFGS = [
    W.small_config("decode", n_seq=3, ctx_tokens=4 * 3000, layers=("F", "U", "U"), cid=201),
    W.small_config("decode", n_seq=2, ctx_tokens=4 * 20003 + 4, layers=("F", "I", "I"), build_pool=True,
                   synthetic_cache=True, cid=202),
    W.small_config("prefill", n_seq=1, ctx_tokens=4 * 2000, chunk=192, layers=("F", "U", "I", "U"),
                   build_pool=True, cid=203),
]


def _state(st):
    out = {f"out{i}": o for i, o in enumerate(st.outs)}
    out.update({f"idx{i}": x for i, x in enumerate(st.idxs)})
    out.update(codes=st.codes, scales=st.scales, win=st.win_all)
    if st.pool is not None:
        out["pool"] = st.pool
    return {k: v.clone() for k, v in out.items()}


def _same(a, b, what):
    for k in a:
        assert torch.equal(a[k], b[k]), f"{what}: {k} differs"


@pytest.mark.parametrize("cfg", CFGS, ids=lambda c: f"{c.name}_{c.cid}")
def test_overlapped_compression_matches_in_order(cfg):
    print(f"[overlap] {cfg.name} {cfg.layers}", flush=True)
    ref_st = from_workload(W.make_workload(cfg, device="cuda"), overlap_compress=False)
    ref_st.setup()
    ref_st.step()
    torch.cuda.synchronize()
    ref = _state(ref_st)

    st = from_workload(W.make_workload(cfg, device="cuda"), overlap_compress=True)
    assert st.overlap
    st.setup()
    st.step()
    torch.cuda.synchronize()
    _same(ref, _state(st), "eager")

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.step()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in st.outs:
            o.fill_(float("nan"))   # eager work between replays; every output is rewritten
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(ref, _state(st), f"graph replay {rep}")
