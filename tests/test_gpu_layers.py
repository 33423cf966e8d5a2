"""GPU parity of whole layer steps (window append, compress + quantize, Full /
Reindex / Reuse layers) against the oracle on the same seeded workloads.

Small workloads are checked on every query; the full-size workloads (the
launch configuration the benchmark times) on sampled queries.  Top-K sets
follow the near-tie rule; attention outputs are compared for every query whose
selected set matches the oracle's exactly (a near-tie swap makes both outputs
correct, so such queries are counted, not compared).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from compressed_sparse_attention_04_amd.step import from_workload
from helpers import OracleStep, check_queries, np_

pytestmark = pytest.mark.gpu


def run_step(cfg):
    wl = W.make_workload(cfg, device="cuda")
    st = from_workload(wl)
    st.setup()
    st.step()
    torch.cuda.synchronize()
    return wl, st


SMALL = [
    W.small_config("decode", n_seq=3, ctx_tokens=4 * 3000, layers=("F", "U", "U"), cid=101),
    W.small_config("decode", n_seq=2, ctx_tokens=4 * 20003 + 4, layers=("F", "I", "I"), build_pool=True,
                   synthetic_cache=True, cid=102),
    W.small_config("prefill", n_seq=1, ctx_tokens=4 * 2000, chunk=192, layers=("F", "U", "I", "U"),
                   build_pool=True, cid=103),
    W.small_config("prefill", n_seq=1, ctx_tokens=4 * 300, chunk=100, layers=("F", "U"), cid=104),
    W.small_config("decode", n_seq=2, ctx_tokens=4 * 100, layers=("F", "U"), cid=105),   # < K entries
    # 33,000 blocks per row: more than one selection block holds, so the pool
    # and the Top-K take the chunked path
    W.small_config("decode", n_seq=1, ctx_tokens=4 * 8 * 33000, layers=("F", "I"), build_pool=True,
                   synthetic_cache=True, cid=106),
    W.small_config("decode", n_seq=1, ctx_tokens=4 * 8 * 33000, layers=("F", "U"), synthetic_cache=True,
                   cid=107),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: f"{c.name}_{c.cid}")
def test_small_steps_all_queries(cfg):
    wl, st = run_step(cfg)
    swaps, compared, skips = check_queries(wl, st, range(cfg.n_queries))
    n_out = cfg.n_queries * len(cfg.layers)
    assert swaps <= max(1, cfg.n_queries // 50), swaps
    assert compared >= n_out // 2, (compared, skips, n_out)


def test_prefill_512_queries_pool_sampled():
    """512 queries (from this many on, the Full-layer selection runs in
    512-thread blocks, two per compute unit) over 20,000 entries: the pool
    selects 2,048 of 2,500 blocks and a Reindex layer rescores inside it;
    every fourth query and the last are checked."""
    cfg = W.small_config("prefill", n_seq=1, ctx_tokens=4 * 20000, chunk=512, layers=("F", "I"),
                         build_pool=True, synthetic_cache=True, cid=108)
    assert cfg.n_queries == 512
    wl, st = run_step(cfg)
    qs = list(range(0, cfg.n_queries, 4)) + [cfg.n_queries - 1]
    swaps, compared, skips = check_queries(wl, st, qs)
    assert swaps <= max(1, len(qs) // 50) and compared >= len(qs), (swaps, compared, skips)


def test_window_and_new_entries_bit_exact():
    """The step's window rows and compressed entries versus the oracle's, at the
    decode workload with 1,024 entries (the 4K-context decode)."""
    cfg = W.CONFIGS[0]
    wl, st = run_step(cfg)
    ref = OracleStep(wl)
    codes, scales, _, x_tail = ref.cache(0)
    p = int(wl.tensors["q_pos"][0])
    win_ref = ref.window(0, p)
    win = np_(st.win[0])
    rows = oracle.window_positions(p) % st.win_cap
    assert np.array_equal(win[rows], win_ref)
    gc, gs = np_(st.codes[0]), np_(st.scales[0])
    # the GPU chain reproduces the oracle's fp32 quantizer input, so every byte agrees
    assert np.array_equal(gc, codes) and np.array_equal(gs, scales)


def test_decode_4k_full_layer():
    cfg = W.CONFIGS[0]
    wl, st = run_step(cfg)
    swaps, compared, skips = check_queries(wl, st, [0])
    assert compared + skips == 1 or swaps == 1


def test_prefill_2048_at_32k_sampled():
    cfg = W.CONFIGS[1]
    wl, st = run_step(cfg)
    qs = list(range(0, cfg.n_queries, 64)) + [cfg.n_queries - 1]
    swaps, compared, skips = check_queries(wl, st, qs)
    assert swaps <= 2 and compared >= len(qs) // 2, (swaps, compared, skips)


@pytest.mark.parametrize("cid,queries", [(2, [0, 37, 63]), (3, [0, 31]), (4, [0, 1, 2047, 4095])])
def test_full_size_workloads_sampled(cid, queries):
    cfg = W.CONFIGS[cid]
    wl, st = run_step(cfg)
    swaps, compared, skips = check_queries(wl, st, queries)
    assert swaps <= 1 and compared >= 1, (swaps, compared, skips)
    del st, wl
    torch.cuda.empty_cache()
