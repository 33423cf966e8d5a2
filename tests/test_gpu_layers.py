"""GPU parity of whole layer steps (window append, compress + quantize, Full /
Reindex / Reuse layers) against the oracle on the same seeded workloads.

Small workloads are checked on every query.  The full-size workloads (the
launch configuration the benchmark times) check the pool and every Full /
Reindex Top-K set on every query, and attention on every query of the decode
batches and on 256 sampled queries per layer of the prefill chunks.  Top-K
sets follow the near-tie rule; every attention output is compared, with the
oracle run on the GPU's own selected ids and cache bytes (so a near-tie swap
does not compound into the attention tolerance).
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


def _report(name, r):
    print(f"[parity] {name}: {r}", flush=True)


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: f"{c.name}_{c.cid}")
def test_small_steps_all_queries(cfg):
    wl, st = run_step(cfg)
    r = check_queries(wl, st, range(cfg.n_queries))
    _report(cfg.name, r)
    n_out = cfg.n_queries * len(cfg.layers)
    n_sel = cfg.n_queries * sum(m in ("F", "I") for m in cfg.layers)
    assert r["swaps"] <= max(1, n_sel // 50), r
    assert r["compared"] == r["outputs"] == n_out, r


def test_prefill_512_queries_pool_sampled():
    """512 queries (from this many on, the Full-layer selection runs in
    512-thread blocks, two per compute unit) over 20,000 entries: the pool
    selects 2,048 of 2,500 blocks and a Reindex layer rescores inside it;
    every query's selection and every fourth query's attention are checked."""
    cfg = W.small_config("prefill", n_seq=1, ctx_tokens=4 * 20000, chunk=512, layers=("F", "I"),
                         build_pool=True, synthetic_cache=True, cid=108)
    assert cfg.n_queries == 512
    wl, st = run_step(cfg)
    qa = list(range(0, cfg.n_queries, 4)) + [cfg.n_queries - 1]
    r = check_queries(wl, st, range(cfg.n_queries), attn_queries=qa)
    _report(cfg.name, r)
    assert r["swaps"] <= max(1, 2 * cfg.n_queries // 50), r
    assert r["compared"] == len(qa) * 2, r


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
    r = check_queries(wl, st, [0])
    _report(cfg.name, r)
    assert r["compared"] == 1 and r["swaps"] + r["exact_sets"] == 1, r


def _sampled(n, k, seed):
    rng = np.random.default_rng(seed)
    return sorted(set([0, n - 1] + rng.choice(n, k, replace=False).tolist()))


def test_prefill_2048_at_32k():
    """Every query's Top-K; attention on 256 sampled queries."""
    cfg = W.CONFIGS[1]
    wl, st = run_step(cfg)
    qa = _sampled(cfg.n_queries, 256, 1)
    r = check_queries(wl, st, range(cfg.n_queries), attn_queries=qa)
    _report(cfg.name, r)
    assert r["swaps"] <= cfg.n_queries // 50 and r["compared"] == len(qa), r


# Decode batches: every query, every layer (selection and attention).
# The 256K prefill: every query's pool and Full / Reindex Top-K, attention on
# 256 sampled queries in each of its five layers.
@pytest.mark.parametrize("cid", [2, 3, 4])
def test_full_size_workloads(cid):
    cfg = W.CONFIGS[cid]
    wl, st = run_step(cfg)
    qa = None if cfg.kind == "decode" else _sampled(cfg.n_queries, 256, cid)
    r = check_queries(wl, st, range(cfg.n_queries), attn_queries=qa)
    _report(cfg.name, r)
    n_sel = cfg.n_queries * sum(m in ("F", "I") for m in cfg.layers)
    n_att = (cfg.n_queries if qa is None else len(qa)) * len(cfg.layers)
    assert r["swaps"] <= max(1, n_sel // 50), r
    assert r["compared"] == n_att, r
    del st, wl
    torch.cuda.empty_cache()
