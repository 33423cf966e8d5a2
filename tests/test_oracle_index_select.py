"""Pins of the oracle's indexer scores, Top-K and hierarchical pool.

Pinned against: exact rational arithmetic (Python fractions) on torch-decoded
E4M3 bytes; the textbook one-hot case; Python's sorted() on (score, id) keys;
exhaustive pairwise order checks on tiny inputs; the page's pool constants; and
the pool-contains-Top-K property (page: Reindex layers search only inside the
pool, which is useful only if the pool holds the Full layer's Top-K).
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import indexer, select
from oracle.layer import layer_full, layer_reindex

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
PAGE = json.load(open(os.path.join(GOLDEN, "page_constants.json")))


def e4m3_bytes(rng, shape):
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32))
    return x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def torch_decode(b):
    return torch.from_numpy(np.ascontiguousarray(b)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_visibility_rule():
    assert [indexer.visible_entries(p) for p in range(0, 12)] == [0, 0, 0, 1, 1, 1, 1, 2, 2, 2, 2, 3]
    assert indexer.visible_entries(131071) == 32768
    assert indexer.visible_entries(10 ** 6, n_entries=5) == 5


def test_scores_exact_against_fractions():
    rng = np.random.default_rng(0)
    q = e4m3_bytes(rng, (8, 128))
    k = e4m3_bytes(rng, (12, 128))
    w = rng.random(8).astype(np.float32)
    got = indexer.index_scores(q, w, k)
    qd, kd = torch_decode(q), torch_decode(k)
    for j in range(12):
        tot = Fraction(0)
        for h in range(8):
            dot = sum(Fraction(float(qd[h, d])) * Fraction(float(kd[j, d])) for d in range(128))
            if dot > 0:
                tot += Fraction(float(w[h])) * dot
        assert abs(Fraction(float(got[j])) - tot) <= abs(tot) * Fraction(1, 2 ** 50)
    assert np.all(got >= 0)


def test_one_hot_weight_is_single_relu_dot():
    rng = np.random.default_rng(1)
    q = e4m3_bytes(rng, (8, 128))
    k = e4m3_bytes(rng, (50, 128))
    w = np.zeros(8, dtype=np.float32)
    w[5] = 1.0
    ref = torch.relu(torch.from_numpy(torch_decode(k)) @ torch.from_numpy(torch_decode(q[5])))
    np.testing.assert_array_equal(indexer.index_scores(q, w, k), ref.numpy())


def test_topk_matches_sorted_with_ties():
    rng = np.random.default_rng(2)
    for trial in range(50):
        n = int(rng.integers(1, 300))
        k = int(rng.integers(1, 40))
        s = rng.integers(0, 6, n).astype(np.float64)       # heavy ties
        ref = sorted(range(n), key=lambda j: (-s[j], j))[:k]
        got = select.topk(s, k)
        assert list(got[: len(ref)]) == sorted(ref)
        assert np.all(got[len(ref):] == -1)


def test_topk_order_property_exhaustive():
    rng = np.random.default_rng(3)
    s = rng.integers(0, 4, 40).astype(np.float64)
    got = set(select.topk(s, 9).tolist())
    for a in got:
        for b in set(range(40)) - got:
            assert (s[a] > s[b]) or (s[a] == s[b] and a < b)


def test_block_pool_brute_force():
    rng = np.random.default_rng(4)
    s = rng.integers(0, 5, 83).astype(np.float64)          # partial last block
    bm = [max(s[8 * b: 8 * b + 8]) for b in range(11)]
    ref = sorted(range(11), key=lambda b: (-bm[b], b))[:4]
    assert list(select.block_pool(s, n_blocks=4)) == sorted(ref)
    assert list(select.block_pool(s, n_blocks=20)) == list(range(11)) + [-1] * 9


@pytest.mark.parametrize("n,k,nb", [(64, 2, 2), (200, 5, 5), (1000, 16, 16), (5000, 40, 64)])
def test_pool_contains_topk_small(n, k, nb):
    rng = np.random.default_rng(n)
    for trial in range(300):
        s = rng.integers(0, int(rng.integers(2, 12)), n).astype(np.float64)
        top = set(select.topk(s, k).tolist()) - {-1}
        pool = select.block_pool(s, n_blocks=nb)
        members = {8 * b + i for b in pool if b >= 0 for i in range(8)}
        assert top <= members


def test_pool_contains_top512_page_sizes():
    """The page's sizes: Top-512 inside 2,048 blocks x 8 = 16,384 candidates."""
    assert PAGE["pool_blocks"] * PAGE["block"] == PAGE["pool_size"]
    rng = np.random.default_rng(5)
    for trial in range(6):
        n = 32768 + int(rng.integers(0, 8))
        s = rng.integers(0, 50, n).astype(np.float64)
        top = select.topk(s, PAGE["top_k"])
        pool = select.block_pool(s, PAGE["pool_blocks"], PAGE["block"])
        ent = indexer.pooled_entries(pool, n)
        assert len(ent) <= PAGE["pool_size"]
        assert set(top.tolist()) <= set(ent.tolist())


def test_reindex_with_full_query_reproduces_full_topk():
    """Corollary of pool >= Top-K: rescoring the pool with the Full layer's own
    indexer query selects exactly the Full layer's Top-K."""
    rng = np.random.default_rng(6)
    n = 3000
    k_fp8 = e4m3_bytes(rng, (n, 128))
    q = e4m3_bytes(rng, (8, 128))
    w = rng.random(8).astype(np.float32)
    codes = rng.integers(0, 256, (n, 256)).astype(np.uint8)
    scales = rng.integers(0x28, 0x31, (n, 32)).astype(np.uint8)
    qa = rng.standard_normal((16, 512)).astype(np.float32)
    win = e4m3_bytes(rng, (128, 512))
    p = 4 * n - 1
    full = layer_full(codes, scales, k_fp8, q, w, qa, p, win, 512 ** -0.5,
                      build_pool=True, k=64, n_blocks=64)
    re = layer_reindex(codes, scales, k_fp8, full.pool, q, w, qa, p, win, 512 ** -0.5, k=64)
    assert np.array_equal(full.idx, re.idx)
    np.testing.assert_array_equal(full.out, re.out)


def test_pooled_entries_partial_last_block():
    """Hand-enumerated candidates of a pool whose blocks end at, inside and
    past the visible prefix: a prefill query that sees 43 entries sees
    entries 40..42 of block 5 and nothing of blocks 6 and up; -1 slots are
    empty (the pool holds 8-entry blocks; a query sees only entries whose
    last token precedes it)."""
    got = indexer.pooled_entries(np.array([0, 3, 5, 6, 11, -1, -1]), 43)
    want = list(range(0, 8)) + list(range(24, 32)) + [40, 41, 42]
    assert got.tolist() == want
    assert indexer.pooled_entries(np.array([2, 9]), 20).tolist() == [16, 17, 18, 19]
    assert indexer.pooled_entries(np.array([5]), 40).tolist() == []       # block 5 starts at the prefix end
    assert indexer.pooled_entries(np.array([5]), 41).tolist() == [40]
    assert indexer.pooled_entries(np.array([4]), 40).tolist() == list(range(32, 40))
    assert indexer.pooled_entries(np.array([-1, -1]), 100).tolist() == []


def test_reindex_never_scores_invisible_pool_entries():
    """A prefill query whose visible prefix ends inside a pool block: the
    Reindex candidates stop at the prefix, so with K above the candidate
    count the selection is exactly the visible pool entries, and the scores
    are those of the visible entries only."""
    rng = np.random.default_rng(12)
    n = 200
    k_fp8 = e4m3_bytes(rng, (n, 128))
    q = e4m3_bytes(rng, (8, 128))
    w = rng.random(8).astype(np.float32)
    codes = rng.integers(0, 256, (n, 256)).astype(np.uint8)
    scales = rng.integers(0x28, 0x31, (n, 32)).astype(np.uint8)
    qa = rng.standard_normal((16, 512)).astype(np.float32)
    win = e4m3_bytes(rng, (128, 512))
    p = 4 * 45 + 2                       # sees entries 0..44 (45 entries): block 5 holds 40..44
    pool = np.array([1, 5, 7, 20, -1])   # block 7 and 20 lie past the prefix
    re = layer_reindex(codes, scales, k_fp8, pool, q, w, qa, p, win, 512 ** -0.5, k=64)
    want = list(range(8, 16)) + [40, 41, 42, 43, 44]
    assert re.idx[:len(want)].tolist() == want and np.all(re.idx[len(want):] == -1)
    assert len(re.scores) == len(want)
    np.testing.assert_array_equal(re.scores, indexer.index_scores(q, w, k_fp8[want]))


def test_index_scores_many_equals_one_query_at_a_time():
    """The batched scoring of a chunk's queries (shared keys) gives each
    query's index_scores up to the order of the final 8-term sum."""
    rng = np.random.default_rng(13)
    k_fp8 = e4m3_bytes(rng, (300, 128))
    q = e4m3_bytes(rng, (5, 8, 128))
    w = rng.random((5, 8)).astype(np.float32)
    many = indexer.index_scores_many(q, w, torch_decode(k_fp8))
    for i in range(5):
        one = indexer.index_scores(q[i], w[i], k_fp8)
        np.testing.assert_allclose(many[i], one, rtol=1e-15, atol=0)
        np.testing.assert_array_equal(indexer.index_scores(q[i], w[i], k_fp8, k_values=torch_decode(k_fp8)), one)
