"""GPU parity of the Full-layer entry point at non-default Top-K and pool
sizes, and of the kernels at the extremes of their size range.

Top-K 64 / 512 / 1024 / 2048 / 4096 and pools of 1,024 to 4,096 blocks (the
largest the entry point accepts): Top-K up to 1,024 with a pool at least that
large goes through the selection that rescores the best blocks, larger Top-K
through the pool + Top-K kernel over written scores (rows of more than 32,768
blocks take its chunked path, covered by the layer tests).  Keys with one
value, or a few distinct rows, make every block max tie, which exercises the
lower-id rule across the block and entry selections.  The compression chain
runs with RoPE on 0, 64 and 512 channels.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import formats, mxfp4
from compressed_sparse_attention_04_amd import ops
from helpers import check_attn, check_topk_set, np_, SM

pytestmark = pytest.mark.gpu
DEV = "cuda"


def t_(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _full_layer(n_ent, top_k, n_pool, build_pool, keys="normal"):
    rng = np.random.default_rng(n_ent + top_k + n_pool)
    n_seq, win_cap = 2, 128
    codes = rng.integers(0, 256, (n_seq, n_ent, 256)).astype(np.uint8)
    scales = rng.integers(0x28, 0x31, (n_seq, n_ent, 32)).astype(np.uint8)
    if keys == "normal":
        k8 = formats.e4m3_encode(rng.standard_normal((n_seq, n_ent, 128)))
    elif keys == "const":
        k8 = np.broadcast_to(formats.e4m3_encode(rng.standard_normal((n_seq, 1, 128))), (n_seq, n_ent, 128))
    else:   # a few distinct rows
        rows = formats.e4m3_encode(rng.standard_normal((n_seq, 4, 128)))
        k8 = rows[np.arange(n_seq)[:, None], rng.integers(0, 4, (n_seq, n_ent))]
    k8 = np.ascontiguousarray(k8)
    q8 = formats.e4m3_encode(rng.standard_normal((n_seq, 8, 128)))
    w = rng.random((n_seq, 8)).astype(np.float32)
    q_attn = rng.standard_normal((n_seq, 16, 512)).astype(np.float32)
    win = formats.e4m3_encode(rng.standard_normal((n_seq, win_cap, 512)))
    pos = np.array([4 * n_ent - 1 - 40 * s for s in range(n_seq)], np.int32)    # second row: a partial block
    idx = torch.empty((n_seq, top_k), dtype=torch.int32, device=DEV)
    out = torch.empty((n_seq, 16, 512), dtype=torch.float32, device=DEV)
    pool = torch.empty((n_seq, n_pool), dtype=torch.int32, device=DEV) if build_pool else None
    call = ops.LayerCall(ops.MODE_FULL, codes=t_(codes), scales=t_(scales), k_fp8=t_(k8), win=t_(win),
                         q_pos=t_(pos), q_attn=t_(q_attn), idx=idx, out=out, n_seq=n_seq, q_per_seq=1,
                         n_entries=n_ent, q_idx=t_(q8), w_idx=t_(w), pool_blocks=pool, build_pool=build_pool,
                         top_k=top_k, n_pool_blocks=n_pool)
    call()
    torch.cuda.synchronize()
    gi, go = np_(idx), np_(out)
    for s in range(n_seq):
        wp = oracle.window_positions(pos[s])
        ref = oracle.layer_full(codes[s], scales[s], k8[s], q8[s], w[s], q_attn[s], pos[s], win[s, wp % win_cap], SM,
                                build_pool=build_pool, k=top_k, n_blocks=n_pool, n_entries=n_ent)
        if build_pool:
            assert np.array_equal(np_(pool)[s], ref.pool)
        if check_topk_set(gi[s], ref.scores, ref.idx, top_k) == 0:
            assert np.array_equal(np.sort(gi[s]), np.sort(ref.idx))
        # attention on the GPU's own selection (a near-tie swap is allowed above)
        check_attn(go[s], oracle.sparse_attention(q_attn[s], codes[s], scales[s], gi[s], win[s, wp % win_cap], SM))


@pytest.mark.parametrize("n_ent,top_k,n_pool,build_pool", [(20000, 2048, 4096, True), (45000, 512, 4096, True),
                                                           (20000, 64, 2048, True), (3000, 4096, 2048, False),
                                                           (40000, 2048, 2048, False), (45000, 1024, 4096, True),
                                                           (45000, 512, 1024, False)])
def test_full_layer_sizes(n_ent, top_k, n_pool, build_pool):
    _full_layer(n_ent, top_k, n_pool, build_pool)


# A decode-sized batch with more than 2^22 scores (2 sequences x 64 queries x
# 45,000 entries): the Full layer's selection runs split -- the pool and the
# best blocks selected by two blocks per query (one without a pool), the
# chosen blocks rescored by several blocks per query and the Top-K taken by
# the block that draws the query's last ticket.  Every query: pool
# bit-exact, Top-K set, attention on the GPU's own selection.
@pytest.mark.parametrize("keys,build_pool", [("normal", True), ("few", True), ("normal", False)])
def test_full_layer_split_selection(keys, build_pool):
    n_seq, qps, n_ent, top_k = 2, 64, 45000, 512
    n_pool = 2048 if build_pool else top_k
    Q, win_cap = n_seq * qps, 128 + qps
    rng = np.random.default_rng(4242 + len(keys))
    codes = rng.integers(0, 256, (n_seq, n_ent, 256)).astype(np.uint8)
    scales = rng.integers(0x28, 0x31, (n_seq, n_ent, 32)).astype(np.uint8)
    if keys == "normal":
        k8 = formats.e4m3_encode(rng.standard_normal((n_seq, n_ent, 128)))
    else:   # a few distinct rows: block maxima tie everywhere
        rows = formats.e4m3_encode(rng.standard_normal((n_seq, 4, 128)))
        k8 = np.ascontiguousarray(rows[np.arange(n_seq)[:, None], rng.integers(0, 4, (n_seq, n_ent))])
    q8 = formats.e4m3_encode(rng.standard_normal((Q, 8, 128)))
    w = rng.random((Q, 8)).astype(np.float32)
    q_attn = rng.standard_normal((Q, 16, 512)).astype(np.float32)
    win = formats.e4m3_encode(rng.standard_normal((n_seq, win_cap, 512)))
    pos = np.array([4 * n_ent - qps + (i % qps) for i in range(Q)], np.int32)
    idx = torch.empty((Q, top_k), dtype=torch.int32, device=DEV)
    out = torch.empty((Q, 16, 512), dtype=torch.float32, device=DEV)
    pool = torch.empty((Q, n_pool), dtype=torch.int32, device=DEV) if build_pool else None
    call = ops.LayerCall(ops.MODE_FULL, codes=t_(codes), scales=t_(scales), k_fp8=t_(k8), win=t_(win),
                         q_pos=t_(pos), q_attn=t_(q_attn), idx=idx, out=out, n_seq=n_seq, q_per_seq=qps,
                         n_entries=n_ent, q_idx=t_(q8), w_idx=t_(w), pool_blocks=pool, build_pool=build_pool,
                         top_k=top_k, n_pool_blocks=n_pool)
    call()
    torch.cuda.synchronize()
    gi, go = np_(idx), np_(out)
    gp = np_(pool) if build_pool else None
    kv = [formats.e4m3_decode(k8[s]) for s in range(n_seq)]
    for qi in range(Q):
        s = qi // qps
        wp = oracle.window_positions(pos[qi])
        ref = oracle.layer_full(codes[s], scales[s], k8[s], q8[qi], w[qi], q_attn[qi], pos[qi],
                                win[s, wp % win_cap], SM, build_pool=build_pool, k=top_k, n_blocks=n_pool,
                                n_entries=n_ent, k_values=kv[s], attend=False)
        if build_pool:
            assert np.array_equal(gp[qi], ref.pool), qi
        if check_topk_set(gi[qi], ref.scores, ref.idx, top_k) == 0:
            assert np.array_equal(np.sort(gi[qi]), np.sort(ref.idx)), qi
        if qi % 8 == 0:
            check_attn(go[qi], oracle.sparse_attention(q_attn[qi], codes[s], scales[s], gi[qi],
                                                       win[s, wp % win_cap], SM))


@pytest.mark.parametrize("n_ent,top_k,n_pool,build_pool,keys", [(3000, 1024, 1024, True, "const"),
                                                                (45000, 512, 2048, True, "few"),
                                                                (45000, 512, 2048, True, "const"),
                                                                (45000, 512, 1024, False, "const"),
                                                                (20000, 2048, 2048, False, "few")])
def test_full_layer_ties(n_ent, top_k, n_pool, build_pool, keys):
    _full_layer(n_ent, top_k, n_pool, build_pool, keys)


@pytest.mark.parametrize("Q,ncols,k", [(2, 100000, 1), (1, 100000, 4096), (3, 7, 4096), (1100, 5000, 512),
                                       (1030, 16384, 512),     # 1,024+ rows: the many-rows block shape
                                       (2, 100000, 16384), (1, 20000, 16384), (2, 40000, 9000)])   # up to CSA_MAX_K
def test_topk_extreme_k(Q, ncols, k):
    rng = np.random.default_rng(ncols + k)
    sc = rng.standard_normal((Q, ncols)).astype(np.float32)
    sc[:, ::11] = -np.inf
    idx = ops.csa_topk(t_(sc), k=k)
    torch.cuda.synchronize()
    got = np_(idx)
    for q in range(Q):
        valid = ~np.isneginf(sc[q])
        ref = oracle.topk(sc[q][valid].astype(np.float64), k, ids=np.arange(ncols)[valid])
        assert np.array_equal(got[q], ref), q


@pytest.mark.parametrize("k", [1, 4096])
def test_sparse_attn_extreme_k(k):
    rng = np.random.default_rng(k)
    n_seq, rows, win_cap = 2, 6000, 128
    codes = rng.integers(0, 256, (n_seq, rows, 256)).astype(np.uint8)
    scales = rng.integers(0x28, 0x31, (n_seq, rows, 32)).astype(np.uint8)
    win = formats.e4m3_encode(rng.standard_normal((n_seq, win_cap, 512)))
    q = rng.standard_normal((n_seq, 16, 512)).astype(np.float32)
    idx = np.stack([np.sort(rng.choice(rows, k, replace=False)) for _ in range(n_seq)]).astype(np.int32)
    pos = np.array([9000, 70], np.int32)
    out = ops.csa_sparse_attn(t_(q), t_(pos), t_(codes), t_(scales), t_(idx), t_(win), n_seq, 1)
    torch.cuda.synchronize()
    for s in range(n_seq):
        wp = oracle.window_positions(pos[s])
        ref = oracle.sparse_attention(q[s], codes[s], scales[s], idx[s], win[s, wp % win_cap], SM)
        check_attn(np_(out)[s], ref)


@pytest.mark.parametrize("rope_dim,n_seq,n_per", [(0, 2, 5), (512, 1, 33), (64, 1, 300)])
def test_compress_quant_rope_widths(rope_dim, n_seq, n_per):
    rng = np.random.default_rng(rope_dim + n_per)
    x = rng.standard_normal((n_seq, 4 * n_per, 512)).astype(np.float32)
    w = (rng.standard_normal((4, 512, 512)) / np.sqrt(2048)).astype(np.float32)
    half = max(rope_dim // 2, 1)
    ang = rng.uniform(0, 100, (n_seq, n_per, half))
    cs = np.stack([np.cos(ang), np.sin(ang)], -1).astype(np.float32)
    codes = torch.zeros((n_seq, n_per, 256), dtype=torch.uint8, device=DEV)
    scales = torch.zeros((n_seq, n_per, 32), dtype=torch.uint8, device=DEV)
    e_out = torch.empty((n_seq * n_per, 512), dtype=torch.float32, device=DEV)
    ops.csa_compress_quant(t_(x), t_(w), t_(cs) if rope_dim else None, codes, scales, n_seq, n_per,
                           x_seq_stride=4 * n_per * 512, out_seq_stride=n_per, rope_dim=rope_dim, e_out=e_out)
    torch.cuda.synchronize()
    e_gpu = np_(e_out).reshape(n_seq, n_per, 512)
    for s in range(n_seq):
        e_ref32 = oracle.compress_rope_fp32(x[s], w, cs[s] if rope_dim else None, rope_dim, 1e-6)
        ulps = np.abs(e_gpu[s].view(np.int32).astype(np.int64) - e_ref32.view(np.int32).astype(np.int64))
        assert ulps.max() <= 1, ulps.max()
        c2, s2 = mxfp4.quantize(e_gpu[s])
        assert np.array_equal(np_(codes)[s], c2) and np.array_equal(np_(scales)[s], s2)


@pytest.mark.parametrize("n_ent,top_k,n_pool,keys", [(45000, 512, 2048, "normal"), (45000, 1024, 4096, "normal"),
                                                     (20000, 64, 1024, "normal"), (45000, 512, 2048, "const"),
                                                     (45000, 512, 2048, "few"), (20000, 2048, 2048, "normal"),
                                                     (20000, 1024, 512, "normal"), (3000, 512, 2048, "normal")])
def test_reindex_layer_sizes(n_ent, top_k, n_pool, keys):
    """Reindex inside a pool of 512 to 4,096 blocks with Top-K 64 to 2,048 (a
    pool smaller than Top-K included) and tie-heavy keys.  Pools hold random
    ascending blocks, -1 padded, with a partially visible last block; the
    selected ids come out ascending."""
    rng = np.random.default_rng(n_ent + 3 * top_k + n_pool)
    n_seq, win_cap = 2, 128
    codes = rng.integers(0, 256, (n_seq, n_ent, 256)).astype(np.uint8)
    scales = rng.integers(0x28, 0x31, (n_seq, n_ent, 32)).astype(np.uint8)
    if keys == "normal":
        k8 = formats.e4m3_encode(rng.standard_normal((n_seq, n_ent, 128)))
    elif keys == "const":
        k8 = np.broadcast_to(formats.e4m3_encode(rng.standard_normal((n_seq, 1, 128))), (n_seq, n_ent, 128))
    else:
        rows = formats.e4m3_encode(rng.standard_normal((n_seq, 4, 128)))
        k8 = rows[np.arange(n_seq)[:, None], rng.integers(0, 4, (n_seq, n_ent))]
    k8 = np.ascontiguousarray(k8)
    q8 = formats.e4m3_encode(rng.standard_normal((n_seq, 8, 128)))
    w = rng.random((n_seq, 8)).astype(np.float32)
    q_attn = rng.standard_normal((n_seq, 16, 512)).astype(np.float32)
    win = formats.e4m3_encode(rng.standard_normal((n_seq, win_cap, 512)))
    pos = np.array([4 * n_ent - 1 - 40 * s for s in range(n_seq)], np.int32)
    n_blk = (n_ent + 7) // 8
    pool = np.full((n_seq, n_pool), -1, np.int32)
    for s in range(n_seq):
        m = min(n_pool - 5, n_blk) if n_pool > 5 else n_pool
        b = np.sort(rng.choice(n_blk, m, replace=False))
        b[-1] = n_blk - 1
        b = np.unique(b)
        pool[s, :len(b)] = b
    idx = torch.empty((n_seq, top_k), dtype=torch.int32, device=DEV)
    out = torch.empty((n_seq, 16, 512), dtype=torch.float32, device=DEV)
    call = ops.LayerCall(ops.MODE_REINDEX, codes=t_(codes), scales=t_(scales), k_fp8=t_(k8), win=t_(win),
                         q_pos=t_(pos), q_attn=t_(q_attn), idx=idx, out=out, n_seq=n_seq, q_per_seq=1,
                         n_entries=n_ent, q_idx=t_(q8), w_idx=t_(w), pool_blocks=t_(pool), top_k=top_k,
                         n_pool_blocks=n_pool)
    call()
    torch.cuda.synchronize()
    gi, go = np_(idx), np_(out)
    for s in range(n_seq):
        wp = oracle.window_positions(pos[s])
        ref = oracle.layer_reindex(codes[s], scales[s], k8[s], pool[s], q8[s], w[s], q_attn[s], pos[s],
                                   win[s, wp % win_cap], SM, k=top_k, n_entries=n_ent)
        nv = oracle.visible_entries(pos[s], n_ent)
        ids = oracle.pooled_entries(pool[s], nv)
        if check_topk_set(gi[s], ref.scores, ref.idx, top_k, ids=ids) == 0:
            assert np.array_equal(np.sort(gi[s]), np.sort(ref.idx))
        assert np.array_equal(gi[s][gi[s] >= 0], np.sort(gi[s][gi[s] >= 0]))   # ascending ids
        check_attn(go[s], oracle.sparse_attention(q_attn[s], codes[s], scales[s], gi[s], win[s, wp % win_cap], SM))
