"""GPU parity of each C-ABI entry point against the oracle, on seeded inputs.

Every test calls the HIP library through its C ABI (ctypes binding) and
compares with the float64 oracle under the method's rules (see helpers.py).
Sizes span several tiles / chunks and end in ragged tails.
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


def t_(a, dtype=None):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV) if dtype is None else \
        torch.from_numpy(np.ascontiguousarray(a)).to(DEV, dtype)


def quant_inputs(rng, n):
    """Entries with varied group magnitudes, zero groups, exact midpoints and saturation."""
    x = rng.standard_normal((n, 512)) * rng.choice([1e-4, 0.01, 1.0, 30.0, 5000.0], (n, 32, 1)).repeat(16, -1).reshape(n, 512)
    x = x.astype(np.float32)
    if n >= 4:
        x[0, :16] = 0.0
        x[1, :16] = -0.0
        # a group of exact E2M1 midpoints times an exact scale
        s = np.float32(0.3125)
        x[2, :16] = s * np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, -0.25, -0.75,
                                  -1.25, -1.75, -2.5, -3.5, -5.0, -6.0], np.float32)
        x[3, :16] = 2688.0 * np.sign(rng.standard_normal(16)).astype(np.float32)
        x[3, 16:32] = 1e30
    return x


@pytest.mark.parametrize("n", [0, 1, 5, 17, 1000])
def test_quantize_bit_exact(n):
    rng = np.random.default_rng(n)
    x = quant_inputs(rng, n)
    codes, scales = ops.csa_quantize(t_(x))
    torch.cuda.synchronize()
    if n == 0:
        return
    rc, rs = mxfp4.quantize(x)
    assert np.array_equal(np_(scales), rs)
    assert np.array_equal(np_(codes), rc)


def test_dequantize_exact():
    rng = np.random.default_rng(1)
    n = 300
    codes = rng.integers(0, 256, (n, 256)).astype(np.uint8)
    scales = rng.integers(0, 0x7F, (n, 32)).astype(np.uint8)        # every finite positive scale
    out = ops.csa_dequantize(t_(codes), t_(scales))
    torch.cuda.synchronize()
    ref = mxfp4.dequantize(codes, scales)
    assert np.array_equal(np_(out).astype(np.float64), ref)


@pytest.mark.parametrize("n_seq,n_tok,cap,p0", [(1, 1, 128, 0), (3, 200, 256, 50), (2, 130, 130, 1000)])
def test_window_append_bit_exact(n_seq, n_tok, cap, p0):
    rng = np.random.default_rng(n_tok)
    x = (rng.standard_normal((n_seq, n_tok, 512)) * rng.choice([1e-3, 1, 300], (n_seq, n_tok, 1))).astype(np.float32)
    x[0, 0, :4] = [500.0, -1e6, -0.0, 2.0 ** -10]
    pos0 = np.array([p0 + 7 * s for s in range(n_seq)], np.int32)
    win = torch.full((n_seq, cap, 512), 0xAB, dtype=torch.uint8, device=DEV)
    ops.csa_window_append(t_(x), t_(pos0), win, n_seq, n_tok)
    torch.cuda.synchronize()
    got = np_(win)
    for s in range(n_seq):
        # later tokens overwrite earlier ones that share a ring row
        expect = np.full((cap, 512), 0xAB, np.uint8)
        for t in range(n_tok):
            expect[(pos0[s] + t) % cap] = formats.e4m3_encode(x[s, t])
        assert np.array_equal(got[s], expect)


@pytest.mark.parametrize("n_per,n_tok", [(3, 1), (0, 2), (2, 0), (5, 130)])
def test_compress_quant_append_matches_separate_calls(n_per, n_tok):
    """csa_compress_quant_append writes the same bytes as csa_compress_quant
    followed by csa_window_append (either part may be empty)."""
    rng = np.random.default_rng(10 * n_per + n_tok)
    n_seq, rows, cap = 3, 12, 160
    x = rng.standard_normal((n_seq, 4 * max(n_per, 1), 512)).astype(np.float32)
    w = (rng.standard_normal((4, 512, 512)) / np.sqrt(2048)).astype(np.float32)
    ang = rng.uniform(0, 100, (n_seq, n_per, 32))
    cs = np.stack([np.cos(ang), np.sin(ang)], -1).astype(np.float32)
    xw = (rng.standard_normal((n_seq, max(n_tok, 1), 512)) * 3).astype(np.float32)
    pos0 = np.array([50 + 9 * s for s in range(n_seq)], np.int32)
    outs = []
    for fused in (False, True):
        codes = torch.full((n_seq, rows, 256), 0x5A, dtype=torch.uint8, device=DEV)
        scales = torch.full((n_seq, rows, 32), 0x5A, dtype=torch.uint8, device=DEV)
        win = torch.full((n_seq, cap, 512), 0xAB, dtype=torch.uint8, device=DEV)
        kw = dict(x_seq_stride=4 * max(n_per, 1) * 512, out_seq_stride=rows, out_offset=2)
        if fused:
            ops.csa_compress_quant_append(t_(x), t_(w), t_(cs), codes, scales, n_seq, n_per, t_(xw), t_(pos0), win,
                                          n_seq, n_tok, xw_seq_stride=max(n_tok, 1) * 512, **kw)
        else:
            ops.csa_compress_quant(t_(x), t_(w), t_(cs), codes, scales, n_seq, n_per, **kw)
            ops.csa_window_append(t_(xw), t_(pos0), win, n_seq, n_tok, x_seq_stride=max(n_tok, 1) * 512)
        torch.cuda.synchronize()
        outs.append((np_(codes), np_(scales), np_(win)))
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
    if n_per:
        assert (outs[1][0][:, 2:2 + n_per] != 0x5A).any()
    if n_tok:
        assert (outs[1][2] != 0xAB).any()


def test_compress_quant_chain():
    """The GPU chain (fp64 GEMM, RMSNorm, RoPE; one rounding to fp32) gives the
    fp32 rounding of the oracle's fp64 result, up to one fp32 ulp where the
    exact value sits on an fp32 rounding boundary; its bytes equal the oracle's
    quantization of the GPU's own fp32 input (strict), and of the oracle chain."""
    rng = np.random.default_rng(2)
    n_seq, n_per, rows = 3, 37, 50
    x = rng.standard_normal((n_seq, 4 * n_per, 512)).astype(np.float32)
    w = (rng.standard_normal((4, 512, 512)) / np.sqrt(2048)).astype(np.float32)
    ang = rng.uniform(0, 100, (n_seq, n_per, 32))
    cs = np.stack([np.cos(ang), np.sin(ang)], -1).astype(np.float32)
    codes = torch.zeros((n_seq, rows, 256), dtype=torch.uint8, device=DEV)
    scales = torch.zeros((n_seq, rows, 32), dtype=torch.uint8, device=DEV)
    e_out = torch.empty((n_seq * n_per, 512), dtype=torch.float32, device=DEV)
    ops.csa_compress_quant(t_(x), t_(w), t_(cs), codes, scales, n_seq, n_per,
                           x_seq_stride=4 * n_per * 512, out_seq_stride=rows, out_offset=5, e_out=e_out)
    torch.cuda.synchronize()
    e_gpu = np_(e_out).reshape(n_seq, n_per, 512)
    gc, gs = np_(codes), np_(scales)
    assert not gc[:, :5].any() and not gc[:, 5 + n_per:].any()
    for s in range(n_seq):
        e_ref32 = oracle.compress_rope_fp32(x[s], w, cs[s], 64, 1e-6)
        ulps = np.abs(e_gpu[s].view(np.int32).astype(np.int64) - e_ref32.view(np.int32).astype(np.int64))
        assert ulps.max() <= 1 and (ulps > 0).mean() < 1e-3, (ulps.max(), (ulps > 0).mean())
        c2, s2 = mxfp4.quantize(e_gpu[s])                 # strict: same fp32 input -> same bytes
        assert np.array_equal(gc[s, 5:5 + n_per], c2) and np.array_equal(gs[s, 5:5 + n_per], s2)
        rc, rsc = mxfp4.quantize(e_ref32)                 # chain level
        assert np.array_equal(rc, c2) and np.array_equal(rsc, s2)


def _scores_case(rng, n_seq, q_per_seq, n_entries, k_rows, pos_base):
    Q = n_seq * q_per_seq
    q8 = formats.e4m3_encode(rng.standard_normal((Q, 8, 128)))
    k8 = formats.e4m3_encode(rng.standard_normal((n_seq, k_rows, 128)))
    w = rng.random((Q, 8)).astype(np.float32)
    pos = np.array([pos_base + (i % q_per_seq) for i in range(Q)], np.int32)
    return q8, k8, w, pos


@pytest.mark.parametrize("n_seq,q_per_seq,n_entries,pos_base",
                         [(3, 1, 3000, 4 * 2990 + 1), (1, 96, 1500, 4 * 1480), (2, 40, 333, 4 * 300)])
def test_index_score_dense(n_seq, q_per_seq, n_entries, pos_base):
    rng = np.random.default_rng(n_entries)
    k_rows = n_entries + 5
    q8, k8, w, pos = _scores_case(rng, n_seq, q_per_seq, n_entries, k_rows, pos_base)
    scores, bm = ops.csa_index_score(t_(q8), t_(w), t_(pos), t_(k8), n_seq, q_per_seq, n_entries,
                                     want_block_max=True)
    torch.cuda.synchronize()
    sc, bmg = np_(scores), np_(bm)
    worst = 0.0
    for qi in range(n_seq * q_per_seq):
        s = qi // q_per_seq
        nv = oracle.visible_entries(pos[qi], n_entries)
        ref = oracle.index_scores(q8[qi], w[qi], k8[s, :nv])
        err = np.abs(sc[qi, :nv] - ref) / np.maximum(1.0, np.abs(ref))
        worst = max(worst, float(err.max()) if nv else 0.0)
        assert np.all(np.isneginf(sc[qi, nv:]))
        # block max = max of this call's own scores, bit for bit
        for b in range(bmg.shape[1]):
            seg = sc[qi, 8 * b: 8 * b + 8]
            assert bmg[qi, b] == seg.max() or (np.isneginf(bmg[qi, b]) and np.all(np.isneginf(seg)))
    assert worst <= 2e-6, worst


def test_index_score_dense_scan_several_chunks_per_block():
    """Decode-shaped scoring (fewer than 32 queries per sequence) where each
    block streams several 1,024-column chunks (1,120 queries, 3 chunks, the
    last one ragged), the launch shape of long-context decode."""
    rng = np.random.default_rng(77)
    n_seq, q_per_seq, n_entries = 70, 16, 2600
    Q = n_seq * q_per_seq
    q8, k8, w, _ = _scores_case(rng, n_seq, q_per_seq, n_entries, n_entries + 3, 0)
    pos = rng.integers(4 * 2000, 4 * n_entries + 40, Q).astype(np.int32)   # partial and full visibility
    scores, bm = ops.csa_index_score(t_(q8), t_(w), t_(pos), t_(k8), n_seq, q_per_seq, n_entries,
                                     want_block_max=True)
    torch.cuda.synchronize()
    sc, bmg = np_(scores), np_(bm)
    qv = formats.e4m3_decode(q8).astype(np.float64)
    kv = formats.e4m3_decode(k8).astype(np.float64)
    for s in range(n_seq):
        rows = slice(s * q_per_seq, (s + 1) * q_per_seq)
        dots = np.einsum("qhd,nd->qhn", qv[rows], kv[s, :n_entries])          # exact for E4M3 operands
        ref = np.einsum("qh,qhn->qn", w[rows].astype(np.float64), np.maximum(dots, 0.0))
        nv = np.minimum((pos[rows].astype(np.int64) + 1) // 4, n_entries)
        vis = np.arange(n_entries)[None, :] < nv[:, None]
        got = sc[rows]
        assert np.all(np.abs(got - ref)[vis] <= 2e-6 * np.maximum(1.0, np.abs(ref[vis])))
        assert np.all(np.isneginf(got[~vis]))
        pad = np.full((q_per_seq, bmg.shape[1] * 8), -np.inf, np.float32)
        pad[:, :n_entries] = got
        assert np.array_equal(bmg[rows], pad.reshape(q_per_seq, -1, 8).max(axis=2))


@pytest.mark.parametrize("n_seq,q_per_seq", [(2, 40), (3, 100)])
def test_index_score_ragged_tiles_stay_in_bounds(n_seq, q_per_seq):
    """Prefill tiles hold 64 queries; a sequence whose query count is not a
    multiple of 64 ends in a partly filled tile.  Its absent rows must not be
    written: guard rows around the score and block-max outputs keep their
    bytes, and the live rows match the oracle."""
    rng = np.random.default_rng(q_per_seq)
    n_entries = 700
    q8, k8, w, pos = _scores_case(rng, n_seq, q_per_seq, n_entries, n_entries, 4 * 660)
    Q, nblk, G = n_seq * q_per_seq, (n_entries + 7) // 8, 64
    guard = np.float32(np.uint32(0x7FC01234).view(np.float32))       # a NaN the kernel never writes
    sc_all = torch.full((Q + 2 * G, n_entries), float(guard), dtype=torch.float32, device=DEV)
    bm_all = torch.full((Q + 2 * G, nblk), float(guard), dtype=torch.float32, device=DEV)
    sc_all.view(torch.int32).fill_(0x7FC01234)
    bm_all.view(torch.int32).fill_(0x7FC01234)
    qd, wd, pd, kd = t_(q8), t_(w), t_(pos), t_(k8)
    lib = ops._lib.load()
    rc = lib.csa_index_score(qd.data_ptr(), wd.data_ptr(), pd.data_ptr(), n_seq, q_per_seq, kd.data_ptr(),
                             n_entries, n_entries, None, 0, sc_all[G].data_ptr(), bm_all[G].data_ptr(),
                             ops._stream())
    assert rc == 0, lib.csa_last_error()
    torch.cuda.synchronize()
    sc_bits, bm_bits = np_(sc_all.view(torch.int32)), np_(bm_all.view(torch.int32))
    for rows in (slice(0, G), slice(G + Q, 2 * G + Q)):
        assert np.all(sc_bits[rows] == 0x7FC01234) and np.all(bm_bits[rows] == 0x7FC01234)
    sc = np_(sc_all)[G:G + Q]
    for qi in range(Q):
        s = qi // q_per_seq
        nv = oracle.visible_entries(pos[qi], n_entries)
        ref = oracle.index_scores(q8[qi], w[qi], k8[s, :nv])
        assert np.all(np.abs(sc[qi, :nv] - ref) <= 2e-6 * np.maximum(1.0, np.abs(ref)))
        assert np.all(np.isneginf(sc[qi, nv:]))


def test_index_score_pooled_matches_dense_bitwise():
    rng = np.random.default_rng(5)
    n_seq, n_entries = 2, 2000
    q8, k8, w, pos = _scores_case(rng, n_seq, 1, n_entries, n_entries, 4 * 1995 + 2)
    nb = 40
    pool = np.full((n_seq, nb), -1, np.int32)
    for s in range(n_seq):
        blocks = np.sort(rng.choice(250, nb - 3, replace=False))
        blocks[-1] = 249                                    # partially visible last block
        pool[s, :nb - 3] = blocks
    dense, _ = ops.csa_index_score(t_(q8), t_(w), t_(pos), t_(k8), n_seq, 1, n_entries)
    pooled, _ = ops.csa_index_score(t_(q8), t_(w), t_(pos), t_(k8), n_seq, 1, n_entries,
                                    pool_blocks=t_(pool))
    torch.cuda.synchronize()
    d, p = np_(dense), np_(pooled)
    for s in range(n_seq):
        nv = oracle.visible_entries(pos[s], n_entries)
        for c in range(8 * nb):
            b = pool[s, c // 8]
            e = 8 * b + c % 8
            if b < 0 or e >= nv:
                assert np.isneginf(p[s, c])
            else:
                assert p[s, c] == d[s, e]


def _oracle_topk_fp32(row, k, ids=None):
    valid = ~(np.isneginf(row) | np.isnan(row))
    ids = np.arange(len(row)) if ids is None else np.asarray(ids)
    return oracle.topk(row[valid].astype(np.float64), k, ids=ids[valid])


def _score_rows(rng, dist, Q, ncols):
    """Score rows of several value distributions (ties, few levels, wide range)."""
    if dist == "ties":
        return rng.integers(0, 200, (Q, ncols)).astype(np.float32) * np.float32(0.25)
    if dist == "few":          # a handful of levels: the threshold bin is large
        return rng.integers(0, 4, (Q, ncols)).astype(np.float32)
    if dist == "const":
        return np.full((Q, ncols), 1.5, np.float32)
    if dist == "normal":
        return rng.standard_normal((Q, ncols)).astype(np.float32)
    # wide: magnitudes over 60 decades, both signs, plus the largest finite values
    v = (10.0 ** rng.uniform(-30, 30, (Q, ncols))) * rng.choice([-1.0, 1.0], (Q, ncols))
    v = v.astype(np.float32)
    v[:, 1::97] = np.float32(3.4e38)
    v[:, 2::89] = np.float32(-3.4e38)
    return v


@pytest.mark.parametrize("Q,ncols,k,dist", [(3, 100, 512, "ties"), (2, 5000, 512, "ties"),
                                            (2, 20000, 512, "ties"), (2, 300000, 512, "ties"),
                                            (2, 40000, 2048, "ties"), (1, 16384, 4096, "ties"),
                                            (2, 16384, 512, "few"), (2, 40000, 512, "few"),
                                            (2, 16384, 512, "const"), (2, 50000, 512, "normal"),
                                            (2, 16384, 512, "wide"), (2, 70000, 1000, "wide")])
def test_topk_exact(Q, ncols, k, dist):
    rng = np.random.default_rng(ncols + k)
    sc = _score_rows(rng, dist, Q, ncols)
    sc[:, ::7] = -np.inf
    sc[0, :ncols // 3] = -np.inf
    if ncols > 10:
        sc[-1, 3] = -0.0
        sc[-1, 4] = 0.0
        sc[-1, 5] = np.nan
    idx = ops.csa_topk(t_(sc), k=k)
    torch.cuda.synchronize()
    got = np_(idx)
    for q in range(Q):
        assert np.array_equal(got[q], _oracle_topk_fp32(sc[q], k)), q


@pytest.mark.parametrize("Q,ncols,k,dist,pooled", [(1024, 16384, 512, "ties", False), (1100, 9000, 512, "few", False),
                                                   (1024, 16384, 512, "ties", True)])
def test_topk_many_rows(Q, ncols, k, dist, pooled):
    """1,024 rows and more take the block shape for many rows (several
    blocks per compute unit); sampled rows are checked exactly."""
    rng = np.random.default_rng(Q + ncols + pooled)
    sc = _score_rows(rng, dist, Q, ncols)
    sc[:, ::11] = -np.inf
    sc[5, :] = -np.inf                       # a row with nothing valid
    sc[6, : ncols - 100] = -np.inf           # fewer valid keys than k
    blocks = None
    if pooled:
        nb = ncols // 8
        blocks = np.stack([np.sort(rng.choice(3 * nb, nb, replace=False)) for _ in range(Q)]).astype(np.int32)
        blocks[7, -9:] = -1
        sc[7, -72:] = -np.inf                # absent blocks score -inf, as the pooled scoring writes them
        idx = ops.csa_topk(t_(sc), k=k, col_blocks=t_(blocks))
    else:
        idx = ops.csa_topk(t_(sc), k=k)
    torch.cuda.synchronize()
    got = np_(idx)
    rows = sorted(set([0, 1, 5, 6, 7, Q // 2, Q - 1] + list(rng.choice(Q, 9, replace=False))))
    for q in rows:
        if pooled:
            ids = (8 * blocks[q][:, None] + np.arange(8)[None]).reshape(-1)
            want = _oracle_topk_fp32(sc[q], k, ids=ids)
        else:
            want = _oracle_topk_fp32(sc[q], k)
        assert np.array_equal(got[q], want), q


@pytest.mark.parametrize("nb,k", [(300, 100), (5000, 512)])     # 5000 blocks: several chunks
def test_topk_pooled_mapping(nb, k):
    rng = np.random.default_rng(9 + nb)
    Q = 2
    blocks = np.stack([np.sort(rng.choice(3 * nb, nb, replace=False)) for _ in range(Q)]).astype(np.int32)
    blocks[1, -7:] = -1
    sc = rng.integers(0, 30, (Q, 8 * nb)).astype(np.float32)
    sc[1, -56:] = -np.inf
    idx = ops.csa_topk(t_(sc), k=k, col_blocks=t_(blocks))
    torch.cuda.synchronize()
    got = np_(idx)
    for q in range(Q):
        ids = (8 * blocks[q][:, None] + np.arange(8)[None]).reshape(-1)
        assert np.array_equal(got[q], _oracle_topk_fp32(sc[q], k, ids=ids))


@pytest.mark.parametrize("is_bm,Q,ncols,nb", [(True, 2, 33000, 2048), (True, 3, 1000, 2048),
                                              (False, 2, 70001, 2048), (False, 1, 4000, 100)])
def test_block_pool_exact(is_bm, Q, ncols, nb):
    rng = np.random.default_rng(ncols)
    v = rng.integers(0, 500, (Q, ncols)).astype(np.float32)
    v[:, ::5] = -np.inf
    pool = ops.csa_block_pool(t_(v), is_block_max=is_bm, n_pool_blocks=nb)
    torch.cuda.synchronize()
    got = np_(pool)
    for q in range(Q):
        if is_bm:
            ref = _oracle_topk_fp32(v[q], nb)
        else:
            row = v[q].astype(np.float64)
            nblk = (ncols + 7) // 8
            bm = np.array([row[8 * b: 8 * b + 8].max() for b in range(nblk)])
            ref = _oracle_topk_fp32(bm, nb)
        assert np.array_equal(got[q], ref)


def _attn_case(rng, n_seq, q_per_seq, rows, k, win_cap, p_base, invalid_frac=0.05):
    Q = n_seq * q_per_seq
    codes = rng.integers(0, 256, (n_seq, rows, 256)).astype(np.uint8)
    scales = rng.integers(0x28, 0x31, (n_seq, rows, 32)).astype(np.uint8)
    win = formats.e4m3_encode(rng.standard_normal((n_seq, win_cap, 512)))
    q = rng.standard_normal((Q, 16, 512)).astype(np.float32)
    idx = np.stack([np.sort(rng.choice(rows, k, replace=False)) for _ in range(Q)]).astype(np.int32)
    idx[rng.random(idx.shape) < invalid_frac] = -1
    pos = np.array([p_base + (i % q_per_seq) for i in range(Q)], np.int32)
    return codes, scales, win, q, idx, pos


def _attn_ref(codes, scales, win, q, idx, pos, q_per_seq, win_cap):
    outs = []
    for qi in range(len(q)):
        s = qi // q_per_seq
        wp = oracle.window_positions(pos[qi])
        outs.append(oracle.sparse_attention(q[qi], codes[s], scales[s], idx[qi], win[s, wp % win_cap], SM))
    return np.stack(outs)


# From 512 queries on (prefill) the launch plan changes: one key group, one split.
@pytest.mark.parametrize("n_seq,q_per_seq,k,p_base", [(4, 1, 512, 5000), (1, 300, 512, 2000),
                                                      (2, 1, 77, 60), (1, 1, 512, 0),
                                                      (1, 523, 512, 50), (2, 300, 77, 3000)])
def test_sparse_attn(n_seq, q_per_seq, k, p_base):
    rng = np.random.default_rng(k + p_base)
    rows, win_cap = 1200, 128 + (q_per_seq if q_per_seq > 1 else 0)
    codes, scales, win, q, idx, pos = _attn_case(rng, n_seq, q_per_seq, rows, k, win_cap, p_base)
    out = ops.csa_sparse_attn(t_(q), t_(pos), t_(codes), t_(scales), t_(idx), t_(win), n_seq, q_per_seq)
    torch.cuda.synchronize()
    check_attn(np_(out), _attn_ref(codes, scales, win, q, idx, pos, q_per_seq, win_cap))


# Decode plans: E entry pairs + one window pair per block for E = 1..4 (Q and
# k chosen so that each E occurs), k not a multiple of the 32-slot pair, the
# largest k of the pair plan (2,048: 16 splits) and the first k past it,
# which the stream kernel takes in splits.
@pytest.mark.parametrize("n_seq,k", [(32, 640), (32, 2048), (8, 2049), (64, 500), (3, 33), (16, 96)])
def test_sparse_attn_decode_plans(n_seq, k):
    rng = np.random.default_rng(7 * k + n_seq)
    rows, win_cap = 2600, 128
    codes, scales, win, q, idx, pos = _attn_case(rng, n_seq, 1, rows, k, win_cap, 9000)
    out = ops.csa_sparse_attn(t_(q), t_(pos), t_(codes), t_(scales), t_(idx), t_(win), n_seq, 1)
    torch.cuda.synchronize()
    check_attn(np_(out), _attn_ref(codes, scales, win, q, idx, pos, 1, win_cap))


def test_sparse_attn_dense_case_and_empty_selection():
    """K >= visible: attention over every entry + window; and no entry selected."""
    rng = np.random.default_rng(11)
    rows = 900
    codes, scales, win, q, _, pos = _attn_case(rng, 1, 1, rows, 10, 128, 7000)
    idx = np.arange(rows, dtype=np.int32)[None]
    out = ops.csa_sparse_attn(t_(q), t_(pos), t_(codes), t_(scales), t_(idx), t_(win), 1, 1)
    none = np.full((1, 512), -1, np.int32)
    out2 = ops.csa_sparse_attn(t_(q), t_(pos), t_(codes), t_(scales), t_(none), t_(win), 1, 1)
    torch.cuda.synchronize()
    check_attn(np_(out), _attn_ref(codes, scales, win, q, idx, pos, 1, 128))
    check_attn(np_(out2), _attn_ref(codes, scales, win, q, none, pos, 1, 128))


# ------------------------------------------------------------------ f2 ----

@pytest.mark.parametrize("cap,n_tok_rule", [(128, "full"), (192, "full"), (128, "short")])
def test_window_rebuild_bit_exact(cap, n_tok_rule):
    """csa_window_rebuild vs the oracle's rebuild for rings at positions that
    cover an empty history, a partial window, the wrap and large positions."""
    ps = [0, 3, 126, 127, 128, 129, 1000, 4095, 262143, (1 << 22) + 5]
    n_tok = 128 if n_tok_rule == "full" else 50
    rng = np.random.default_rng(cap + n_tok)
    x = (rng.standard_normal((len(ps), n_tok, 512)) * 40).astype(np.float32)
    x[0, -1, :8] = [0.0, -0.0, 1e-9, 500.0, -500.0, 448.0, 464.0, 2.0 ** -9]
    win = torch.full((len(ps), cap, 512), 0xAB, dtype=torch.uint8, device=DEV)
    ops.csa_window_rebuild(torch.from_numpy(x).to(DEV), torch.tensor(ps, dtype=torch.int32, device=DEV), win,
                           len(ps), n_tok)
    got = np_(win)
    for r, p in enumerate(ps):
        n = min(n_tok, p + 1)
        ref = oracle.window_rebuild(x[r, n_tok - n:], p, cap)
        assert np.array_equal(got[r], ref), (r, p)


def test_window_rebuild_then_append_matches_rebuild_later():
    """Rebuild at position p, append token p+1 with csa_window_append: the ring
    equals the rebuild at p+1 (decode continues from a rebuilt window)."""
    rng = np.random.default_rng(5)
    n_ring, p = 6, 10_000
    x = torch.from_numpy(rng.standard_normal((n_ring, 129, 512)).astype(np.float32)).to(DEV)
    pl = torch.full((n_ring,), p, dtype=torch.int32, device=DEV)
    a = torch.empty((n_ring, 128, 512), dtype=torch.uint8, device=DEV)
    b = torch.empty_like(a)
    ops.csa_window_rebuild(x, pl, a, n_ring, 128, x_ring_stride=129 * 512)
    ops.csa_window_append(x, pl + 1, a, n_ring, 1, x_seq_stride=129 * 512, x_offset=128 * 512)
    ops.csa_window_rebuild(x, pl + 1, b, n_ring, 128, x_ring_stride=129 * 512, x_offset=512)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_index_score_pooled_ids_beyond_entries():
    """Pool ids whose entries lie at or past n_entries score -inf (a partly
    valid last block keeps its valid entries), including ids so large that
    8 * id does not fit 32 bits; valid blocks match the oracle."""
    rng = np.random.default_rng(21)
    n_seq, n_entries = 2, 1001                     # block 125 holds entry 1000 only
    q8, k8, w, pos = _scores_case(rng, n_seq, 1, n_entries, n_entries + 3, 4 * 1100)
    pool = np.array([[0, 5, 125, 126, 4000, (1 << 30) - 1, -1, -1],
                     [3, 7, 125, (1 << 28) + 1, 2 ** 31 - 1, -1, -1, -1]], np.int32)
    sc, _ = ops.csa_index_score(t_(q8), t_(w), t_(pos), t_(k8), n_seq, 1, n_entries, pool_blocks=t_(pool))
    torch.cuda.synchronize()
    got = np_(sc)
    for s in range(n_seq):
        ref = oracle.index_scores(q8[s], w[s], k8[s, :n_entries])
        for c in range(8 * pool.shape[1]):
            b = int(pool[s, c // 8])
            e = 8 * b + c % 8
            if b < 0 or e >= n_entries:
                assert np.isneginf(got[s, c]), (s, c, b)
            else:
                assert abs(got[s, c] - ref[e]) <= 2e-6 * max(1.0, abs(ref[e])), (s, c, b)


def test_index_score_pooled_nothing_visible():
    """Pooled scoring with no visible entry (no entries at all, or a query
    before the first complete entry): every column is -inf."""
    rng = np.random.default_rng(9)
    q8 = formats.e4m3_encode(rng.standard_normal((2, 8, 128)))
    w = rng.random((2, 8)).astype(np.float32)
    k8 = formats.e4m3_encode(rng.standard_normal((2, 64, 128)))
    pool = np.tile(np.arange(8, dtype=np.int32), (2, 1))
    for n_entries, pos in [(0, [100, 200]), (64, [2, 1])]:
        sc, _ = ops.csa_index_score(t_(q8), t_(w), t_(np.array(pos, np.int32)), t_(k8), 2, 1, n_entries,
                                    pool_blocks=t_(pool))
        torch.cuda.synchronize()
        assert np.isneginf(np_(sc)).all()


def _peaked_case(rng, n_seq, q_per_seq, rows, k):
    """Selections holding two entries a, b with equal first halves (u) and
    opposite second halves (+v, -v) at scale 1, among small entries and a
    small window; half of the heads point at u (logit ~25-30) with a slight
    lean to +v, so the softmax puts nearly all weight on a and b and their v
    halves cancel in the output; the other heads are 8 x N(0,1), a peaked
    softmax over keys of mixed sign."""
    Q = n_seq * q_per_seq
    codes = rng.integers(0, 256, (n_seq, rows, 256)).astype(np.uint8)
    scales = rng.integers(0x20, 0x28, (n_seq, rows, 32)).astype(np.uint8)
    ia, ib = 10, 20
    mag = rng.integers(1, 8, (n_seq, 512)).astype(np.uint8)         # E2M1 magnitudes 0.5 .. 6
    sgn = rng.integers(0, 2, (n_seq, 512)).astype(np.uint8) << 3
    ca = mag | sgn
    cb = ca.copy()
    cb[:, 256:] ^= 8                                                 # opposite sign on the v half
    codes[:, ia] = ca[:, 0::2] | (ca[:, 1::2] << 4)
    codes[:, ib] = cb[:, 0::2] | (cb[:, 1::2] << 4)
    scales[:, ia] = scales[:, ib] = 0x38                             # 1.0
    win = formats.e4m3_encode(0.1 * rng.standard_normal((n_seq, 128 + q_per_seq, 512)))
    idx = np.stack([np.sort(np.concatenate([[ia, ib], rng.choice(np.arange(30, rows), k - 2, replace=False)]))
                    for _ in range(Q)]).astype(np.int32)
    q = (8.0 * rng.standard_normal((Q, 16, 512))).astype(np.float64)
    for qi in range(Q):
        s = qi // q_per_seq
        a = mxfp4.dequantize(codes[s, ia], scales[s, ia])
        u, v = a.copy(), a.copy()
        u[256:] = 0.0
        v[:256] = 0.0
        for h in range(8):
            gam = rng.uniform(25, 30) * np.sqrt(512) / (u @ u)
            dl = rng.uniform(0.0, 1.0) * np.sqrt(512) / (v @ v)
            q[qi, h] = gam * u + dl * v
    pos = np.array([5000 + (i % q_per_seq) for i in range(Q)], np.int32)
    return codes, scales, win, q.astype(np.float32), idx, pos


# decode (split plan: few queries) and prefill (stream plan: 512+ queries)
@pytest.mark.parametrize("n_seq,q_per_seq", [(4, 1), (1, 520)])
def test_sparse_attn_peaked_cancelling_softmax(n_seq, q_per_seq):
    rng = np.random.default_rng(31 + q_per_seq)
    rows, k, win_cap = 1500, 512, 128 + q_per_seq
    codes, scales, win, q, idx, pos = _peaked_case(rng, n_seq, q_per_seq, rows, k)
    out = ops.csa_sparse_attn(t_(q), t_(pos), t_(codes), t_(scales), t_(idx), t_(win), n_seq, q_per_seq)
    torch.cuda.synchronize()
    qs = range(n_seq * q_per_seq) if q_per_seq == 1 else list(range(0, 520, 13)) + [519]
    got = np_(out)
    for qi in qs:
        s = qi // q_per_seq
        wp = oracle.window_positions(pos[qi])
        ref = oracle.sparse_attention(q[qi], codes[s], scales[s], idx[qi], win[s, wp % win_cap], SM)
        check_attn(got[qi], ref)
        # the case is what it claims: the u heads put more than 99% of their
        # softmax weight on a and b (whose v halves then largely cancel)
        kv = mxfp4.dequantize(codes[s][[10, 20]], scales[s][[10, 20]])
        allk = np.concatenate([mxfp4.dequantize(codes[s][idx[qi]], scales[s][idx[qi]]),
                               formats.e4m3_decode(win[s, wp % win_cap])])
        lg = (q[qi, :8].astype(np.float64) @ allk.T) * SM
        lab = (q[qi, :8].astype(np.float64) @ kv.T) * SM
        wab = np.exp(lab - lg.max(-1, keepdims=True)).sum(-1) / np.exp(lg - lg.max(-1, keepdims=True)).sum(-1)
        assert wab.min() > 0.99, wab.min()


@pytest.mark.parametrize("n_ent,top_k", [(3000, 4096), (16000, 16384)])
def test_full_layer_k_at_least_visible_is_dense(n_ent, top_k):
    """Check (b) through the library: a Full layer whose Top-K covers every
    visible entry selects all of them (ascending, -1 padded) and its
    attention is dense attention over the compressed cache plus the window."""
    rng = np.random.default_rng(n_ent)
    n_seq, win_cap = 2, 128
    codes = rng.integers(0, 256, (n_seq, n_ent, 256)).astype(np.uint8)
    scales = rng.integers(0x28, 0x31, (n_seq, n_ent, 32)).astype(np.uint8)
    k8 = formats.e4m3_encode(rng.standard_normal((n_seq, n_ent, 128)))
    q8 = formats.e4m3_encode(rng.standard_normal((n_seq, 8, 128)))
    w = rng.random((n_seq, 8)).astype(np.float32)
    q_attn = rng.standard_normal((n_seq, 16, 512)).astype(np.float32)
    win = formats.e4m3_encode(rng.standard_normal((n_seq, win_cap, 512)))
    pos = np.array([4 * n_ent - 1, 4 * n_ent - 1 - 403], np.int32)      # second: a partial block
    idx = torch.empty((n_seq, top_k), dtype=torch.int32, device=DEV)
    out = torch.empty((n_seq, 16, 512), dtype=torch.float32, device=DEV)
    call = ops.LayerCall(ops.MODE_FULL, codes=t_(codes), scales=t_(scales), k_fp8=t_(k8), win=t_(win),
                         q_pos=t_(pos), q_attn=t_(q_attn), idx=idx, out=out, n_seq=n_seq, q_per_seq=1,
                         n_entries=n_ent, q_idx=t_(q8), w_idx=t_(w), top_k=top_k)
    call()
    torch.cuda.synchronize()
    gi, go = np_(idx), np_(out)
    for s in range(n_seq):
        nv = oracle.visible_entries(pos[s], n_ent)
        want = np.full(top_k, -1, np.int64)
        want[:nv] = np.arange(nv)
        assert np.array_equal(gi[s], want), s
        wp = oracle.window_positions(pos[s])
        dense = oracle.sparse_attention(q_attn[s], codes[s], scales[s], np.arange(nv), win[s, wp % win_cap], SM)
        check_attn(go[s], dense)
        ref = oracle.layer_full(codes[s], scales[s], k8[s], q8[s], w[s], q_attn[s], pos[s], win[s, wp % win_cap],
                                SM, k=top_k, n_entries=n_ent)
        assert np.array_equal(ref.idx, want)


def test_side_stream_call_keeps_its_workspace():
    """csa_sparse_attn launched on a side stream with a binding-allocated
    workspace (decode plan: split partials): the current stream then
    allocates and overwrites memory at once; the side stream's output still
    matches the oracle (the workspace was recorded as in use there)."""
    rng = np.random.default_rng(41)
    rows, k, win_cap = 3000, 512, 128
    codes, scales, win, q, idx, pos = _attn_case(rng, 16, 1, rows, k, win_cap, 9000)
    tq, tpos, tc, ts, ti, tw = t_(q), t_(pos), t_(codes), t_(scales), t_(idx), t_(win)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())   # the inputs were written on the current stream
    out = ops.csa_sparse_attn(tq, tpos, tc, ts, ti, tw, 16, 1, stream=side)
    junk = [torch.full((1 << 22,), 1e30, device=DEV) for _ in range(8)]   # reuse freed blocks at once
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    check_attn(np_(out), _attn_ref(codes, scales, win, q, idx, pos, 1, win_cap))
