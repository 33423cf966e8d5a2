"""Pins of the oracle's sparse attention and layer modes.

Pinned against: torch's scaled_dot_product_attention in float64 on the CPU (a
library routine) when K covers every visible entry (dense attention over the
compressed cache plus the window); closed forms (zero query -> mean of keys, a
single key -> that key); invariance to the order of the selected ids; Reuse
with the Full layer's query reproducing the Full layer's output; and a tiny
end-to-end chain checked stage by stage.
"""

import numpy as np
import torch

from oracle import attention, formats, mxfp4, select, indexer, compressor
from oracle.layer import layer_full, layer_reuse, layer_reindex, window_encode

SM = 512 ** -0.5


def rand_cache(rng, n):
    codes = rng.integers(0, 256, (n, 256)).astype(np.uint8)
    scales = rng.integers(0x28, 0x31, (n, 32)).astype(np.uint8)
    return codes, scales


def sdpa(q, kv):
    qt = torch.from_numpy(np.asarray(q, np.float64))[None, :, None, :]   # [1, H, 1, D]
    kt = torch.from_numpy(kv)[None, None].expand(1, q.shape[0], -1, -1)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, scale=SM)
    return out[0, :, 0, :].numpy()


def test_dense_case_equals_library_attention():
    rng = np.random.default_rng(0)
    n = 300
    codes, scales = rand_cache(rng, n)
    win = formats.e4m3_encode(rng.standard_normal((128, 512)))
    q = rng.standard_normal((16, 512)).astype(np.float32)
    idx = np.arange(n)                                    # K >= visible
    out = attention.sparse_attention(q, codes, scales, idx, win, SM)
    kv = np.concatenate([mxfp4.dequantize(codes, scales), formats.e4m3_decode(win)])
    np.testing.assert_allclose(out, sdpa(q, kv), rtol=1e-12, atol=1e-12)


def test_zero_query_gives_mean_of_keys_and_single_key():
    rng = np.random.default_rng(1)
    codes, scales = rand_cache(rng, 20)
    win = formats.e4m3_encode(rng.standard_normal((5, 512)))
    q = np.zeros((16, 512), np.float32)
    idx = np.array([3, 7, -1, 11])
    out = attention.sparse_attention(q, codes, scales, idx, win, SM)
    kv = np.concatenate([mxfp4.dequantize(codes[[3, 7, 11]], scales[[3, 7, 11]]),
                         formats.e4m3_decode(win)])
    np.testing.assert_allclose(out, np.broadcast_to(kv.mean(0), (16, 512)), rtol=1e-13, atol=1e-13)
    one = attention.sparse_attention(rng.standard_normal((16, 512)).astype(np.float32),
                                     codes, scales, np.array([-1, -1]), win[:1], SM)
    np.testing.assert_array_equal(one, np.broadcast_to(formats.e4m3_decode(win[0]), (16, 512)))


def test_order_invariance_and_window_positions():
    rng = np.random.default_rng(2)
    codes, scales = rand_cache(rng, 64)
    win = formats.e4m3_encode(rng.standard_normal((128, 512)))
    q = rng.standard_normal((16, 512)).astype(np.float32)
    idx = rng.permutation(64)[:20]
    a = attention.sparse_attention(q, codes, scales, idx, win, SM)
    b = attention.sparse_attention(q, codes, scales, np.sort(idx), win, SM)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)
    assert list(attention.window_positions(5)) == list(range(0, 6))
    assert list(attention.window_positions(1000)) == list(range(873, 1001))
    assert len(attention.window_positions(10 ** 6)) == 128


def test_reuse_with_full_query_reproduces_full_output():
    rng = np.random.default_rng(3)
    n = 700
    codes, scales = rand_cache(rng, n)
    k_fp8 = formats.e4m3_encode(rng.standard_normal((n, 128)))
    q = formats.e4m3_encode(rng.standard_normal((8, 128)))
    w = rng.random(8).astype(np.float32)
    qa = rng.standard_normal((16, 512)).astype(np.float32)
    win = formats.e4m3_encode(rng.standard_normal((128, 512)))
    full = layer_full(codes, scales, k_fp8, q, w, qa, 4 * n - 1, win, SM, k=512)
    re = layer_reuse(codes, scales, full.idx, qa, win, SM)
    np.testing.assert_array_equal(full.out, re.out)
    # Reindex without a pool scores every visible entry: same as Full
    ri = layer_reindex(codes, scales, k_fp8, None, q, w, qa, 4 * n - 1, win, SM)
    assert np.array_equal(ri.idx, full.idx)


def test_tiny_chain_stage_by_stage():
    """Brute force on tiny inputs: 24 entries, K = 2, 2 pool blocks of 8.

    (The pool holds the Top-K whenever the number of pool blocks is at least K.)
    """
    rng = np.random.default_rng(4)
    n, d = 24, 512
    x = rng.standard_normal((4 * n, d)).astype(np.float32)
    w = (rng.standard_normal((4, d, d)) / np.sqrt(4 * d)).astype(np.float32)
    ang = rng.uniform(0, 6, (n, 32))
    cs = np.stack([np.cos(ang), np.sin(ang)], -1).astype(np.float32)
    e32 = compressor.compress_rope_fp32(x, w, cs, 64, 1e-6)
    codes, scales = mxfp4.quantize(e32)
    # quantization error within one scale step
    deq = mxfp4.dequantize(codes, scales)
    s = np.repeat(formats.e4m3_decode(scales), 16, -1)
    assert np.all(np.abs(deq - e32) <= s)
    k_fp8 = formats.e4m3_encode(rng.standard_normal((n, 128)))
    q = formats.e4m3_encode(rng.standard_normal((8, 128)))
    wi = rng.random(8).astype(np.float32)
    p = 4 * 20 + 1                     # 20 entries visible (4*19+3 <= 81 < 4*20+3)
    assert indexer.visible_entries(p) == 20
    win = window_encode(x[max(0, p - 127): p + 1])
    full = layer_full(codes, scales, k_fp8, q, wi, rng.standard_normal((16, d)).astype(np.float32),
                      p, win, SM, build_pool=True, k=2, n_blocks=2)
    sc = full.scores
    assert len(sc) == 20
    chosen = set(full.idx.tolist())
    for a in chosen:
        for b in set(range(20)) - chosen:
            assert sc[a] > sc[b] or (sc[a] == sc[b] and a < b)
    bm = [sc[0:8].max(), sc[8:16].max(), sc[16:20].max()]
    order = sorted(range(3), key=lambda b: (-bm[b], b))[:2]
    assert list(full.pool) == sorted(order)
    members = {8 * b + i for b in full.pool for i in range(8)}
    assert chosen <= members
    assert len(win) == p + 1 and win.dtype == np.uint8
