"""Sequence compression (m = 4 tokens -> 1 entry), RMSNorm and RoPE.

"DeepSeek-V4.1 架构解析" §02 lists "compress the sequence dimension: every m tokens become one entry"
among CSA2's three compression means; the DeepSeek V4 overview page §2.1 gives the predecessor's ratio of
4:1.  "DeepSeek-V4.1 架构解析" §03 says RMSNorm brings the entry's magnitude to about 1 (so the L2
norm of a 512-d latent is at most sqrt(512) ~ 22.6), that RoPE is applied before
quantization, and that RoPE preserves the norm.

Readings where the pages are silent (no compressor formula is given):
  * m = 4, non-overlapping windows; entry j covers tokens 4j .. 4j+3;
  * y_j = sum_{i<4} W_i @ X[4j+i] with each W_i of shape [out=512, in=512], no
    bias; e_j = y_j / sqrt(mean(y_j ** 2) + eps) (RMSNorm with unit gain);
  * RoPE acts on the last ``rope_dim`` channels as adjacent pairs
    (c, c+1), c even, rotated by the angle of the entry's last token position
    4j+3; the cos/sin table is an input ([n, rope_dim/2, 2] = (cos, sin)), so no
    transcendental is evaluated here;
  * the quantizer input is the float32 rounding of the float64 result.
"""

import numpy as np

M_TOKENS = 4


def compress(x_tokens, w, eps):
    """RMSNorm(sum_i W_i X[4j+i]) for every entry, in float64.

    x_tokens: [4n, D_in] or [n, 4, D_in]; w: [4, D_out, D_in].
    Returns e: [n, D_out] float64.
    """
    x = np.asarray(x_tokens, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    if x.ndim == 2:
        x = x.reshape(-1, M_TOKENS, x.shape[-1])
    y = np.zeros((x.shape[0], w.shape[1]), dtype=np.float64)
    for i in range(M_TOKENS):
        y += x[:, i, :] @ w[i].T
    rms = np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + eps)
    return y / rms


def rope_rotate(e, rope_cs, rope_dim):
    """Rotate the last ``rope_dim`` channels of e in adjacent pairs.

    e: [n, D]; rope_cs: [n, rope_dim/2, 2] holding (cos, sin) of each pair's
    angle.  (x0, x1) -> (x0 cos - x1 sin, x0 sin + x1 cos).
    """
    e = np.array(e, dtype=np.float64, copy=True)
    if rope_dim == 0:
        return e
    d = e.shape[-1]
    c0 = d - rope_dim
    cs = np.asarray(rope_cs, dtype=np.float64)
    cos = cs[..., 0]
    sin = cs[..., 1]
    x0 = e[:, c0::2].copy()
    x1 = e[:, c0 + 1::2].copy()
    e[:, c0::2] = x0 * cos - x1 * sin
    e[:, c0 + 1::2] = x0 * sin + x1 * cos
    return e


def compress_rope_fp32(x_tokens, w, rope_cs, rope_dim, eps):
    """The quantizer input: float32(RoPE(compress(X)))."""
    e = compress(x_tokens, w, eps)
    e = rope_rotate(e, rope_cs, rope_dim)
    return e.astype(np.float32)
