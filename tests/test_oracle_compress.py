"""Pins of the oracle's compressor, RMSNorm and RoPE.

Pinned against: torch's rms_norm (library) in the special case W_0 = I,
W_1..3 = 0; the page's norm bound sqrt(512) ~ 22.6 (RMSNorm output magnitude
about 1); linearity of the compressor checked with numpy's einsum over the
whole [n, 4, 512] x [4, 512, 512] contraction; RoPE as complex multiplication
(numpy complex arithmetic), its norm preservation (page), and exact quarter
turns.
"""

import json
import os

import numpy as np
import torch

from oracle import compressor as C

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
PAGE = json.load(open(os.path.join(GOLDEN, "page_constants.json")))


def test_identity_weight_reduces_to_rmsnorm():
    rng = np.random.default_rng(0)
    n, d = 64, 512
    x = rng.standard_normal((4 * n, d)).astype(np.float32)
    w = np.zeros((4, d, d))
    w[0] = np.eye(d)
    e = C.compress(x, w, eps=1e-6)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x[0::4].astype(np.float64)), (d,), eps=1e-6)
    np.testing.assert_allclose(e, ref.numpy(), rtol=1e-13, atol=1e-13)


def test_each_weight_slot_sees_its_token():
    rng = np.random.default_rng(1)
    n, d = 16, 512
    x = rng.standard_normal((n, 4, d))
    w = rng.standard_normal((4, d, d)) / np.sqrt(4 * d)
    y = np.einsum("nic,ioc->no", x, w)
    ref = y / np.sqrt((y ** 2).mean(-1, keepdims=True) + 1e-6)
    np.testing.assert_allclose(C.compress(x, w, 1e-6), ref, rtol=1e-12, atol=1e-12)
    # swapping two tokens of an entry is not the same as swapping the weights' slots
    # unless the weights are swapped too
    x2 = x[:, [1, 0, 2, 3], :]
    w2 = w[[1, 0, 2, 3]]
    np.testing.assert_allclose(C.compress(x2, w2, 1e-6), ref, rtol=1e-12, atol=1e-12)


def test_norm_bound_from_page():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((4 * 128, 512)) * rng.choice([1e-4, 1, 1e3], (4 * 128, 1))).astype(np.float32)
    w = rng.standard_normal((4, 512, 512)) / np.sqrt(2048)
    e = C.compress(x, w, 1e-6)
    norms = np.linalg.norm(e, axis=-1)
    assert np.all(norms <= PAGE["norm_bound"] + 0.03)   # sqrt(512) = 22.627
    assert np.all(norms <= np.sqrt(PAGE["latent_dim"]) * (1 + 1e-12))
    rms = np.sqrt((e ** 2).mean(-1))
    assert np.all(rms <= 1.0 + 1e-12)


def test_rope_is_complex_multiplication_on_last_channels():
    rng = np.random.default_rng(3)
    n, d, rd = 8, 512, 64
    e = rng.standard_normal((n, d))
    ang = rng.uniform(-10, 10, (n, rd // 2))
    cs = np.stack([np.cos(ang), np.sin(ang)], -1)
    out = C.rope_rotate(e, cs, rd)
    np.testing.assert_array_equal(out[:, : d - rd], e[:, : d - rd])
    z = (e[:, d - rd::2] + 1j * e[:, d - rd + 1::2]) * np.exp(1j * ang)
    np.testing.assert_allclose(out[:, d - rd::2], z.real, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out[:, d - rd + 1::2], z.imag, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(out, axis=-1), np.linalg.norm(e, axis=-1), rtol=1e-12)


def test_rope_quarter_turn_and_identity_are_exact():
    e = np.arange(512, dtype=np.float64)[None] + 0.5
    cs = np.zeros((1, 32, 2))
    cs[..., 0] = 1.0
    np.testing.assert_array_equal(C.rope_rotate(e, cs, 64), e)
    cs = np.zeros((1, 32, 2))
    cs[..., 1] = 1.0                     # angle pi/2: (x0, x1) -> (-x1, x0)
    out = C.rope_rotate(e, cs, 64)
    assert out[0, 448] == -e[0, 449] and out[0, 449] == e[0, 448]
    assert C.rope_rotate(e, cs, 0) is not e and np.array_equal(C.rope_rotate(e, cs, 0), e)


def test_quantizer_input_is_fp32_rounding():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((16, 512)).astype(np.float32)
    w = rng.standard_normal((4, 512, 512)) / np.sqrt(2048)
    cs = np.stack([np.ones((4, 32)), np.zeros((4, 32))], -1)
    e32 = C.compress_rope_fp32(x, w, cs, 64, 1e-6)
    assert e32.dtype == np.float32
    np.testing.assert_array_equal(e32, C.compress(x, w, 1e-6).astype(np.float32))
