"""Pins of the oracle's number formats and MXFP4 quantizer.

Pinned against: torch's float8_e4m3fn dtype (an independent library
implementation of the same format), the page's constants (448, 6, 2688, groups
of 16), hand-worked groups in tests/golden, and the round-trip property.
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import formats, mxfp4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
PAGE = json.load(open(os.path.join(GOLDEN, "page_constants.json")))


def torch_e4m3_decode(bytes_u8):
    t = torch.from_numpy(np.asarray(bytes_u8, dtype=np.uint8).copy())
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_e4m3_encode(x):
    t = torch.from_numpy(np.asarray(x, dtype=np.float32).copy())
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_all_bytes_match_torch():
    b = np.arange(256, dtype=np.uint8)
    ours = formats.e4m3_decode(b)
    ref = torch_e4m3_decode(b)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_e4m3_max_is_page_value():
    assert formats.E4M3_MAX == PAGE["e4m3_max"]
    assert formats.E2M1_MAX == PAGE["e2m1_max"]
    assert formats.E4M3_MAX * formats.E2M1_MAX == PAGE["mxfp4_range"]


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(1)
    vals = [rng.standard_normal(20000) * s for s in (1e-3, 0.1, 1, 30, 200)]
    # every midpoint of adjacent finite values, and +-1 ulp (fp32) around it
    pos = formats.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    x = np.concatenate(vals + [mids, up, dn, -mids, pos.astype(np.float32)]).astype(np.float32)
    x = x[np.abs(x) < 464]           # torch's cast is non-saturating from 464 on
    assert np.array_equal(formats.e4m3_encode(x), torch_e4m3_encode(x))


def test_e4m3_encode_saturates():
    x = np.array([464.0, 1000.0, 1e30, -500.0], dtype=np.float32)
    assert list(formats.e4m3_encode(x)) == [0x7E, 0x7E, 0x7E, 0xFE]


def test_e2m1_value_set():
    # E2M1: exponent bias 1, one mantissa bit; subnormals 0 and 0.5.
    expect = sorted({0.0, 0.5} | {2.0 ** (e - 1) * (1 + m / 2) for e in (1, 2, 3) for m in (0, 1)})
    assert list(formats.E2M1_VALUES) == expect
    c = np.arange(16)
    v = formats.e2m1_decode(c)
    assert np.array_equal(np.abs(v), np.tile(formats.E2M1_VALUES, 2))
    assert np.all(np.signbit(v[8:])) and not np.any(np.signbit(v[:8]))


def test_e2m1_encode_exhaustive_roundtrip_and_ties():
    c = np.arange(16)
    assert np.array_equal(formats.e2m1_encode(formats.e2m1_decode(c)), c)
    # ties go to the even code
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    assert list(formats.e2m1_encode(mids)) == [0, 2, 2, 4, 4, 6, 6]
    assert list(formats.e2m1_encode([6.1, 100.0, -7.0])) == [7, 7, 15]


def _load_cases():
    cases, cur = [], None
    for line in open(os.path.join(GOLDEN, "mxfp4_hand_worked.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, rest = line.split(None, 1)
        if key == "case":
            cur = {"name": rest}
            cases.append(cur)
        elif key == "x":
            cur["x"] = np.array([float(v) for v in rest.split()], dtype=np.float32)
        elif key == "scale":
            cur["scale"] = int(rest, 16)
        elif key == "codes":
            cur["codes"] = [int(v, 16) for v in rest.split()]
    return cases


@pytest.mark.parametrize("case", _load_cases(), ids=lambda c: c["name"])
def test_quantize_hand_worked(case):
    x = np.zeros(32, dtype=np.float32)
    x[:16] = case["x"]
    codes, scales = mxfp4.quantize(x[None])
    assert scales[0, 0] == case["scale"]
    nib = mxfp4.unpack_codes(codes)[0, :16]
    assert list(nib) == case["codes"]


def test_packing_layout():
    # channel 2k in the low nibble of byte k
    x = np.zeros(32, dtype=np.float32)
    x[0], x[1] = 6.0, -6.0     # codes 7 and f
    codes, scales = mxfp4.quantize(x[None])
    assert codes[0, 0] == 0xF7
    assert codes.shape == (1, 16) and scales.shape == (1, 2)


def test_roundtrip_exact_on_representable_groups():
    """s * v groups (s E4M3, v E2M1) with one element at +-6s quantize back exactly."""
    rng = np.random.default_rng(7)
    n = 4000
    s_bytes = rng.integers(0x08, 0x7F, size=n).astype(np.uint8)   # normal scales
    s = formats.e4m3_decode(s_bytes)
    codes = rng.integers(0, 16, size=(n, 16))
    lead = rng.integers(0, 16, size=n)
    codes[np.arange(n), lead] = np.where(rng.random(n) < 0.5, 7, 15)
    vals = formats.e2m1_decode(codes) * s[:, None]
    x = vals.astype(np.float32)
    assert np.array_equal(x.astype(np.float64), vals)          # exact in fp32
    q_codes, q_scales = mxfp4.quantize(x.reshape(n // 2, 32))
    assert np.array_equal(q_scales.reshape(n), s_bytes)
    got = mxfp4.unpack_codes(q_codes).reshape(n, 16)
    # +0 and -0 elements keep their sign bit
    assert np.array_equal(got, codes)
    back = mxfp4.dequantize(q_codes, q_scales).reshape(n, 16)
    assert np.array_equal(back, vals)


def test_quantize_error_bound_and_norm_range():
    """|x - deq| <= s (or the zero-scale bound) and |deq| <= 2688 everywhere."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((256, 512)) * rng.choice([1e-3, 1, 30], (256, 1))).astype(np.float32)
    codes, scales = mxfp4.quantize(x)
    deq = mxfp4.dequantize(codes, scales)
    s = np.repeat(formats.e4m3_decode(scales), 16, axis=-1)
    err = np.abs(deq - x.astype(np.float64))
    # grid spacing is at most 2s (between 4s and 6s) and the rounded scale
    # leaves |x|/s <= 6 * 17/16, so err <= s; a zero scale means amax <= 6 * 2**-10
    assert np.all(err <= np.maximum(s, 6 * 2.0 ** -10))
    assert np.all(np.abs(deq) <= PAGE["mxfp4_range"])
