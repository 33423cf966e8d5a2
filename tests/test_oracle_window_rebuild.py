"""Pins of the oracle's window rebuild ("DeepSeek-V4.1 架构解析" §03, SWA Bounded Replay: only the
latest n_win = 128 tokens are replayed).  The rebuild places each replayed
token directly at its ring row; the pins compare it with a different
computation, a ring that receives every token of the history one at a time,
and with the attention window the layer functions read.  CPU only."""

import numpy as np
import pytest

import oracle

rng = np.random.default_rng(11)


def ring_by_appending(x_hist, win_cap):
    """A zeroed ring that receives tokens 0 .. len-1 in order (token t at row t mod win_cap)."""
    ring = np.zeros((win_cap, x_hist.shape[1]), dtype=np.uint8)
    for t in range(len(x_hist)):
        ring[t % win_cap] = oracle.window_encode(x_hist[t])
    return ring


@pytest.mark.parametrize("p", [0, 1, 5, 126, 127, 128, 129, 255, 256, 1000])
def test_rebuild_equals_appending_the_history(p):
    x = rng.standard_normal((p + 1, 512)).astype(np.float32) * 3
    n = min(128, p + 1)
    ring = oracle.window_rebuild(x[p + 1 - n:], p, 128)
    assert np.array_equal(ring, ring_by_appending(x, 128))


@pytest.mark.parametrize("p,cap", [(300, 192), (100, 192), (5000, 256)])
def test_larger_ring_keeps_the_last_128_rows_and_zeros_the_rest(p, cap):
    x = rng.standard_normal((p + 1, 512)).astype(np.float32)
    n = min(128, p + 1)
    ring = oracle.window_rebuild(x[p + 1 - n:], p, cap)
    full = ring_by_appending(x, cap)
    recent = oracle.window_positions(p)
    assert np.array_equal(ring[recent % cap], full[recent % cap])
    others = np.setdiff1d(np.arange(cap), recent % cap)
    assert not ring[others].any()


def test_attention_window_rows_come_from_the_rebuilt_ring():
    """The rows the attention reads (positions max(0, p-127) .. p) hold those
    positions' tokens, in window order."""
    p = 777
    x = rng.standard_normal((p + 1, 512)).astype(np.float32)
    ring = oracle.window_rebuild(x[p - 127:], p, 128)
    pos = oracle.window_positions(p)
    assert np.array_equal(ring[pos % 128], oracle.window_encode(x[pos]))


def test_fewer_tokens_than_the_window_leave_zero_rows():
    p = 500
    x = rng.standard_normal((40, 512)).astype(np.float32)
    ring = oracle.window_rebuild(x, p, 128)
    filled = np.arange(p - 39, p + 1) % 128
    assert np.array_equal(ring[filled], oracle.window_encode(x))
    assert not np.delete(ring, filled, axis=0).any()
