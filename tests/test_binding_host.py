"""Host-side behaviour of the Python binding (CPU only)."""

import torch

from compressed_sparse_attention_04_amd import ops


class _FakeTensor:
    def __init__(self):
        self.recorded = []

    def record_stream(self, s):
        self.recorded.append(s)


def test_keep_records_side_stream_use(monkeypatch):
    """A call launched on a stream other than the current one marks the
    tensors the binding allocated for it as used by that stream; on the
    current stream (or with no stream given) nothing is recorded."""
    current, side = object(), object()
    monkeypatch.setattr(torch.cuda, "current_stream", lambda: current)
    a, b = _FakeTensor(), _FakeTensor()
    ops._keep(side, a, None, b)
    assert a.recorded == [side] and b.recorded == [side]
    c = _FakeTensor()
    ops._keep(current, c)
    ops._keep(None, c)
    assert c.recorded == []
