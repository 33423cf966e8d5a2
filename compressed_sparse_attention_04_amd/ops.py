"""Python binding of libcsa: one function per C entry point, same names.

Every function checks devices, dtypes, shapes and contiguity of the torch
tensors it is given, allocates outputs and workspaces with torch (device
memory is the only thing torch provides here), and calls the C entry point on
the current HIP stream.  All computation happens in the library's kernels.
"""

import ctypes
import os
import math

import torch

from . import _lib
from ._lib import CsaLayerArgs

D, HEADS, IDX_HEADS, IDX_DIM = 512, 16, 8, 128
TOP_K, POOL_BLOCKS, BLOCK, N_WIN = 512, 2048, 8, 128
MODE_FULL, MODE_REINDEX, MODE_REUSE = 0, 1, 2


class CsaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"libcsa status {status}: {message}")
        self.status = status
        self.message = message


def _call(name, *args):
    lib = _lib.load()
    rc = getattr(lib, name)(*args)
    if rc != 0:
        raise CsaError(rc, lib.csa_last_error().decode())


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype, device=None, shape=None, contiguous=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _keep(stream, *tensors):
    """Tensors this binding allocated for a call launched on ``stream`` (when
    that is not the current stream) are recorded as used by that stream, so
    the caching allocator, which tracks the current stream, does not hand
    their memory to later work before the call's kernels have finished."""
    if stream is None or stream == torch.cuda.current_stream():
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def _workspace(nbytes, device):
    if nbytes == 0:
        return None
    return torch.empty(int(nbytes), dtype=torch.uint8, device=device)


def version():
    return _lib.load().csa_version()


# ------------------------------------------------------------------ a2 ----

def csa_quantize(e, codes=None, scales=None, stream=None):
    """e float32 [n, 512] -> (codes uint8 [n, 256], scales uint8 [n, 32])."""
    _need(e, "e", torch.float32)
    n = e.numel() // D
    if e.shape[-1] != D:
        raise ValueError("e must end in 512 channels")
    codes = codes if codes is not None else torch.empty((n, D // 2), dtype=torch.uint8, device=e.device)
    scales = scales if scales is not None else torch.empty((n, D // 16), dtype=torch.uint8, device=e.device)
    _need(codes, "codes", torch.uint8, e.device)
    _need(scales, "scales", torch.uint8, e.device)
    if codes.numel() != n * (D // 2) or scales.numel() != n * (D // 16):
        raise ValueError("codes / scales sizes do not match e")
    _call("csa_quantize", _p(e), n, _p(codes), _p(scales), _stream(stream))
    _keep(stream, codes, scales)
    return codes, scales


def csa_dequantize(codes, scales, out=None, stream=None):
    _need(codes, "codes", torch.uint8)
    _need(scales, "scales", torch.uint8, codes.device)
    n = codes.numel() // (D // 2)
    if scales.numel() != n * (D // 16):
        raise ValueError("scales size does not match codes")
    out = out if out is not None else torch.empty((n, D), dtype=torch.float32, device=codes.device)
    _need(out, "out", torch.float32, codes.device)
    _call("csa_dequantize", _p(codes), _p(scales), n, _p(out), _stream(stream))
    _keep(stream, out)
    return out


# ------------------------------------------------------------- a1 + a2 ----

def _ptr_off(t, offset):
    return ctypes.c_void_p(t.data_ptr() + int(offset) * t.element_size())


def _compress_args(x, w, rope_cs, codes, scales, n_seq, n_per_seq, x_seq_stride, out_seq_stride, x_offset,
                   out_offset, rope_dim, eps, e_out):
    """Checks and C arguments (with the workspace) of a compression call."""
    _need(x, "x", torch.float32)
    dev = x.device
    _need(w, "w", torch.float32, dev, shape=(4, D, D))
    _need(codes, "codes", torch.uint8, dev)
    _need(scales, "scales", torch.uint8, dev)
    n = n_seq * n_per_seq
    xs = x_seq_stride if x_seq_stride is not None else n_per_seq * 4 * D
    os_ = out_seq_stride if out_seq_stride is not None else n_per_seq
    if n > 0:
        if x_offset < 0 or x_offset + (n_seq - 1) * xs + n_per_seq * 4 * D > x.numel():
            raise ValueError("x is too small for the requested entries")
        rows = out_offset + (n_seq - 1) * os_ + n_per_seq
        if out_offset < 0 or codes.numel() < rows * (D // 2) or scales.numel() < rows * (D // 16):
            raise ValueError("codes / scales are too small for the requested rows")
    if rope_dim:
        _need(rope_cs, "rope_cs", torch.float32, dev)
        if rope_cs.numel() != n * rope_dim:
            raise ValueError("rope_cs must hold [n_seq, n_per_seq, rope_dim/2, 2] floats")
    if e_out is not None:
        _need(e_out, "e_out", torch.float32, dev)
        if e_out.numel() != n * D:
            raise ValueError("e_out must hold [n, 512] floats")
    ws = _workspace(_lib.load().csa_compress_quant_workspace_size(n), dev)
    args = (_ptr_off(x, x_offset), n_seq, n_per_seq, xs, _p(w),
            _p(rope_cs) if rope_dim else None, rope_dim, ctypes.c_float(eps),
            _ptr_off(codes, out_offset * (D // 2)), _ptr_off(scales, out_offset * (D // 16)), os_,
            _p(e_out), _p(ws), 0 if ws is None else ws.numel())
    return args, ws


def csa_compress_quant(x, w, rope_cs, codes, scales, n_seq, n_per_seq, x_seq_stride=None,
                       out_seq_stride=None, x_offset=0, out_offset=0, rope_dim=64, eps=1e-6,
                       e_out=None, stream=None):
    """Compress 4-token groups, RMSNorm, RoPE, quantize and store into codes/scales.

    x: contiguous float32 tensor; entry (s, r) reads its 4 tokens at element
    x_offset + s * x_seq_stride + r * 2048.  codes / scales: contiguous uint8
    tensors of 256- / 32-byte rows; entry (s, r) goes to row
    out_offset + s * out_seq_stride + r.  rope_cs: float32
    [n_seq, n_per_seq, rope_dim / 2, 2].
    """
    args, ws = _compress_args(x, w, rope_cs, codes, scales, n_seq, n_per_seq, x_seq_stride, out_seq_stride,
                              x_offset, out_offset, rope_dim, eps, e_out)
    _call("csa_compress_quant", *args, _stream(stream))
    _keep(stream, ws)


def csa_compress_quant_append(x, w, rope_cs, codes, scales, n_seq, n_per_seq, xw, pos0, win, nw_seq, nw_tok,
                              x_seq_stride=None, out_seq_stride=None, x_offset=0, out_offset=0, rope_dim=64,
                              eps=1e-6, e_out=None, xw_seq_stride=None, xw_offset=0, stream=None):
    """csa_compress_quant(x, ...) and csa_window_append(xw, pos0, win, nw_seq,
    nw_tok, ...) in one call (two launches instead of three); arguments as in
    those two functions."""
    args, ws = _compress_args(x, w, rope_cs, codes, scales, n_seq, n_per_seq, x_seq_stride, out_seq_stride,
                              x_offset, out_offset, rope_dim, eps, e_out)
    wargs = _append_args(xw, pos0, win, nw_seq, nw_tok, xw_seq_stride, xw_offset)
    _call("csa_compress_quant_append", *args, *wargs, _stream(stream))
    _keep(stream, ws)


# ------------------------------------------------------------------ a9 ----

def csa_window_append(x, pos0, win, n_seq, n_tok, x_seq_stride=None, x_offset=0, stream=None):
    """Append n_tok float32 tokens per sequence to the E4M3 window ring win [S, cap, 512].

    Token t of sequence s is read at element x_offset + s * x_seq_stride + t * 512
    and lands in row (pos0[s] + t) % cap.
    """
    _call("csa_window_append", *_append_args(x, pos0, win, n_seq, n_tok, x_seq_stride, x_offset), _stream(stream))


def _append_args(x, pos0, win, n_seq, n_tok, x_seq_stride, x_offset):
    """Checks and C arguments of a window append."""
    _need(x, "x", torch.float32)
    dev = x.device
    _need(pos0, "pos0", torch.int32, dev, shape=(n_seq,))
    _need(win, "win", torch.uint8, dev)
    if win.dim() != 3 or win.shape[0] != n_seq or win.shape[2] != D:
        raise ValueError("win must be [n_seq, win_cap, 512]")
    xs = x_seq_stride if x_seq_stride is not None else n_tok * D
    if n_seq * n_tok and (x_offset < 0 or x_offset + (n_seq - 1) * xs + n_tok * D > x.numel()):
        raise ValueError("x is too small")
    return (_ptr_off(x, x_offset), n_seq, n_tok, xs, _p(pos0), _p(win), win.shape[1])


def csa_window_rebuild(x, p_last, win, n_ring, n_tok, x_ring_stride=None, x_offset=0, stream=None):
    """Rebuild n_ring E4M3 window rings win [n_ring, cap, 512] from their last
    n_tok float32 tokens (token i of ring r at element x_offset + r *
    x_ring_stride + i * 512, the last one at position p_last[r])."""
    _need(x, "x", torch.float32)
    dev = x.device
    _need(p_last, "p_last", torch.int32, dev, shape=(n_ring,))
    _need(win, "win", torch.uint8, dev)
    if win.dim() != 3 or win.shape[0] != n_ring or win.shape[2] != D:
        raise ValueError("win must be [n_ring, win_cap, 512]")
    xs = x_ring_stride if x_ring_stride is not None else n_tok * D
    if n_ring and (x_offset < 0 or x_offset + (n_ring - 1) * xs + n_tok * D > x.numel()):
        raise ValueError("x is too small")
    _call("csa_window_rebuild", _ptr_off(x, x_offset), n_ring, n_tok, xs, _p(p_last), _p(win), win.shape[1],
          _stream(stream))


# ------------------------------------------------------------------ f4 ----

KV_STAGE_BYTES = 64 << 20


def kv_stage(nbytes=KV_STAGE_BYTES):
    """A pinned host staging buffer for csa_kv_save / csa_kv_load."""
    return torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)


def _kv_bufs(codes, scales, k_fp8):
    _need(codes, "codes", torch.uint8)
    dev = codes.device
    S, rows = codes.shape[0], codes.shape[1]
    _need(codes, "codes", torch.uint8, dev, shape=(S, rows, D // 2))
    _need(scales, "scales", torch.uint8, dev, shape=(S, rows, D // 16))
    _need(k_fp8, "k_fp8", torch.uint8, dev, shape=(S, rows, IDX_DIM))
    return S, rows


def csa_kv_save(path, codes, scales, k_fp8, n_entries, stage=None, stream=None):
    """Write the first n_entries rows of every sequence's global KV to path."""
    S, rows = _kv_bufs(codes, scales, k_fp8)
    stage = kv_stage() if stage is None else stage
    _call("csa_kv_save", os.fsencode(path), _p(codes), _p(scales), _p(k_fp8), S, rows, n_entries,
          ctypes.c_void_p(stage.data_ptr()), stage.numel(), _stream(stream))


def csa_kv_load(path, codes, scales, k_fp8, stage=None, stream=None):
    """Read a global-KV file into the buffers; returns its n_entries."""
    S, rows = _kv_bufs(codes, scales, k_fp8)
    stage = kv_stage() if stage is None else stage
    n = ctypes.c_int64(0)
    _call("csa_kv_load", os.fsencode(path), _p(codes), _p(scales), _p(k_fp8), S, rows, ctypes.byref(n),
          ctypes.c_void_p(stage.data_ptr()), stage.numel(), _stream(stream))
    return n.value


def csa_kv_file_info(path):
    """(n_seq, n_entries) of a global-KV file (header and size checked)."""
    a, b = ctypes.c_int64(0), ctypes.c_int64(0)
    _call("csa_kv_file_info", os.fsencode(path), ctypes.byref(a), ctypes.byref(b))
    return a.value, b.value


# ------------------------------------------------------------------ a3 ----

def csa_index_score(q_fp8, w, q_pos, k_fp8, n_seq, q_per_seq, n_entries, pool_blocks=None,
                    want_scores=True, want_block_max=False, stream=None):
    """Indexer scores.  Returns (scores or None, block_max or None)."""
    dev = q_fp8.device
    Q = n_seq * q_per_seq
    _need(q_fp8, "q_fp8", torch.uint8, dev, shape=(Q, IDX_HEADS, IDX_DIM))
    _need(w, "w", torch.float32, dev, shape=(Q, IDX_HEADS))
    _need(q_pos, "q_pos", torch.int32, dev, shape=(Q,))
    _need(k_fp8, "k_fp8", torch.uint8, dev)
    if k_fp8.dim() != 3 or k_fp8.shape[0] != n_seq or k_fp8.shape[2] != IDX_DIM:
        raise ValueError("k_fp8 must be [n_seq, k_rows, 128]")
    nb = 0
    if pool_blocks is not None:
        _need(pool_blocks, "pool_blocks", torch.int32, dev)
        if pool_blocks.dim() != 2 or pool_blocks.shape[0] != Q:
            raise ValueError("pool_blocks must be [Q, n_pool_blocks]")
        nb = pool_blocks.shape[1]
        ncols = BLOCK * nb
    else:
        ncols = n_entries
    scores = torch.empty((Q, ncols), dtype=torch.float32, device=dev) if want_scores else None
    bm = None
    if want_block_max:
        bm = torch.empty((Q, (ncols + 7) // 8), dtype=torch.float32, device=dev)
    _call("csa_index_score", _p(q_fp8), _p(w), _p(q_pos), n_seq, q_per_seq, _p(k_fp8), k_fp8.shape[1],
          n_entries, _p(pool_blocks), nb, _p(scores), _p(bm), _stream(stream))
    _keep(stream, scores, bm)
    return scores, bm


# ------------------------------------------------------------------ a4 ----

def csa_topk(scores, k=TOP_K, col_blocks=None, idx=None, stream=None):
    _need(scores, "scores", torch.float32)
    dev = scores.device
    Q, ncols = scores.shape
    if col_blocks is not None:
        _need(col_blocks, "col_blocks", torch.int32, dev, shape=(Q, ncols // 8))
    idx = idx if idx is not None else torch.empty((Q, k), dtype=torch.int32, device=dev)
    _need(idx, "idx", torch.int32, dev, shape=(Q, k))
    ws = _workspace(_lib.load().csa_topk_workspace_size(Q, ncols, k), dev)
    _call("csa_topk", _p(scores), Q, ncols, _p(col_blocks), k, _p(idx), _p(ws),
          0 if ws is None else ws.numel(), _stream(stream))
    _keep(stream, ws, idx)
    return idx


# ------------------------------------------------------------------ a5 ----

def csa_block_pool(values, is_block_max=True, n_pool_blocks=POOL_BLOCKS, out=None, stream=None):
    _need(values, "values", torch.float32)
    dev = values.device
    Q, ncols = values.shape
    out = out if out is not None else torch.empty((Q, n_pool_blocks), dtype=torch.int32, device=dev)
    _need(out, "pool_blocks", torch.int32, dev, shape=(Q, n_pool_blocks))
    ws = _workspace(_lib.load().csa_block_pool_workspace_size(Q, ncols, int(is_block_max), n_pool_blocks),
                    dev)
    _call("csa_block_pool", _p(values), int(is_block_max), Q, ncols, n_pool_blocks, _p(out), _p(ws),
          0 if ws is None else ws.numel(), _stream(stream))
    _keep(stream, ws, out)
    return out


# ------------------------------------------------------------------ a7 ----

def csa_sparse_attn(q, q_pos, codes, scales, idx, win, n_seq, q_per_seq, sm_scale=None, out=None,
                    stream=None):
    """q float32 [Q, 16, 512]; codes [S, rows, 256]; scales [S, rows, 32]; idx int32 [Q, k];
    win uint8 [S, cap, 512].  Returns out float32 [Q, 16, 512]."""
    dev = q.device
    Q = n_seq * q_per_seq
    _need(q, "q", torch.float32, dev, shape=(Q, HEADS, D))
    _need(q_pos, "q_pos", torch.int32, dev, shape=(Q,))
    _need(codes, "codes", torch.uint8, dev)
    _need(scales, "scales", torch.uint8, dev)
    if codes.dim() != 3 or codes.shape[0] != n_seq or codes.shape[2] != D // 2:
        raise ValueError("codes must be [n_seq, rows, 256]")
    if tuple(scales.shape) != (n_seq, codes.shape[1], D // 16):
        raise ValueError("scales must be [n_seq, rows, 32]")
    _need(idx, "idx", torch.int32, dev)
    if idx.dim() != 2 or idx.shape[0] != Q:
        raise ValueError("idx must be [Q, k]")
    _need(win, "win", torch.uint8, dev)
    if win.dim() != 3 or win.shape[0] != n_seq or win.shape[2] != D:
        raise ValueError("win must be [n_seq, cap, 512]")
    k = idx.shape[1]
    sm = sm_scale if sm_scale is not None else 1.0 / math.sqrt(D)
    out = out if out is not None else torch.empty((Q, HEADS, D), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, dev, shape=(Q, HEADS, D))
    ws = _workspace(_lib.load().csa_sparse_attn_workspace_size(Q, k), dev)
    _call("csa_sparse_attn", _p(q), _p(q_pos), n_seq, q_per_seq, _p(codes), _p(scales), codes.shape[1],
          _p(idx), k, _p(win), win.shape[1], ctypes.c_float(sm), _p(out), _p(ws),
          0 if ws is None else ws.numel(), _stream(stream))
    _keep(stream, ws, out)
    return out


def csa_sparse_attn_noalloc(q, q_pos, codes, scales, idx, win, n_seq, q_per_seq, out, sm_scale=None,
                            stream=None):
    """csa_sparse_attn without a workspace: the library's static device scratch
    holds the split partials (no allocation by the library or here; ``out``
    is the caller's).  Calls that overlap on one GPU race."""
    dev = q.device
    Q = n_seq * q_per_seq
    _need(q, "q", torch.float32, dev, shape=(Q, HEADS, D))
    _need(q_pos, "q_pos", torch.int32, dev, shape=(Q,))
    _need(codes, "codes", torch.uint8, dev)
    _need(scales, "scales", torch.uint8, dev)
    if codes.dim() != 3 or codes.shape[0] != n_seq or codes.shape[2] != D // 2:
        raise ValueError("codes must be [n_seq, rows, 256]")
    if tuple(scales.shape) != (n_seq, codes.shape[1], D // 16):
        raise ValueError("scales must be [n_seq, rows, 32]")
    _need(idx, "idx", torch.int32, dev)
    if idx.dim() != 2 or idx.shape[0] != Q:
        raise ValueError("idx must be [Q, k]")
    _need(win, "win", torch.uint8, dev)
    if win.dim() != 3 or win.shape[0] != n_seq or win.shape[2] != D:
        raise ValueError("win must be [n_seq, cap, 512]")
    _need(out, "out", torch.float32, dev, shape=(Q, HEADS, D))
    sm = sm_scale if sm_scale is not None else 1.0 / math.sqrt(D)
    _call("csa_sparse_attn_noalloc", _p(q), _p(q_pos), n_seq, q_per_seq, _p(codes), _p(scales), codes.shape[1],
          _p(idx), idx.shape[1], _p(win), win.shape[1], ctypes.c_float(sm), _p(out), _stream(stream))
    return out


# ------------------------------------------------------------- a6 + a8 ----

class LayerCall:
    """A prepared layer call: argument struct + workspace, reusable across steps."""

    def __init__(self, mode, *, codes, scales, k_fp8, win, q_pos, q_attn, idx, out, n_seq, q_per_seq,
                 n_entries, q_idx=None, w_idx=None, pool_blocks=None, build_pool=False,
                 top_k=TOP_K, n_pool_blocks=POOL_BLOCKS, sm_scale=None, ws=None, alloc_ws=True):
        dev = codes.device
        Q = n_seq * q_per_seq
        _need(codes, "codes", torch.uint8, dev)
        _need(scales, "scales", torch.uint8, dev)
        _need(win, "win", torch.uint8, dev)
        _need(q_pos, "q_pos", torch.int32, dev, shape=(Q,))
        _need(q_attn, "q_attn", torch.float32, dev, shape=(Q, HEADS, D))
        _need(idx, "idx", torch.int32, dev, shape=(Q, top_k))
        _need(out, "out", torch.float32, dev, shape=(Q, HEADS, D))
        if codes.dim() != 3 or codes.shape[0] != n_seq or codes.shape[2] != D // 2:
            raise ValueError("codes must be [n_seq, rows, 256]")
        if tuple(scales.shape) != (n_seq, codes.shape[1], D // 16):
            raise ValueError("scales must be [n_seq, rows, 32]")
        if win.dim() != 3 or win.shape[0] != n_seq or win.shape[2] != D:
            raise ValueError("win must be [n_seq, cap, 512]")
        k_rows = 0
        if mode != MODE_REUSE:
            _need(k_fp8, "k_fp8", torch.uint8, dev)
            if k_fp8.dim() != 3 or k_fp8.shape[0] != n_seq or k_fp8.shape[2] != IDX_DIM:
                raise ValueError("k_fp8 must be [n_seq, rows, 128]")
            k_rows = k_fp8.shape[1]
            _need(q_idx, "q_idx", torch.uint8, dev, shape=(Q, IDX_HEADS, IDX_DIM))
            _need(w_idx, "w_idx", torch.float32, dev, shape=(Q, IDX_HEADS))
        if pool_blocks is not None:
            _need(pool_blocks, "pool_blocks", torch.int32, dev, shape=(Q, n_pool_blocks))
        self.mode = mode
        self.keep = [codes, scales, k_fp8, win, q_pos, q_attn, idx, out, q_idx, w_idx, pool_blocks]
        a = CsaLayerArgs()
        a.codes, a.scales, a.kv_rows = _p(codes), _p(scales), codes.shape[1]
        a.k_fp8, a.k_rows, a.n_entries = _p(k_fp8), k_rows, n_entries
        a.win, a.win_cap = _p(win), win.shape[1]
        a.n_seq, a.q_per_seq = n_seq, q_per_seq
        a.q_pos, a.q_attn, a.q_idx, a.w_idx = _p(q_pos), _p(q_attn), _p(q_idx), _p(w_idx)
        a.sm_scale = sm_scale if sm_scale is not None else 1.0 / math.sqrt(D)
        a.top_k, a.build_pool, a.n_pool_blocks = top_k, int(build_pool), n_pool_blocks
        a.pool_blocks, a.idx, a.out = _p(pool_blocks), _p(idx), _p(out)
        self.ws_need = _lib.load().csa_layer_workspace_size(mode, ctypes.byref(a))
        self.args = a
        self.ws = None
        if ws is None and alloc_ws:
            ws = _workspace(self.ws_need, dev)
        if ws is not None or alloc_ws:
            self.set_workspace(ws)

    def set_workspace(self, ws):
        """Use ``ws`` (uint8 tensor of at least ``ws_need`` bytes, or None when none is needed)."""
        if self.ws_need and (ws is None or ws.numel() < self.ws_need):
            raise ValueError(f"layer workspace needs {self.ws_need} bytes")
        self.ws = ws
        self.args.ws = None if ws is None else ws.data_ptr()
        self.args.ws_bytes = 0 if ws is None else ws.numel()

    def set_attn_after(self, event):
        """Make the layer's attention (not its scoring and selection) wait for
        ``event`` (a torch.cuda.Event recorded on another stream), or for
        nothing with None.  The event object is kept alive with the call.  An
        event gets its HIP handle when first recorded, so record it first."""
        if event is not None and not event.cuda_event:
            raise ValueError("attn_after: record the event before passing it")
        self.attn_event = event
        self.args.attn_after = None if event is None else ctypes.c_void_p(event.cuda_event)

    def __call__(self, stream=None):
        name = {MODE_FULL: "csa_layer_full", MODE_REINDEX: "csa_layer_reindex",
                MODE_REUSE: "csa_layer_reuse"}[self.mode]
        _call(name, ctypes.byref(self.args), _stream(stream))
        _keep(stream, self.ws)


def csa_layer_full(**kw):
    stream = kw.pop("stream", None)
    LayerCall(MODE_FULL, **kw)(stream)


def csa_layer_reindex(**kw):
    stream = kw.pop("stream", None)
    LayerCall(MODE_REINDEX, **kw)(stream)


def csa_layer_reuse(**kw):
    stream = kw.pop("stream", None)
    LayerCall(MODE_REUSE, **kw)(stream)
