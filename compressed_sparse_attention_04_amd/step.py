"""One CSA2 layer-group step driven through the C ABI.

A step, in order ("DeepSeek-V4.1 架构解析" §02 layer modes; "DeepSeek-V4.1 架构解析" §03 window / MXFP4 store):
  1. append the step's tokens to the FP8 window ring (a9);
  2. compress + RoPE + MXFP4-store the entries the step's tokens complete (a1, a2);
  3. run the layer group: Full (score, Top-K, optional pool), then Reuse and
     Reindex layers in their static order (a3..a8).
``setup()`` fills the state that exists before the step (prior entries when
they are built from token latents, and the 127 window tokens before the
step's first token); it is not part of the timed work.

Steps 1-2 write only what attention reads (the new cache rows and the
window), not the indexer keys, so they can run on a second stream beside the
first layer's scoring and selection, with that layer's attention waiting for
them (``overlap_compress``); every result is the same as in order.  Prefill
steps do so by default: a captured step then takes ~1-3 % less (the
compression hides under the dense scoring).  Decode steps do not: with the
fork and join in the graph a decode step measured 6-12 us slower (4K, 128K
and 1M contexts), more than the compression it hides.

A schedule (``ScheduleStep``) runs several groups in order, each with its own
global KV; a decode token passes through every group ("DeepSeek-V4.1 架构解析" §01, §02).
"""

import math

import torch

from . import ops
from .ops import D, HEADS, LayerCall, MODE_FULL, MODE_REINDEX, MODE_REUSE

M = 4
N_WIN = 128


class LayerStep:
    """State and prepared calls of one step.

    kind: "decode" (one query per sequence at position q_pos, the last token)
    or "prefill" (q_per_seq queries at consecutive positions).
    x_tail: float32 [S, 127 + n_step, 512] -- the 127 tokens before the step
    and the step's n_step tokens.  The last 4 * new_entries rows of x_tail are
    compressed into entries prior_entries .. prior_entries + new_entries - 1.
    x_win: optional float32 [L, S, 127 + n_step, 512] -- every layer's own
    window latents (laid out like x_tail); without it the group's layers
    share one window built from x_tail.
    """

    def __init__(self, *, kind, layers, build_pool, x_tail, w, rope_cs, codes, scales, k_fp8, q_pos,
                 q_attn, q_fp8, w_idx, prior_entries, new_entries, first_pos, x_prior=None,
                 rope_prior=None, top_k=ops.TOP_K, n_pool_blocks=ops.POOL_BLOCKS, rope_dim=64,
                 eps=1e-6, x_win=None, overlap_compress=None):
        dev = codes.device
        S, cap = codes.shape[0], codes.shape[1]
        self.kind, self.layers = kind, list(layers)
        self.S, self.cap = S, cap
        self.n_step = x_tail.shape[1] - (N_WIN - 1)
        self.q_per_seq = 1 if kind == "decode" else self.n_step
        self.Q = S * self.q_per_seq
        self.prior, self.new = prior_entries, new_entries
        self.x_tail, self.w, self.rope_cs = x_tail, w, rope_cs
        self.x_prior, self.rope_prior = x_prior, rope_prior
        self.codes, self.scales, self.k_fp8 = codes, scales, k_fp8
        self.rope_dim, self.eps = rope_dim, eps
        self.win_cap = N_WIN if kind == "decode" else self.n_step + N_WIN
        L = len(self.layers)
        # windows: one per layer ([L * S] rings appended in one call), or one per group
        self.x_win = x_win
        self.n_win = L if x_win is not None else 1
        if x_win is not None and tuple(x_win.shape) != (L, S, x_tail.shape[1], D):
            raise ValueError("x_win must be [layers, sequences, 127 + n_step, 512]")
        self.win_all = torch.zeros((self.n_win, S, self.win_cap, D), dtype=torch.uint8, device=dev)
        self.wins = [self.win_all[li if x_win is not None else 0] for li in range(L)]
        self.win = self.wins[0]
        # position of x_tail row 0 of every sequence (repeated for every window)
        self.pos_tail = first_pos.to(torch.int32).repeat(self.n_win).contiguous()
        self.pos_step = (first_pos + (N_WIN - 1)).to(torch.int32).repeat(self.n_win).contiguous()
        self.n_entries = prior_entries + new_entries
        self.outs, self.idxs, self.calls = [], [], []
        self.pool = None
        if build_pool:
            self.pool = torch.empty((self.Q, n_pool_blocks), dtype=torch.int32, device=dev)
        idx_latest = None
        for li, mode in enumerate(self.layers):
            out = torch.empty((self.Q, HEADS, D), dtype=torch.float32, device=dev)
            common = dict(codes=codes, scales=scales, k_fp8=k_fp8, win=self.wins[li], q_pos=q_pos,
                          q_attn=q_attn[li], out=out, n_seq=S, q_per_seq=self.q_per_seq,
                          n_entries=self.n_entries, top_k=top_k, n_pool_blocks=n_pool_blocks,
                          alloc_ws=False)
            if mode == "F":
                idx = torch.empty((self.Q, top_k), dtype=torch.int32, device=dev)
                call = LayerCall(MODE_FULL, idx=idx, q_idx=q_fp8[li], w_idx=w_idx[li],
                                 pool_blocks=self.pool, build_pool=build_pool, **common)
                idx_latest = idx
            elif mode == "I":
                idx = torch.empty((self.Q, top_k), dtype=torch.int32, device=dev)
                call = LayerCall(MODE_REINDEX, idx=idx, q_idx=q_fp8[li], w_idx=w_idx[li],
                                 pool_blocks=self.pool, **common)
                idx_latest = idx
            elif mode == "U":
                if idx_latest is None:
                    raise ValueError("a Reuse layer needs an earlier Full or Reindex layer")
                idx = idx_latest
                call = LayerCall(MODE_REUSE, idx=idx, **common)
            else:
                raise ValueError(f"unknown layer mode {mode!r}")
            self.outs.append(out)
            self.idxs.append(idx)
            self.calls.append(call)
        # every layer call runs on the same stream in order, so one workspace
        # serves all (the compression on the side stream allocates its own)
        big = max((c.ws_need for c in self.calls), default=0)
        self.ws = torch.empty(big, dtype=torch.uint8, device=dev) if big else None
        for c in self.calls:
            c.set_workspace(self.ws)
        if overlap_compress is None:
            overlap_compress = kind == "prefill"
        self.overlap = bool(overlap_compress) and len(self.calls) > 0
        if self.overlap:
            self.side = torch.cuda.Stream(device=dev)   # default priority
            self.ev_fork = torch.cuda.Event()
            self.ev_join = torch.cuda.Event()

    def setup(self):
        """Untimed: prior entries (from token latents) and the first 127 window tokens."""
        if self.x_prior is not None and self.prior > 0:
            ops.csa_compress_quant(self.x_prior, self.w, self.rope_prior, self.codes, self.scales,
                                   n_seq=self.S, n_per_seq=self.prior,
                                   x_seq_stride=self.x_prior.shape[1] * D, out_seq_stride=self.cap,
                                   rope_dim=self.rope_dim, eps=self.eps)
        tail = self.x_tail.shape[1]
        ops.csa_window_append(self._win_src(), self.pos_tail, self._win_rings(), self.n_win * self.S, N_WIN - 1,
                              x_seq_stride=tail * D)

    def _win_src(self):
        return self.x_tail if self.x_win is None else self.x_win

    def _win_rings(self):
        return self.win_all.view(self.n_win * self.S, self.win_cap, D)

    def step(self):
        if not self.overlap:
            self._compress()
        else:
            main = torch.cuda.current_stream()
            self.ev_fork.record(main)
            self.side.wait_event(self.ev_fork)
            with torch.cuda.stream(self.side):
                self._compress()
            self.ev_join.record(self.side)
            # (an event has its handle once recorded) the first call's attention
            # waits for ev_join; every later call follows it on this stream
            self.calls[0].set_attn_after(self.ev_join)
        for call in self.calls:
            call()

    def _compress(self):
        tail = self.x_tail.shape[1]
        ops.csa_compress_quant_append(self.x_tail, self.w, self.rope_cs, self.codes, self.scales,
                                      n_seq=self.S, n_per_seq=self.new, xw=self._win_src(), pos0=self.pos_step,
                                      win=self._win_rings(), nw_seq=self.n_win * self.S, nw_tok=self.n_step,
                                      x_seq_stride=tail * D, x_offset=(tail - M * self.new) * D,
                                      out_seq_stride=self.cap, out_offset=self.prior, rope_dim=self.rope_dim,
                                      eps=self.eps, xw_seq_stride=tail * D, xw_offset=(N_WIN - 1) * D)


def from_workload(wl, device=None, overlap_compress=None):
    """LayerStep for a workload object with ``cfg`` and ``tensors`` (see workloads)."""
    cfg, t = wl.cfg, wl.tensors
    dev = device or t["codes"].device
    S = cfg.n_seq
    if cfg.kind == "decode":
        first = torch.full((S,), cfg.ctx_tokens - N_WIN, dtype=torch.int32, device=dev)
    else:
        first = torch.full((S,), cfg.ctx_tokens - (N_WIN - 1), dtype=torch.int32, device=dev)
    return LayerStep(kind=cfg.kind, layers=cfg.layers, build_pool=cfg.build_pool, x_tail=t["x_tail"],
                     w=t["w"], rope_cs=t["rope_cs"], codes=t["codes"], scales=t["scales"],
                     k_fp8=t["k_fp8"], q_pos=t["q_pos"], q_attn=t["q_attn"], q_fp8=t["q_fp8"],
                     w_idx=t["w_idx"], prior_entries=cfg.prior_entries, new_entries=cfg.new_entries,
                     first_pos=first, x_prior=t.get("x_prior"), rope_prior=t.get("rope_prior"),
                     x_win=t.get("x_win"), overlap_compress=overlap_compress)


class ScheduleStep:
    """Groups of layers run in order on one stream ("DeepSeek-V4.1 架构解析" §02 schedule); every
    group is a LayerStep with its own global KV.  One workspace serves all."""

    def __init__(self, groups):
        self.groups = list(groups)
        big = max((c.ws_need for g in self.groups for c in g.calls), default=0)
        dev = self.groups[0].codes.device
        self.ws = torch.empty(big, dtype=torch.uint8, device=dev) if big else None
        for g in self.groups:
            g.ws = self.ws
            for c in g.calls:
                c.set_workspace(self.ws)

    def setup(self):
        for g in self.groups:
            g.setup()

    def step(self):
        for g in self.groups:
            g.step()


def from_schedule(wls, device=None):
    """ScheduleStep for a list of group workloads."""
    return ScheduleStep([from_workload(wl, device) for wl in wls])
