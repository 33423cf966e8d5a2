"""Shared helpers of the GPU parity tests: the oracle side of a whole layer
step (numpy float64, from the same seeded inputs) and the comparison rules.

Comparison rules (the method's tolerances):
  * quantized bytes, pool membership, window bytes: bit-exact on identical inputs;
  * Top-K id sets: exact, except ids whose oracle score lies within
    1e-5 * max(1, |s_K|) of the oracle's K-th score s_K;
  * attention output: |o_gpu - o_ref| <= 1e-3 * max(1, |o_ref|) per element.
"""

import numpy as np
import torch

import oracle
from oracle import formats, mxfp4

TOPK_REL = 1e-5
ATTN_TOL = 1e-3
SM = 512 ** -0.5


def has_gpu():
    return torch.cuda.is_available()


def np_(t):
    return t.detach().cpu().numpy()


def check_topk_set(gpu_ids, ref_scores, ref_ids, k, ids=None):
    """GPU ids vs the oracle's Top-K; returns the number of near-tie swaps."""
    gpu = set(int(v) for v in gpu_ids if v >= 0)
    ref = set(int(v) for v in ref_ids if v >= 0)
    assert len(gpu) == len(ref), (len(gpu), len(ref))
    diff = gpu ^ ref
    if not diff:
        return 0
    ids = np.arange(len(ref_scores)) if ids is None else np.asarray(ids)
    pos = {int(e): i for i, e in enumerate(ids)}
    order = np.lexsort((ids, -ref_scores))
    s_k = ref_scores[order[min(k, len(order)) - 1]]
    tol = TOPK_REL * max(1.0, abs(s_k))
    for e in diff:
        assert abs(ref_scores[pos[e]] - s_k) <= tol, (e, ref_scores[pos[e]], s_k)
    return len(diff) // 2


def check_attn(gpu_out, ref_out):
    ref = np.asarray(ref_out, dtype=np.float64)
    err = np.abs(np.asarray(gpu_out, dtype=np.float64) - ref)
    bound = ATTN_TOL * np.maximum(1.0, np.abs(ref))
    worst = float((err / bound).max())
    assert worst <= 1.0, f"attention error {worst:.3f} x tolerance (max abs {err.max():.3e})"
    return float(err.max())


class OracleStep:
    """The oracle's version of one step of a workload, built lazily per sequence."""

    def __init__(self, wl):
        self.wl = wl
        self.cfg = wl.cfg
        t = wl.tensors
        self.w = np_(t["w"]).astype(np.float64)
        self._cache = {}

    def cache(self, s):
        """(codes, scales, k_fp8, x_tail) of sequence s after the step's compression."""
        if s in self._cache:
            return self._cache[s]
        cfg, t = self.cfg, self.wl.tensors
        prior, new = cfg.prior_entries, cfg.new_entries
        codes = np_(t["codes"][s]).copy()
        scales = np_(t["scales"][s]).copy()
        if not cfg.synthetic_cache and prior > 0:
            e32 = oracle.compress_rope_fp32(np_(t["x_prior"][s]), self.w, np_(t["rope_prior"][s]), 64, 1e-6)
            codes[:prior], scales[:prior] = mxfp4.quantize(e32)
        x_tail = np_(t["x_tail"][s])
        toks = x_tail[x_tail.shape[0] - 4 * new:]
        e32 = oracle.compress_rope_fp32(toks, self.w, np_(t["rope_cs"][s]), 64, 1e-6)
        codes[prior:prior + new], scales[prior:prior + new] = mxfp4.quantize(e32)
        k_fp8 = np_(t["k_fp8"][s])
        self._cache[s] = (codes, scales, k_fp8, x_tail)
        return self._cache[s]

    def window(self, s, p):
        """E4M3 bytes of the window tokens of a query at position p."""
        cfg = self.cfg
        x_tail = self.cache(s)[3]
        first = (cfg.ctx_tokens - 128) if cfg.kind == "decode" else (cfg.ctx_tokens - 127)
        pos = oracle.window_positions(p)
        return oracle.window_encode(x_tail[pos - first])

    def query(self, qi):
        """Per-layer oracle results for query qi: list of LayerState."""
        cfg, t = self.cfg, self.wl.tensors
        s = qi // cfg.chunk
        p = int(t["q_pos"][qi])
        codes, scales, k_fp8, _ = self.cache(s)
        win = self.window(s, p)
        n_entries = cfg.entries_total
        res, idx, pool = [], None, None
        for li, mode in enumerate(cfg.layers):
            qa = np_(t["q_attn"][li][qi])
            if mode == "F":
                st = oracle.layer_full(codes, scales, k_fp8, np_(t["q_fp8"][li][qi]),
                                       np_(t["w_idx"][li][qi]), qa, p, win, SM,
                                       build_pool=cfg.build_pool, n_entries=n_entries)
                pool = st.pool
            elif mode == "I":
                st = oracle.layer_reindex(codes, scales, k_fp8, pool, np_(t["q_fp8"][li][qi]),
                                          np_(t["w_idx"][li][qi]), qa, p, win, SM, n_entries=n_entries)
            else:
                st = oracle.layer_reuse(codes, scales, idx, qa, win, SM)
            idx = st.idx
            res.append(st)
        return res
