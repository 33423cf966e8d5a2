"""The oracle's version of one layer-group step of a seeded workload.

TEST INFRASTRUCTURE ONLY (see the package header).  It reads the workload's
input tensors (copying one sequence at a time to the host) and runs the
oracle functions of this package on them; nothing here touches the GPU path.
"""

import numpy as np

from .attention import sparse_attention, window_positions
from .compressor import compress, rope_rotate
from .formats import e4m3_decode
from .indexer import index_scores_many, visible_entries
from .layer import layer_full, layer_reindex, layer_reuse, window_encode
from .mxfp4 import quantize

SM = 512 ** -0.5


def _np(t):
    return t.detach().cpu().numpy() if hasattr(t, "detach") else np.asarray(t)


class OracleStep:
    """The oracle's version of one step of a workload, built lazily per sequence."""

    def __init__(self, wl):
        self.wl = wl
        self.cfg = wl.cfg
        t = wl.tensors
        self.w = _np(t["w"]).astype(np.float64)
        self._cache = {}

    def cache(self, s):
        """(codes, scales, k_fp8, x_tail) of sequence s after the step's compression."""
        if s in self._cache:
            return self._cache[s]
        cfg, t = self.cfg, self.wl.tensors
        prior, new = cfg.prior_entries, cfg.new_entries
        codes = _np(t["codes"][s]).copy()
        scales = _np(t["scales"][s]).copy()
        e64 = np.full((cfg.entries_total, 512), np.nan)      # pre-quantization values (computed rows)
        if not cfg.synthetic_cache and prior > 0:
            e = rope_rotate(compress(_np(t["x_prior"][s]), self.w, 1e-6),
                                   _np(t["rope_prior"][s]), 64)
            e64[:prior] = e
            codes[:prior], scales[:prior] = quantize(e.astype(np.float32))
        x_tail = _np(t["x_tail"][s])
        toks = x_tail[x_tail.shape[0] - 4 * new:]
        e = rope_rotate(compress(toks, self.w, 1e-6), _np(t["rope_cs"][s]), 64)
        e64[prior:prior + new] = e
        codes[prior:prior + new], scales[prior:prior + new] = quantize(e.astype(np.float32))
        k_fp8 = _np(t["k_fp8"][s])
        self._cache[s] = (codes, scales, k_fp8, x_tail)
        self._e64 = getattr(self, "_e64", {})
        self._e64[s] = e64
        return self._cache[s]

    def e64(self, s):
        self.cache(s)
        return self._e64[s]

    def window(self, s, p, li=0):
        """E4M3 bytes of the window tokens of a query at position p (layer li's
        own window when every layer has one, else the group's)."""
        cfg = self.cfg
        t = self.wl.tensors
        x = _np(t["x_win"][li][s]) if "x_win" in t else self.cache(s)[3]
        first = (cfg.ctx_tokens - 128) if cfg.kind == "decode" else (cfg.ctx_tokens - 127)
        pos = window_positions(p)
        return window_encode(x[pos - first])

    def keys(self, s):
        """Sequence s's indexer keys decoded to float64 (the latest sequence
        asked for is kept)."""
        if getattr(self, "_keys_s", None) != s:
            self._keys = e4m3_decode(self.cache(s)[2])
            self._keys_s = s
        return self._keys

    def precompute_full_scores(self, queries, batch=64):
        """Full-layer scores of many queries of one chunk at once (prefill
        queries of a sequence share its keys): fills a cache that query()
        uses.  The scores equal index_scores' up to the order of the final
        8-term weighted sum."""
        cfg, t = self.cfg, self.wl.tensors
        self._scores = getattr(self, "_scores", {})
        fl = [li for li, m in enumerate(cfg.layers) if m == "F"]
        by_seq = {}
        for qi in queries:
            by_seq.setdefault(qi // cfg.chunk, []).append(qi)
        for s, qs in by_seq.items():
            kv = self.keys(s)
            for li in fl:
                q8, w = _np(t["q_fp8"][li]), _np(t["w_idx"][li])
                for b in range(0, len(qs), batch):
                    qb = np.array(qs[b:b + batch])
                    nvs = [visible_entries(int(t["q_pos"][qi]), cfg.entries_total) for qi in qb]
                    sc = index_scores_many(q8[qb], w[qb], kv[:max(nvs)])
                    for i, qi in enumerate(qb):
                        self._scores[(int(qi), li)] = sc[i, :nvs[i]]

    def query(self, qi, attend=True):
        """Per-layer oracle results for query qi: list of LayerState
        (attend=False: selection only, every out is None)."""
        cfg, t = self.cfg, self.wl.tensors
        s = qi // cfg.chunk
        p = int(t["q_pos"][qi])
        codes, scales, k_fp8, _ = self.cache(s)
        kv = self.keys(s)
        per_layer = "x_win" in t
        win = None if (per_layer or not attend) else self.window(s, p)
        n_entries = cfg.entries_total
        cached = getattr(self, "_scores", {})
        res, idx, pool = [], None, None
        for li, mode in enumerate(cfg.layers):
            if per_layer and attend:
                win = self.window(s, p, li)
            qa = _np(t["q_attn"][li][qi]) if attend else None
            if mode == "F":
                st = layer_full(codes, scales, k_fp8, _np(t["q_fp8"][li][qi]),
                                _np(t["w_idx"][li][qi]), qa, p, win, SM,
                                build_pool=cfg.build_pool, n_entries=n_entries, k_values=kv,
                                scores=cached.get((qi, li)), attend=attend)
                pool = st.pool
            elif mode == "I":
                st = layer_reindex(codes, scales, k_fp8, pool, _np(t["q_fp8"][li][qi]),
                                   _np(t["w_idx"][li][qi]), qa, p, win, SM, n_entries=n_entries,
                                   k_values=kv, attend=attend)
            else:
                st = layer_reuse(codes, scales, idx, qa, win, SM, attend=attend)
            idx = st.idx
            res.append(st)
        return res

    def attention(self, qi, li, idx, codes, scales):
        """Layer li's attention output for query qi over the given selected
        ids and cache bytes (codes / scales of the query's sequence), with
        the oracle's own window bytes."""
        t = self.wl.tensors
        s = qi // self.cfg.chunk
        p = int(t["q_pos"][qi])
        win = self.window(s, p, li if "x_win" in t else 0)
        return sparse_attention(_np(t["q_attn"][li][qi]), codes, scales, idx, win, SM)
