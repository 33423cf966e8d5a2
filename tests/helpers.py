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


# The GPU chain computes in fp64 and rounds once to fp32, so its quantizer
# input is within one fp32 ulp of the oracle's; entries are RMS-normalized
# (|x| <= sqrt(512) < 32, ulp <= 2**-19), so a differing byte must come from a
# value within 2e-6 of a rounding decision.
CHAIN_ABS = 2e-6


def boundary_distance(x):
    """Absolute distance (in entry units) of a 16-value group (float64) to the
    nearest rounding decision of the quantizer: amax against 6 x the E4M3
    midpoints (scale decision), every |x| against s x the E2M1 midpoints under
    the oracle's scale s (element decisions), and every x against 0 (the sign
    bit, which a value rounding to magnitude 0 keeps)."""
    x = np.asarray(x, dtype=np.float64)
    amax = np.abs(x).max()
    d0 = float(np.min(np.abs(x)))
    pos = formats.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    d = float(np.min(np.abs(amax - 6 * mids)))
    s = formats.e4m3_decode(formats.e4m3_encode(amax / 6))
    if s > 0:
        em = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]) * s
        d = min(d, float(np.min(np.abs(np.abs(x)[:, None] - em[None]))))
    return min(d, d0)


def cache_flips(gpu_codes, gpu_scales, ref_codes, ref_scales, ref_e64, rows, tol=CHAIN_ABS):
    """Entries (within ``rows``) whose dequantized values differ between the GPU
    and the oracle.  Every 16-channel group whose bytes differ must have the
    oracle's float64 pre-quantization value within ``tol`` of a rounding
    decision, i.e. within the float32 chain's error of a boundary.  (Groups that
    differ only in the sign of a zero magnitude dequantize to the same values.)"""
    flipped = set()
    for r in rows:
        gc, rc = gpu_codes[r], ref_codes[r]
        gs, rs = gpu_scales[r], ref_scales[r]
        if np.array_equal(gc, rc) and np.array_equal(gs, rs):
            continue
        for g in range(32):
            if gs[g] != rs[g] or not np.array_equal(gc[8 * g:8 * g + 8], rc[8 * g:8 * g + 8]):
                d = boundary_distance(ref_e64[r, 16 * g:16 * g + 16])
                assert d <= tol, f"entry {r} group {g}: bytes differ {d:.2e} from a rounding decision"
        if not np.array_equal(mxfp4.dequantize(gc, gs), mxfp4.dequantize(rc, rs)):
            flipped.add(int(r))
    return flipped


from oracle.runner import OracleStep  # noqa: E402


def check_queries(wl, st, queries, attn_queries=None):
    """Check a layer-group step against the oracle, query by query.

    Every query in ``queries``: pool bit-exact, each Full / Reindex Top-K set
    exact up to near-ties (check_topk_set).  Every query in ``attn_queries``
    (default: all of ``queries``): every layer's attention output, with the
    oracle run on the GPU's own selected ids and the GPU's own cache bytes,
    so that a near-tie swap or a boundary flip of a quantized byte (both
    allowed, and checked separately) does not compound into the attention
    tolerance.  The oracle's window bytes are used, so a wrong window byte
    fails the comparison.

    Returns a dict: swaps (layers whose set differs by near-ties), exact_sets
    (Full / Reindex layers whose set equals the oracle's), compared (attention
    outputs compared), outputs (attention outputs asked for), flipped_entries
    (cache entries whose bytes differ at a rounding boundary).
    """
    ref = OracleStep(wl)
    cfg = wl.cfg
    queries = list(queries)
    attn_set = set(queries if attn_queries is None else attn_queries)
    if cfg.kind == "prefill":
        ref.precompute_full_scores(queries)
    pool_gpu = np_(st.pool) if st.pool is not None else None
    r = dict(swaps=0, exact_sets=0, compared=0, outputs=0, flipped_entries=0)
    seq_bytes = {}

    def gpu_cache(s):
        if s not in seq_bytes:
            seq_bytes.clear()
            gc, gs = np_(st.codes[s]), np_(st.scales[s])
            rc, rs, _, _ = ref.cache(s)
            computed = range(0 if not cfg.synthetic_cache else cfg.prior_entries, cfg.entries_total)
            r["flipped_entries"] += len(cache_flips(gc, gs, rc, rs, ref.e64(s), computed))
            seq_bytes[s] = (gc, gs)
        return seq_bytes[s]

    for qi in queries:
        s = qi // cfg.chunk
        gc, gs = gpu_cache(s)
        res = ref.query(qi, attend=False)
        for li, mode in enumerate(cfg.layers):
            rl = res[li]
            gi = np_(st.idxs[li][qi])
            if mode in ("F", "I"):
                ids = None
                if mode == "F" and cfg.build_pool:
                    assert np.array_equal(pool_gpu[qi], rl.pool), f"pool differs at query {qi}"
                if mode == "I":
                    nv = oracle.visible_entries(int(wl.tensors["q_pos"][qi]), cfg.entries_total)
                    ids = oracle.pooled_entries(rl.pool, nv) if rl.pool is not None else np.arange(nv)
                n = check_topk_set(gi, rl.scores, rl.idx, len(rl.idx), ids=ids)
                r["swaps"] += n > 0
                if n == 0:
                    assert np.array_equal(np.sort(gi), np.sort(rl.idx))
                    r["exact_sets"] += 1
            if qi in attn_set:
                r["outputs"] += 1
                check_attn(np_(st.outs[li][qi]), ref.attention(qi, li, gi, gc, gs))
                r["compared"] += 1
    return r
