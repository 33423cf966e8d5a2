"""Host-side checks of the C ABI (no GPU needed).

The library loads, exports every function declared in include/csa.h, and
rejects invalid arguments with the documented status before any launch (no
device is touched: these calls fail validation first).
"""

import ctypes
import os
import re

import pytest

from compressed_sparse_attention_04_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")

OK, INVALID, UNSUPPORTED, ALIGN, WORKSPACE = 0, 1, 2, 3, 4
P = ctypes.c_void_p(4096)            # a fake, aligned, never-dereferenced address
P_ODD = ctypes.c_void_p(4097)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) == 29
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES), set(names) ^ set(_lib.SIGNATURES)


def test_status_strings_and_version(lib):
    assert lib.csa_status_string(0) == b"ok"
    assert lib.csa_status_string(4) == b"workspace too small"
    assert lib.csa_version() >= 100


def test_layer_struct_matches_header():
    text = open(HEADER).read()
    body = text[text.index("typedef struct csa_layer_args"):text.index("} csa_layer_args;")]
    fields = re.findall(r"\b([a-z_0-9]+);", body)
    assert fields == [f for f, _ in _lib.CsaLayerArgs._fields_]


def test_quantize_validation(lib):
    assert lib.csa_quantize(None, 0, None, None, None) == OK              # n = 0: no-op
    assert lib.csa_quantize(None, 4, P, P, None) == INVALID
    assert b"NULL" in lib.csa_last_error()
    assert lib.csa_quantize(P, -1, P, P, None) == INVALID
    assert lib.csa_quantize(P_ODD, 4, P, P, None) == ALIGN


def test_compress_append_validation(lib):
    """The fused call checks each non-empty part as the separate calls do and
    enqueues nothing when either is invalid."""
    f = lib.csa_compress_quant_append
    need = lib.csa_compress_quant_workspace_size(10)
    comp = [P, 1, 10, 10 * 2048, P, P, 64, ctypes.c_float(1e-6), P, P, 10, None, P, need]
    none_comp = [None, 0, 0, 0, None, None, 0, ctypes.c_float(1e-6), None, None, 0, None, None, 0]
    app = [P, 2, 1, 4096, P, P, 128]
    none_app = [None, 0, 0, 0, None, None, 0]
    assert f(*none_comp, *none_app, None) == OK                           # both parts empty
    a = list(app); a[0] = None
    assert f(*none_comp, *a, None) == INVALID                             # window part: x missing
    a = list(app); a[6] = 127
    assert f(*none_comp, *a, None) == UNSUPPORTED                         # window part: win_cap < 128
    a = list(app); a[5] = P_ODD
    assert f(*comp, *a, None) == ALIGN                                    # valid compression, bad window
    a = list(comp); a[6] = 63
    assert f(*a, *app, None) == UNSUPPORTED                               # bad compression, valid window
    a = list(comp); a[13] = need - 1
    assert f(*a, *none_app, None) == WORKSPACE
    assert f(*none_comp[:1], -1, *none_comp[2:], *none_app, None) == INVALID
    assert b"csa_compress_quant_append" in lib.csa_last_error()


def test_compress_validation(lib):
    f = lib.csa_compress_quant
    need = lib.csa_compress_quant_workspace_size(10)
    assert need > 0
    args = [P, 1, 10, 10 * 2048, P, P, 64, ctypes.c_float(1e-6), P, P, 10, None, P, need, None]
    a = list(args); a[6] = 63
    assert f(*a) == UNSUPPORTED                                           # odd rope_dim
    a = list(args); a[5] = None
    assert f(*a) == INVALID                                               # rope table missing
    a = list(args); a[13] = need - 1
    assert f(*a) == WORKSPACE
    a = list(args); a[8] = P_ODD
    assert f(*a) == ALIGN
    a = list(args); a[1] = 2; a[3] = 100
    assert f(*a) == INVALID                                               # overlapping sequences


def test_topk_and_pool_validation(lib):
    assert lib.csa_topk(P, 2, 100, None, 0, P, None, 0, None) == UNSUPPORTED
    assert lib.csa_topk(P, 2, 100, None, 16385, P, None, 0, None) == UNSUPPORTED   # k above CSA_MAX_K
    assert lib.csa_topk(P, 2, 100, P, 10, P, None, 0, None) == INVALID     # pooled, 100 % 8 != 0
    need = lib.csa_topk_workspace_size(2, 100000, 512)
    assert need > 0
    assert lib.csa_topk(P, 2, 100000, None, 512, P, P, need - 8, None) == WORKSPACE
    assert lib.csa_block_pool(P, 2, 1, 10, 8, P, None, 0, None) == INVALID
    assert lib.csa_block_pool(P, 1, 1, 10, 0, P, None, 0, None) == UNSUPPORTED


def test_score_and_attn_validation(lib):
    f = lib.csa_index_score
    assert f(P, P, P, 1, 1, P, 100, 101, None, 0, P, None, None) == INVALID   # n_entries > k_rows
    assert f(P, P, P, 1, 1, P, 100, 50, None, 0, None, None, None) == INVALID  # no output
    assert f(P_ODD, P, P, 1, 1, P, 100, 50, None, 0, P, None, None) == ALIGN
    g = lib.csa_sparse_attn
    base = [P, P, 1, 1, P, P, 100, P, 512, P, 128, ctypes.c_float(0.04), P, P, 1 << 30, None]
    a = list(base); a[10] = 64
    assert g(*a) == UNSUPPORTED                                           # window ring too small
    a = list(base); a[8] = 0
    assert g(*a) == UNSUPPORTED
    a = list(base); a[11] = ctypes.c_float(float("nan"))
    assert g(*a) == INVALID


def test_layer_validation(lib):
    a = _lib.CsaLayerArgs()
    a.n_seq, a.q_per_seq, a.top_k = 1, 1, 512
    a.kv_rows, a.k_rows, a.n_entries = 100, 100, 100
    assert lib.csa_layer_full(ctypes.byref(a), None) == INVALID           # null pointers
    assert lib.csa_layer_full(None, None) == INVALID
    a.top_k = 0
    assert lib.csa_layer_reuse(ctypes.byref(a), None) == UNSUPPORTED
    assert lib.csa_layer_workspace_size(7, ctypes.byref(a)) == 0


def test_layer_pool_size_validation(lib):
    """Pool sizes outside [top_k, 4096] are rejected before anything is launched."""
    a = _lib.CsaLayerArgs()
    for f in ["codes", "scales", "k_fp8", "win", "q_pos", "q_attn", "q_idx", "w_idx", "pool_blocks",
              "idx", "out"]:
        setattr(a, f, 1 << 20)
    a.kv_rows = a.k_rows = a.n_entries = 1000
    a.win_cap, a.n_seq, a.q_per_seq = 128, 2, 1
    a.sm_scale, a.top_k, a.build_pool = 0.044, 512, 1
    a.ws, a.ws_bytes = 1 << 20, 1 << 40
    for nb in (4097, 5000, 511, 0):
        a.n_pool_blocks = nb
        assert lib.csa_layer_full(ctypes.byref(a), None) in (UNSUPPORTED, INVALID), nb


@pytest.mark.skipif(__import__("torch").cuda.is_available(),
                    reason="would launch on fake pointers; host-only check")
def test_valid_layer_args_pass_validation(lib):
    """With valid arguments validation succeeds and the launch is attempted;
    without a GPU that launch reports CSA_ERR_HIP (status 5)."""
    a = _lib.CsaLayerArgs()
    for f in ["codes", "scales", "k_fp8", "win", "q_pos", "q_attn", "q_idx", "w_idx", "pool_blocks",
              "idx", "out"]:
        setattr(a, f, 1 << 20)
    a.kv_rows = a.k_rows = a.n_entries = 1000
    a.win_cap, a.n_seq, a.q_per_seq = 128, 2, 1
    a.sm_scale, a.top_k, a.build_pool, a.n_pool_blocks = 0.044, 512, 1, 2048
    need = [lib.csa_layer_workspace_size(m, ctypes.byref(a)) for m in (0, 1, 2)]
    a.ws, a.ws_bytes = 1 << 20, max(need)
    for fn in (lib.csa_layer_full, lib.csa_layer_reindex, lib.csa_layer_reuse):
        assert fn(ctypes.byref(a), None) == 5, lib.csa_last_error()
    a.ws_bytes = need[0] - 1
    assert lib.csa_layer_full(ctypes.byref(a), None) == WORKSPACE


def test_window_rebuild_validation(lib):
    """csa_window_rebuild rejects bad sizes, capacities and alignment before
    anything is launched."""
    f = lib.csa_window_rebuild
    P = 1 << 20
    # (n_ring, n_tok, x_ring_stride, x, p_last, win, win_cap)
    assert f(P, 2, 0, 128 * 512, P, P, 128, None) == INVALID           # n_tok < 1
    assert f(P, 2, 129, 129 * 512, P, P, 128, None) == INVALID         # n_tok > win_cap
    assert f(P, 2, 128, 128 * 512, P, P, 64, None) == UNSUPPORTED      # win_cap < 128
    assert f(P, 2, 128, 100 * 512, P, P, 128, None) == INVALID         # overlapping rings
    assert f(P + 4, 2, 128, 128 * 512, P, P, 128, None) == ALIGN       # x not 16-byte aligned
    assert f(None, 2, 128, 128 * 512, P, P, 128, None) != 0            # null pointer
    assert f(P, 0, 128, 128 * 512, P, P, 128, None) == 0               # nothing to do


def test_attn_after_needs_a_recorded_event():
    """An unrecorded torch event has no HIP handle yet; passing it would make
    the layer's attention wait for nothing, so the binding refuses it."""
    import torch
    from compressed_sparse_attention_04_amd import ops

    call = ops.LayerCall.__new__(ops.LayerCall)
    call.args = _lib.CsaLayerArgs()
    with pytest.raises(ValueError):
        call.set_attn_after(torch.cuda.Event())
    call.set_attn_after(None)
    assert call.args.attn_after is None
