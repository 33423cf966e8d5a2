"""Global-KV file format and argument checks of csa_kv_file_info / csa_kv_save
/ csa_kv_load that run before any device copy (CPU only).  Files are written
here from the layout the header documents (64-byte header, per-sequence code,
scale and key rows, FNV-1a checksum over 64-bit words)."""

import ctypes
import os
import struct

import numpy as np
import pytest

from compressed_sparse_attention_04_amd import _lib

OK, INVALID, UNSUPPORTED, ALIGN, WORKSPACE, HIP, IO = 0, 1, 2, 3, 4, 5, 6
ROW = 256 + 32 + 128


def fnv_words(payload):
    h = 0xcbf29ce484222325
    for w in np.frombuffer(payload, dtype="<u8"):
        h ^= int(w)
        h = (h * 0x100000001b3) & 0xFFFFFFFFFFFFFFFF
    return h


def write_file(path, n_seq, n_entries, magic=b"CSA2GKV1", version=1, rows=(256, 32, 128), extra=b"",
               checksum=None, payload=None):
    if payload is None:
        payload = np.random.default_rng(1).integers(0, 256, n_seq * n_entries * ROW, dtype=np.uint8).tobytes()
    cs = fnv_words(payload) if checksum is None else checksum
    hdr = magic + struct.pack("<IIqqIIIIQQ", version, 64, n_seq, n_entries, rows[0], rows[1], rows[2], 0, cs, 0)
    assert len(hdr) == 64
    with open(path, "wb") as f:
        f.write(hdr + payload + extra)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def info(lib, path):
    a, b = ctypes.c_int64(-1), ctypes.c_int64(-1)
    rc = lib.csa_kv_file_info(os.fsencode(str(path)), ctypes.byref(a), ctypes.byref(b))
    return rc, a.value, b.value


def test_file_info_reads_a_valid_header(lib, tmp_path):
    p = tmp_path / "kv.bin"
    write_file(p, 3, 17)
    assert info(lib, p) == (OK, 3, 17)
    write_file(p, 2, 0)
    assert info(lib, p) == (OK, 2, 0)


@pytest.mark.parametrize("kw", [dict(magic=b"CSA2GKV2"), dict(version=2), dict(rows=(256, 32, 64)),
                                dict(extra=b"\0" * 8)])
def test_file_info_rejects_bad_headers_and_sizes(lib, tmp_path, kw):
    p = tmp_path / "kv.bin"
    write_file(p, 2, 5, **kw)
    assert info(lib, p)[0] == IO


def test_file_info_rejects_truncated_and_missing_files(lib, tmp_path):
    p = tmp_path / "kv.bin"
    write_file(p, 2, 5)
    data = p.read_bytes()
    p.write_bytes(data[:-8])
    assert info(lib, p)[0] == IO
    p.write_bytes(data[:40])
    assert info(lib, p)[0] == IO
    assert info(lib, tmp_path / "missing.bin")[0] == IO
    assert "missing.bin" in lib.csa_last_error().decode()


def test_load_checks_before_copying(lib, tmp_path):
    """Sequence count and capacity mismatches, and a bad stage, are rejected
    before any device copy (fake device pointers are never touched)."""
    p = tmp_path / "kv.bin"
    write_file(p, 2, 10)
    stage = (ctypes.c_uint8 * 16384)()
    sp = ctypes.cast(stage, ctypes.c_void_p).value
    n = ctypes.c_int64(0)
    P = 1 << 20
    f = lib.csa_kv_load
    path = os.fsencode(str(p))
    assert f(path, P, P, P, 3, 10, ctypes.byref(n), sp, 16384, None) == INVALID   # n_seq differs
    assert f(path, P, P, P, 2, 9, ctypes.byref(n), sp, 16384, None) == INVALID    # too few rows
    assert f(path, P, P, P, 2, 10, ctypes.byref(n), None, 16384, None) == INVALID  # no stage
    assert f(path, P, P, P, 2, 10, ctypes.byref(n), sp, 4096, None) == WORKSPACE  # stage too small
    assert f(path, P, P, P, 2, 10, ctypes.byref(n), sp + 8, 16000, None) == ALIGN  # misaligned stage


def test_save_checks_before_copying(lib, tmp_path):
    stage = (ctypes.c_uint8 * 16384)()
    sp = ctypes.cast(stage, ctypes.c_void_p).value
    P = 1 << 20
    f = lib.csa_kv_save
    assert f(os.fsencode(str(tmp_path / "a.bin")), P, P, P, 2, 10, 11, sp, 16384, None) == INVALID  # n > rows
    assert f(os.fsencode(str(tmp_path / "no" / "dir" / "a.bin")), P, P, P, 2, 10, 10, sp, 16384, None) == IO
    assert f(None, P, P, P, 2, 10, 10, sp, 16384, None) == INVALID


def test_status_string_of_io_error(lib):
    assert lib.csa_status_string(IO) == b"file error"


def test_file_info_rejects_a_header_whose_payload_size_overflows(lib, tmp_path):
    """Sizes inside the per-field caps whose product with the 416-byte row
    does not fit int64: reported as an overflow, not compared after a wrap."""
    p = tmp_path / "kv.bin"
    write_file(p, 1, 1)
    raw = bytearray(open(p, "rb").read())
    raw[16:32] = struct.pack("<qq", 1 << 24, 1 << 32)       # n_seq, n_entries at the caps
    open(p, "wb").write(bytes(raw))
    rc, _, _ = info(lib, p)
    assert rc == IO
    assert b"overflow" in lib.csa_last_error()
