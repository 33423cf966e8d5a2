// Global-KV files: the MXFP4 entries (codes, scales) and indexer keys of a
// group's sequences written to a file and read back, so that decoding resumes
// from a persistent cache ("DeepSeek-V4.1 架构解析" §03: the global KV is what stays in the
// persistent cache; the window is rebuilt by replay instead).
//
// File layout, little-endian:
//   bytes  0..7   magic "CSA2GKV1"
//          8..11  u32 version (1)        12..15 u32 header bytes (64)
//         16..23  i64 n_seq              24..31 i64 n_entries
//         32..35  u32 code bytes / row (256)   36..39 u32 scale bytes / row (32)
//         40..43  u32 key bytes / row (128)    44..47 u32 flags (0)
//         48..55  u64 payload checksum   56..63 u64 reserved (0)
//   payload: for every sequence s: its n_entries code rows, then its scale
//   rows, then its key rows.
// Checksum: FNV-1a over the payload read as little-endian 64-bit words
// (h = 0xcbf29ce484222325; for each word: h ^= word, h *= 0x100000001b3).
//
// Copies go through a caller-provided pinned host buffer split in two halves:
// while one half is written to (or read from) the file, the other half's
// device copy is in flight on the caller's stream.
#include <cerrno>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <algorithm>

#include "common.h"
#include "status.h"

using namespace csa;

namespace {

constexpr char KV_MAGIC[8] = {'C', 'S', 'A', '2', 'G', 'K', 'V', '1'};
constexpr uint32_t KV_VERSION = 1;
constexpr uint32_t KV_HEADER = 64;
constexpr uint64_t FNV_OFFSET = 0xcbf29ce484222325ull;
constexpr uint64_t FNV_PRIME = 0x100000001b3ull;
constexpr int64_t ROW_BYTES[3] = {CODE_BYTES, SCALE_BYTES, ID};

struct KvHeader {
  char magic[8];
  uint32_t version, header_bytes;
  int64_t n_seq, n_entries;
  uint32_t code_bytes, scale_bytes, key_bytes, flags;
  uint64_t checksum, reserved;
};
static_assert(sizeof(KvHeader) == KV_HEADER, "header layout");

uint64_t fnv_words(uint64_t h, const uint8_t* p, size_t n) {   // n is a multiple of 8
  for (size_t i = 0; i < n; i += 8) {
    uint64_t w;
    memcpy(&w, p + i, 8);
    h ^= w;
    h *= FNV_PRIME;
  }
  return h;
}

struct File {
  FILE* f = nullptr;
  ~File() {
    if (f) fclose(f);
  }
};

// One contiguous device region of the payload: sequence s, array a (0 codes, 1 scales, 2 keys).
struct Region {
  uint8_t* dev;
  int64_t bytes;
};

Region region(uint8_t* const base[3], int64_t seq_rows, int64_t n_entries, int64_t s, int a) {
  return Region{base[a] + s * seq_rows * ROW_BYTES[a], n_entries * ROW_BYTES[a]};
}

csa_status check_header(const char* fn, const KvHeader& h, int64_t file_bytes, const char* path) {
  if (memcmp(h.magic, KV_MAGIC, 8) != 0) return fail(CSA_ERR_IO, "%s: %s is not a global-KV file", fn, path);
  if (h.version != KV_VERSION || h.header_bytes != KV_HEADER)
    return fail(CSA_ERR_IO, "%s: %s has version %u / header %u, expected %u / %u", fn, path, h.version,
                h.header_bytes, KV_VERSION, KV_HEADER);
  if (h.code_bytes != CODE_BYTES || h.scale_bytes != SCALE_BYTES || h.key_bytes != ID || h.flags != 0)
    return fail(CSA_ERR_IO, "%s: %s has row sizes %u/%u/%u, expected %d/%d/%d", fn, path, h.code_bytes,
                h.scale_bytes, h.key_bytes, CODE_BYTES, SCALE_BYTES, ID);
  if (h.n_seq < 0 || h.n_entries < 0 || h.n_seq > ((int64_t)1 << 24) || h.n_entries > ((int64_t)1 << 32))
    return fail(CSA_ERR_IO, "%s: %s has sizes out of range", fn, path);
  // the header's sizes are untrusted: the payload size must not overflow
  // int64 (a wrapped product could match the file size)
  int64_t rows = 0, payload = 0;
  if (__builtin_mul_overflow(h.n_seq, h.n_entries, &rows) ||
      __builtin_mul_overflow(rows, (int64_t)(CODE_BYTES + SCALE_BYTES + ID), &payload) ||
      payload > INT64_MAX - (int64_t)KV_HEADER)
    return fail(CSA_ERR_IO, "%s: %s has sizes whose payload overflows", fn, path);
  if (file_bytes != (int64_t)KV_HEADER + payload)
    return fail(CSA_ERR_IO, "%s: %s holds %lld bytes, its header needs %lld", fn, path, (long long)file_bytes,
                (long long)(KV_HEADER + payload));
  return CSA_OK;
}

csa_status open_and_read_header(const char* fn, const char* path, File& file, KvHeader& h) {
  file.f = fopen(path, "rb");
  if (!file.f) return fail(CSA_ERR_IO, "%s: cannot open %s: %s", fn, path, strerror(errno));
  if (fseek(file.f, 0, SEEK_END) != 0) return fail(CSA_ERR_IO, "%s: cannot seek %s", fn, path);
  const long size = ftell(file.f);
  if (size < 0 || fseek(file.f, 0, SEEK_SET) != 0) return fail(CSA_ERR_IO, "%s: cannot seek %s", fn, path);
  if (size < (long)KV_HEADER || fread(&h, KV_HEADER, 1, file.f) != 1)
    return fail(CSA_ERR_IO, "%s: %s is shorter than a header", fn, path);
  return check_header(fn, h, (int64_t)size, path);
}

csa_status check_stage(const char* fn, void* stage, size_t stage_bytes) {
  if (!stage) return fail(CSA_ERR_INVALID_ARG, "%s: stage is NULL", fn);
  if (stage_bytes < 2 * 4096) return fail(CSA_ERR_WORKSPACE, "%s: stage needs at least 8 KiB", fn);
  if (reinterpret_cast<uintptr_t>(stage) % 16 != 0)
    return fail(CSA_ERR_ALIGNMENT, "%s: stage is not 16-byte aligned", fn);
  return CSA_OK;
}

}  // namespace

extern "C" {

csa_status csa_kv_file_info(const char* path, int64_t* n_seq, int64_t* n_entries) {
  const char* fn = "csa_kv_file_info";
  if (!path || !n_seq || !n_entries) return fail(CSA_ERR_INVALID_ARG, "%s: NULL argument", fn);
  File file;
  KvHeader h;
  const csa_status st = open_and_read_header(fn, path, file, h);
  if (st != CSA_OK) return st;
  *n_seq = h.n_seq;
  *n_entries = h.n_entries;
  return CSA_OK;
}

csa_status csa_kv_save(const char* path, const uint8_t* codes, const uint8_t* scales, const uint8_t* k_fp8,
                       int64_t n_seq, int64_t seq_rows, int64_t n_entries, void* stage, size_t stage_bytes,
                       hipStream_t stream) {
  const char* fn = "csa_kv_save";
  if (!path) return fail(CSA_ERR_INVALID_ARG, "%s: path is NULL", fn);
  if (n_seq < 0 || n_entries < 0 || n_entries > seq_rows || n_seq > ((int64_t)1 << 24))
    return fail(CSA_ERR_INVALID_ARG, "%s: need 0 <= n_entries <= seq_rows and 0 <= n_seq", fn);
  if (n_seq * n_entries > 0 && (!codes || !scales || !k_fp8))
    return fail(CSA_ERR_INVALID_ARG, "%s: NULL cache pointer", fn);
  csa_status st = check_stage(fn, stage, stage_bytes);
  if (st != CSA_OK) return st;
  File file;
  file.f = fopen(path, "wb");
  if (!file.f) return fail(CSA_ERR_IO, "%s: cannot create %s: %s", fn, path, strerror(errno));
  KvHeader h{};
  memcpy(h.magic, KV_MAGIC, 8);
  h.version = KV_VERSION;
  h.header_bytes = KV_HEADER;
  h.n_seq = n_seq;
  h.n_entries = n_entries;
  h.code_bytes = CODE_BYTES;
  h.scale_bytes = SCALE_BYTES;
  h.key_bytes = ID;
  if (fwrite(&h, KV_HEADER, 1, file.f) != 1) return fail(CSA_ERR_IO, "%s: write failed on %s", fn, path);

  uint8_t* const base[3] = {const_cast<uint8_t*>(codes), const_cast<uint8_t*>(scales), const_cast<uint8_t*>(k_fp8)};
  const size_t half = (stage_bytes / 2) & ~(size_t)15;
  uint8_t* buf[2] = {static_cast<uint8_t*>(stage), static_cast<uint8_t*>(stage) + half};
  hipEvent_t ev[2];
  if (hipEventCreateWithFlags(&ev[0], hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&ev[1], hipEventDisableTiming) != hipSuccess)
    return fail(CSA_ERR_HIP, "%s: event creation failed", fn);
  uint64_t sum = FNV_OFFSET;
  // chunks in payload order: (sequence, array, offset)
  struct Chunk {
    uint8_t* dev;
    size_t bytes;
  };
  int64_t s = 0, off = 0;
  int a = 0;
  auto next = [&](Chunk& c) -> bool {
    while (s < n_seq) {
      const Region r = region(base, seq_rows, n_entries, s, a);
      if (off < r.bytes) {
        c.dev = r.dev + off;
        c.bytes = (size_t)std::min<int64_t>((int64_t)half, r.bytes - off);
        off += (int64_t)c.bytes;
        return true;
      }
      off = 0;
      if (++a == 3) {
        a = 0;
        ++s;
      }
    }
    return false;
  };
  csa_status res = CSA_OK;
  Chunk cur{}, nxt{};
  bool have = next(cur);
  int slot = 0;
  if (have) {
    if (hipMemcpyAsync(buf[0], cur.dev, cur.bytes, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipEventRecord(ev[0], stream) != hipSuccess)
      res = fail(CSA_ERR_HIP, "%s: device-to-host copy failed", fn);
  }
  while (have && res == CSA_OK) {
    const bool more = next(nxt);
    if (more && (hipMemcpyAsync(buf[slot ^ 1], nxt.dev, nxt.bytes, hipMemcpyDeviceToHost, stream) != hipSuccess ||
                 hipEventRecord(ev[slot ^ 1], stream) != hipSuccess)) {
      res = fail(CSA_ERR_HIP, "%s: device-to-host copy failed", fn);
      break;
    }
    if (hipEventSynchronize(ev[slot]) != hipSuccess) {
      res = fail(CSA_ERR_HIP, "%s: device-to-host copy failed", fn);
      break;
    }
    sum = fnv_words(sum, buf[slot], cur.bytes);
    if (fwrite(buf[slot], 1, cur.bytes, file.f) != cur.bytes) {
      res = fail(CSA_ERR_IO, "%s: write failed on %s", fn, path);
      break;
    }
    cur = nxt;
    have = more;
    slot ^= 1;
  }
  // the other half may still be in flight after an error: drain before the stage is reused
  if (hipStreamSynchronize(stream) != hipSuccess && res == CSA_OK)
    res = fail(CSA_ERR_HIP, "%s: device-to-host copy failed", fn);
  (void)hipEventDestroy(ev[0]);
  (void)hipEventDestroy(ev[1]);
  if (res != CSA_OK) return res;
  h.checksum = sum;
  if (fseek(file.f, 0, SEEK_SET) != 0 || fwrite(&h, KV_HEADER, 1, file.f) != 1 || fflush(file.f) != 0)
    return fail(CSA_ERR_IO, "%s: write failed on %s", fn, path);
  return CSA_OK;
}

csa_status csa_kv_load(const char* path, uint8_t* codes, uint8_t* scales, uint8_t* k_fp8, int64_t n_seq,
                       int64_t seq_rows, int64_t* n_entries_out, void* stage, size_t stage_bytes,
                       hipStream_t stream) {
  const char* fn = "csa_kv_load";
  if (!path || !n_entries_out) return fail(CSA_ERR_INVALID_ARG, "%s: NULL argument", fn);
  csa_status st = check_stage(fn, stage, stage_bytes);
  if (st != CSA_OK) return st;
  File file;
  KvHeader h;
  st = open_and_read_header(fn, path, file, h);
  if (st != CSA_OK) return st;
  if (h.n_seq != n_seq)
    return fail(CSA_ERR_INVALID_ARG, "%s: %s holds %lld sequences, the buffers %lld", fn, path,
                (long long)h.n_seq, (long long)n_seq);
  if (h.n_entries > seq_rows)
    return fail(CSA_ERR_INVALID_ARG, "%s: %s holds %lld entries per sequence, the buffers %lld rows", fn, path,
                (long long)h.n_entries, (long long)seq_rows);
  const int64_t n_entries = h.n_entries;
  if (n_seq * n_entries > 0 && (!codes || !scales || !k_fp8))
    return fail(CSA_ERR_INVALID_ARG, "%s: NULL cache pointer", fn);

  uint8_t* const base[3] = {codes, scales, k_fp8};
  const size_t half = (stage_bytes / 2) & ~(size_t)15;
  uint8_t* buf[2] = {static_cast<uint8_t*>(stage), static_cast<uint8_t*>(stage) + half};
  hipEvent_t ev[2];
  if (hipEventCreateWithFlags(&ev[0], hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&ev[1], hipEventDisableTiming) != hipSuccess)
    return fail(CSA_ERR_HIP, "%s: event creation failed", fn);
  bool pending[2] = {false, false};
  uint64_t sum = FNV_OFFSET;
  csa_status res = CSA_OK;
  int slot = 0;
  for (int64_t s = 0; s < n_seq && res == CSA_OK; ++s) {
    for (int a = 0; a < 3 && res == CSA_OK; ++a) {
      const Region r = region(base, seq_rows, n_entries, s, a);
      for (int64_t off = 0; off < r.bytes; off += (int64_t)half) {
        const size_t n = (size_t)std::min<int64_t>((int64_t)half, r.bytes - off);
        if (pending[slot] && hipEventSynchronize(ev[slot]) != hipSuccess) {   // this half's last copy is done
          res = fail(CSA_ERR_HIP, "%s: host-to-device copy failed", fn);
          break;
        }
        if (fread(buf[slot], 1, n, file.f) != n) {
          res = fail(CSA_ERR_IO, "%s: read failed on %s", fn, path);
          break;
        }
        sum = fnv_words(sum, buf[slot], n);
        if (hipMemcpyAsync(r.dev + off, buf[slot], n, hipMemcpyHostToDevice, stream) != hipSuccess ||
            hipEventRecord(ev[slot], stream) != hipSuccess) {
          res = fail(CSA_ERR_HIP, "%s: host-to-device copy failed", fn);
          break;
        }
        pending[slot] = true;
        slot ^= 1;
      }
    }
  }
  if (hipStreamSynchronize(stream) != hipSuccess && res == CSA_OK)
    res = fail(CSA_ERR_HIP, "%s: host-to-device copy failed", fn);
  (void)hipEventDestroy(ev[0]);
  (void)hipEventDestroy(ev[1]);
  if (res != CSA_OK) return res;
  if (sum != h.checksum)
    return fail(CSA_ERR_IO, "%s: %s fails its checksum (the buffers now hold its damaged contents)", fn, path);
  *n_entries_out = n_entries;
  return CSA_OK;
}

}  // extern "C"
