// Measurement probes: what this GPU sustains for the two resources the
// indexer is bound by, so that its roofline fractions can be read against
// the box as well as against the published peaks.  Not part of the method.
//
//   mfma_probe_kernel: every wave runs 32 independent chains of
//     v_mfma_f32_16x16x32_f16 (the indexer's instruction) on register
//     operands; 2 x 16 x 16 x 32 flops per instruction.  (Fewer chains leave
//     the matrix pipe waiting on each chain's previous result: 8 chains per
//     wave measured ~1.05 PFLOP/s, 16 ~1.6-1.7, 32 ~1.85 on an MI355X.)
//   mfma_f8_probe_kernel: the same for the FP8 matrix instructions (the
//     published dense FP8 peak is twice the fp16 one).
//   read_probe_kernel: whole-line 16-byte non-temporal loads over a buffer
//     (the indexer's load), grid-strided over 2,048 blocks, summed so the
//     loads stay live.
#include "common.h"
#include "status.h"

using namespace csa;

namespace {

constexpr int PROBE_CHAINS = 32;

__global__ __launch_bounds__(256) void mfma_probe_kernel(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  f16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(0.001f * (lane + i));
    b[i] = (_Float16)(0.002f * (lane - i));
  }
  f32x4 acc[PROBE_CHAINS];
#pragma unroll
  for (int c = 0; c < PROBE_CHAINS; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < PROBE_CHAINS; ++c) acc[c] = mfma_f16_16x16x32(a, b, acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < PROBE_CHAINS; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  if (s == 1234.5f) out[0] = s;   // keeps the chains live; practically never true
}

// FP8 matrix instructions, PROBE_CHAINS independent chains per wave:
// VARIANT 0 = v_mfma_scale_f32_16x16x128_f8f6f4 with E4M3 operands (scale
// bytes 127 = 1.0; 2 x 16 x 16 x 128 flops), VARIANT 1 =
// v_mfma_f32_16x16x32_fp8_fp8 (2 x 16 x 16 x 32 flops).
template <int VARIANT>
__global__ __launch_bounds__(256) void mfma_f8_probe_kernel(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  i32x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = 0x38383838 ^ (lane * 0x01010101 + i);   // E4M3 bytes around 1.0
    b[i] = 0x30303030 ^ (lane * 0x01000100 + 3 * i);
  }
  f32x4 acc[PROBE_CHAINS];
#pragma unroll
  for (int c = 0; c < PROBE_CHAINS; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < PROBE_CHAINS; ++c) {
      if constexpr (VARIANT == 0)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[c], 0, 0, 0, 127, 0, 127);
      else
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(((long)a[0] << 32) | (uint32_t)a[1],
                                                            ((long)b[0] << 32) | (uint32_t)b[1], acc[c], 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < PROBE_CHAINS; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  if (s == 1234.5f) out[0] = s;   // keeps the chains live; practically never true
}

__global__ __launch_bounds__(256) void read_probe_kernel(const uint8_t* buf, int64_t n16, float* out) {
  using i32x4v = int __attribute__((ext_vector_type(4)));
  const i32x4v* p = reinterpret_cast<const i32x4v*>(buf);
  i32x4v acc = {0, 0, 0, 0};
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
    acc += __builtin_nontemporal_load(p + i);
  if (acc[0] == 0x12345678 && acc[1] == 0x9abcdef) out[0] = 1.f;
}

}  // namespace

extern "C" {

csa_status csa_probe_mfma_f16(float* out, int32_t blocks, int32_t iters, hipStream_t stream) {
  const char* fn = "csa_probe_mfma_f16";
  if (!out) return fail(CSA_ERR_INVALID_ARG, "%s: out is NULL", fn);
  if (blocks < 1 || iters < 1) return fail(CSA_ERR_INVALID_ARG, "%s: blocks and iters must be >= 1", fn);
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, out, iters);
  return hip_status(hipGetLastError(), fn);
}

csa_status csa_probe_mfma_f8(float* out, int32_t blocks, int32_t iters, int32_t variant, hipStream_t stream) {
  const char* fn = "csa_probe_mfma_f8";
  if (!out) return fail(CSA_ERR_INVALID_ARG, "%s: out is NULL", fn);
  if (blocks < 1 || iters < 1) return fail(CSA_ERR_INVALID_ARG, "%s: blocks and iters must be >= 1", fn);
  if (variant == 0)
    hipLaunchKernelGGL(mfma_f8_probe_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, stream, out, iters);
  else if (variant == 1)
    hipLaunchKernelGGL(mfma_f8_probe_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, stream, out, iters);
  else
    return fail(CSA_ERR_INVALID_ARG, "%s: variant must be 0 or 1", fn);
  return hip_status(hipGetLastError(), fn);
}

csa_status csa_probe_read(const uint8_t* buf, int64_t bytes, float* out, hipStream_t stream) {
  const char* fn = "csa_probe_read";
  if (!buf || !out) return fail(CSA_ERR_INVALID_ARG, "%s: NULL argument", fn);
  if (bytes < 16 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return fail(CSA_ERR_ALIGNMENT, "%s: buf and bytes must be 16-byte multiples", fn);
  // 2,048 blocks: the fastest grid for this load on an MI355X (~7.1-7.2 TB/s;
  // 8,192 blocks of one load per thread measured ~6.5)
  hipLaunchKernelGGL(read_probe_kernel, dim3(2048), dim3(256), 0, stream, buf, bytes / 16, out);
  return hip_status(hipGetLastError(), fn);
}

}  // extern "C"
