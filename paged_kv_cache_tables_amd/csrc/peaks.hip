// Measurement helpers: the device rates that the attention kernels' figures are
// read against, measured on the same GPU (not part of the attention path).
//
//   * A streaming read: every 16-byte chunk of a buffer loaded once with the
//     non-temporal hint the decode kernel uses for K/V.
//   * A matrix-core loop: every wave issues back-to-back independent
//     v_mfma_f32_32x32x16_bf16 (the prefill kernel's instruction) on register
//     operands, with no memory traffic.
// Both fold what they compute into one value that is stored only if it equals a
// constant it cannot reach, so nothing is optimised away and nothing is written.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "pagedkv.h"

namespace pkv {
namespace {

constexpr int kPeakThreads = 256;
constexpr uint32_t kNever = 0x9e3779b9u;

// Each wave reads a contiguous share of the buffer, 16 KiB (16 wave-wide 16-byte loads)
// in flight at a time; 16 waves per compute unit.  This was the fastest arrangement of a
// read-only probe on this device (more waves beat more bytes in flight per wave).
constexpr int kReadBatch = 16;

__global__ __launch_bounds__(kPeakThreads) void peak_read_kernel(const uint4* __restrict__ buf, int64_t n16,
                                                                 uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t waves = (int64_t)gridDim.x * (kPeakThreads / kWave);
  const int64_t w = (int64_t)blockIdx.x * (kPeakThreads / kWave) + threadIdx.x / kWave;
  const int64_t rows = n16 / kWave;              // wave-wide rows of 1 KiB
  const int64_t r0 = rows * w / waves, r1 = rows * (w + 1) / waves;
  uint32_t acc = 0;
  int64_t r = r0;
  for (; r + kReadBatch <= r1; r += kReadBatch) {
    uint4 v[kReadBatch];
#pragma unroll
    for (int k = 0; k < kReadBatch; ++k) v[k] = load_stream16(buf + (r + k) * kWave + lane);
#pragma unroll
    for (int k = 0; k < kReadBatch; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; r < r1; ++r) {
    const uint4 a = load_stream16(buf + r * kWave + lane);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (w == waves - 1)                            // the tail past the last whole row
    for (int64_t i = rows * kWave + lane; i < n16; i += kWave) {
      const uint4 a = load_stream16(buf + i);
      acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
  if (acc == kNever) sink[0] = acc;
}

constexpr int kPeakAcc = 8;   // independent accumulators per wave (128 registers)

__global__ __launch_bounds__(kPeakThreads) void peak_mfma_kernel(int64_t iterations, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & (kWave - 1);
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(0.001f * (float)((lane + j) & 7));
    b[j] = (__bf16)(0.001f * (float)((lane * 3 + j) & 7));
  }
  floatx16 acc[kPeakAcc];
#pragma unroll
  for (int k = 0; k < kPeakAcc; ++k)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[k][i] = 0.f;
  for (int64_t it = 0; it < iterations; ++it) {
#pragma unroll
    for (int k = 0; k < kPeakAcc; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kPeakAcc; ++k)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[k][i];
  if (__float_as_uint(s) == kNever) sink[0] = __float_as_uint(s);
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  return cus;
}

}  // namespace
}  // namespace pkv

extern "C" {

int pkv_peak_read(const void* buf, int64_t bytes, void* sink, void* stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16 != 0 || ((uintptr_t)buf % 16) != 0 || ((uintptr_t)sink % 4) != 0)
    return PKV_EINVAL;
  const int blocks = pkv::device_cus() * 4;       // 4 workgroups of 4 waves per compute unit
  hipLaunchKernelGGL(pkv::peak_read_kernel, dim3(blocks), dim3(pkv::kPeakThreads), 0, (hipStream_t)stream,
                     (const uint4*)buf, bytes / 16, (uint32_t*)sink);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

int pkv_peak_mfma_bf16(int64_t iterations, void* sink, int64_t* flops, void* stream) {
  if (iterations <= 0 || !sink || !flops || ((uintptr_t)sink % 4) != 0) return PKV_EINVAL;
  const int blocks = pkv::device_cus() * 2;       // two waves per SIMD
  *flops = (int64_t)blocks * (pkv::kPeakThreads / pkv::kWave) * iterations * pkv::kPeakAcc * (2LL * 32 * 32 * 16);
  hipLaunchKernelGGL(pkv::peak_mfma_kernel, dim3(blocks), dim3(pkv::kPeakThreads), 0, (hipStream_t)stream,
                     iterations, (uint32_t*)sink);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

}  // extern "C"
