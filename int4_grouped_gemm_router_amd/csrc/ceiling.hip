// Measured ceilings of the device (gfx950): a streaming read of a buffer
// larger than the last-level cache, and a loop of independent bf16 matrix-core
// operations. They are not part of the layer: they give the achievable HBM
// read bandwidth and bf16 MFMA rate, so that roofline fractions can be stated
// against measured ceilings as well as against the published peaks.
#include "device.h"

namespace moe {

namespace {

constexpr int kCeilThreads = 256;
constexpr int kReadBlocks = 2048;  // 8 blocks per compute unit
constexpr int kMfmaBlocks = 1024;  // four waves per SIMD
constexpr int kMfmaChains = 8;     // independent accumulators per wave
constexpr uint32_t kNever = 0x9E3779B9u;

// Block b reads the b-th contiguous 1/gridDim of the buffer (whole DRAM
// pages per block measured faster than a grid-stride order), each lane eight
// 16-byte vectors in flight per step; the XOR of everything a lane read
// decides a store that practically never happens, so no load can be dropped.
__global__ __launch_bounds__(kCeilThreads) void ceiling_read_kernel(const u32x4* __restrict__ p,
                                                                    int64_t n16, uint32_t* sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = (int64_t)blockIdx.x * per, b1 = min(b0 + per, n16);
  u32x4 acc = {0u, 0u, 0u, 0u};
  int64_t i = b0 + threadIdx.x;
  for (; i + 7 * kCeilThreads < b1; i += 8 * kCeilThreads) {
    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = p[i + j * kCeilThreads];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= v[j];
  }
  for (; i < b1; i += kCeilThreads) acc ^= p[i];
  const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (x == kNever) sink[0] = x;
}

// Each wave runs kMfmaChains independent chains of 16x16x32 bf16 MFMAs on
// register operands derived from the lane index.
__global__ __launch_bounds__(kCeilThreads) void ceiling_mfma_kernel(int iters, float* sink) {
  const uint32_t l = threadIdx.x;
  const u32x4 a = {0x3F80u | (l << 16), 0x3F81u, 0x3F82u ^ l, 0x3F83u};
  const u32x4 b = {0x3F84u, 0x3F85u | (l << 16), 0x3F86u, 0x3F87u ^ l};
  f32x4 acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) acc[c] = f32x4{(float)c, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) acc[c] = mfma16(a, b, acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  if (__float_as_uint(s) == kNever) sink[0] = s;
}

}  // namespace

}  // namespace moe

extern "C" {

int moe_ceiling_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16) return -1;
  hipLaunchKernelGGL(moe::ceiling_read_kernel, dim3(moe::kReadBlocks), dim3(moe::kCeilThreads), 0,
                     (hipStream_t)stream, static_cast<const moe::u32x4*>(buf), (int64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int moe_ceiling_mfma(int32_t iters, float* sink, double* flops, void* stream) {
  if (iters <= 0 || !sink || !flops) return -1;
  *flops = (double)moe::kMfmaBlocks * (moe::kCeilThreads / 64) * moe::kMfmaChains * iters * (16.0 * 16 * 32 * 2);
  hipLaunchKernelGGL(moe::ceiling_mfma_kernel, dim3(moe::kMfmaBlocks), dim3(moe::kCeilThreads), 0,
                     (hipStream_t)stream, (int)iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
