// Measured ceilings of the device (gfx950): a streaming read of a buffer
// larger than the last-level cache, and a loop of independent bf16 matrix-core
// operations. They are not part of the layer: they give the achievable HBM
// read bandwidth and bf16 MFMA rate, so that roofline fractions can be stated
// against measured ceilings as well as against the published peaks.
#include "../../include/moe_int4.h"
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

// Each wave runs kMfmaChains independent chains of 16x16x32 bf16 MFMAs.
// Operands: with `random`, four A and four B fragments per lane hold random
// bf16 values of magnitude in [0.5, 1) and random sign (a hash of the lane's
// global index), and consecutive operations take different ones, so the
// matrix cores switch as they do on layer data; otherwise the operands are
// nearly constant. The device draws more power in the first case and
// sustains a lower shader clock. If `clocks` is given, thread 0 of each block
// writes the block's real-time ticks (s_memrealtime, 100 MHz) and shader
// clock ticks (s_memtime) over its loop, from which the clock follows.
__device__ inline uint32_t ceil_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x85EBCA6Bu;
  x ^= x >> 13;
  x *= 0xC2B2AE35u;
  return x ^ (x >> 16);
}

__global__ __launch_bounds__(kCeilThreads) void ceiling_mfma_kernel(int iters, int random, float* sink,
                                                                    unsigned long long* clocks) {
  const uint32_t l = threadIdx.x, g = blockIdx.x * kCeilThreads + l;
  u32x4 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t ra = (ceil_hash(g * 32u + 4u * i + e) & 0x807F807Fu) | 0x3F003F00u;
      const uint32_t rb = (ceil_hash(g * 32u + 16u + 4u * i + e) & 0x807F807Fu) | 0x3F003F00u;
      a[i][e] = random ? ra : (e == 0 ? (0x3F80u | (l << 16)) : 0x3F813F81u);
      b[i][e] = random ? rb : (e == 1 ? (0x3F85u | (l << 16)) : 0x3F843F84u);
    }
  f32x4 acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) acc[c] = f32x4{(float)c, 0.f, 0.f, 0.f};
  const unsigned long long t0 = __builtin_amdgcn_s_memrealtime(), c0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int c = 0; c < kMfmaChains; ++c) acc[c] = mfma16(a[c % 4], b[(c / 4 + j) % 4], acc[c]);
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memrealtime(), c1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  if (__float_as_uint(s) == kNever) sink[0] = s;
  if (clocks && l == 0) {
    clocks[2 * blockIdx.x] = t1 - t0;
    clocks[2 * blockIdx.x + 1] = c1 - c0;
  }
}

}  // namespace

}  // namespace moe

extern "C" {

int moe_ceiling_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16) return MOE_EINVAL;
  hipLaunchKernelGGL(moe::ceiling_read_kernel, dim3(moe::kReadBlocks), dim3(moe::kCeilThreads), 0,
                     (hipStream_t)stream, static_cast<const moe::u32x4*>(buf), (int64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

// iters loop trips of 4 kMfmaChains operations per wave; clocks (optional)
// receives 2 values per block (kMfmaBlocks blocks): real-time and shader-clock
// ticks over the loop.
int moe_ceiling_mfma(int32_t iters, int32_t random, float* sink, unsigned long long* clocks,
                     double* flops, void* stream) {
  if (iters <= 0 || !sink || !flops) return MOE_EINVAL;
  *flops = (double)moe::kMfmaBlocks * (moe::kCeilThreads / 64) * moe::kMfmaChains * 4.0 * iters *
           (16.0 * 16 * 32 * 2);
  hipLaunchKernelGGL(moe::ceiling_mfma_kernel, dim3(moe::kMfmaBlocks), dim3(moe::kCeilThreads), 0,
                     (hipStream_t)stream, (int)iters, (int)random, sink, clocks);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

}  // extern "C"
