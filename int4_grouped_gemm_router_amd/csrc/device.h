// Device helpers for the gfx950 kernels: vector types, the 16x16x32 bf16
// matrix-core op, int4 -> bf16 expansion and small wave primitives.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// D = A(16x32) * B(32x16) + C; lane l holds A row l%16 / B column l%16 and
// eight consecutive K-values of block l/16; D lane l holds column l%16 and
// rows 4*(l/16) .. 4*(l/16)+3.
__device__ inline f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Constants of the int4 -> bf16 expansion, materialised once per kernel in
// registers. Hiding their values from the optimiser lets the instruction
// selector fuse (w & mask) | magic into one v_and_or_b32 (gfx9 VOP3 forms take
// no literal, so with literal constants it emits a separate AND and OR); the
// fused op is ordinary compiler output, so the hazard recognizer still sees
// it when it is interleaved with matrix-core instructions.
struct ExpandConsts {
  uint32_t mask, magic;
};

__device__ inline ExpandConsts expand_consts() {
  ExpandConsts k;
  asm volatile("s_mov_b32 %0, 0x000F000F" : "=s"(k.mask));
  asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(k.magic));
  return k;
}

// Eight int4 codes (one u32 in the packed order) -> eight exact bf16 values
// 128 + q, two per 32-bit lane word: bf16 0x4300 | q is 128 + q exactly.
__device__ inline u32x4 expand_codes(uint32_t w, ExpandConsts k) {
  u32x4 r;
  r.x = (w & k.mask) | k.magic;
  r.y = ((w >> 4) & k.mask) | k.magic;
  r.z = ((w >> 8) & k.mask) | k.magic;
  r.w = ((w >> 12) & k.mask) | k.magic;
  return r;
}

__device__ inline float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ inline float bf16hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ inline float bf16f(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// Round-to-nearest-even fp32 -> bf16 bits: the conversion instruction of
// this target (v_cvt_pk_bf16_f32), bit-identical on finite inputs to adding
// 0x7FFF plus the kept LSB and truncating.
__device__ inline uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two values rounded to bf16 in one conversion: lo in bits 0..15, hi in 16..31.
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// Split an fp32 value into a truncated bf16 head and the bf16 of the rest.
__device__ inline void split_hi_lo(float v, uint16_t& hi, uint16_t& lo) {
  const uint32_t h = __float_as_uint(v) & 0xFFFF0000u;
  const float r = v - __uint_as_float(h);
  hi = (uint16_t)(h >> 16);
  lo = (uint16_t)(__float_as_uint(r) >> 16);
}

// silu(z) = z / (1 + e^-z) with the hardware exponential and reciprocal
// (about one ulp each in fp32; every use rounds the result to bf16). An IEEE
// division here cost about four times as many instructions, which made it
// the largest part of the gate/up epilogue.
__device__ inline float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Barrier for LDS hand-off only: waits for this wave's LDS operations, not
// for its outstanding global loads (a plain __syncthreads would drain them).
// The memory clobber keeps the compiler from moving LDS or global memory
// operations across it.
__device__ inline void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ inline float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Lanes of the wave whose key equals this lane's key (keys < 2^bits).
__device__ inline uint64_t match_any(uint32_t key, int bits) {
  uint64_t mask = __ballot(1);
  for (int b = 0; b < bits; ++b) {
    const bool bit = (key >> b) & 1u;
    const uint64_t bb = __ballot(bit);
    mask &= bit ? bb : ~bb;
  }
  return mask;
}

__device__ inline uint64_t lanemask_lt() {
  const int l = threadIdx.x & 63;
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

}  // namespace moe
