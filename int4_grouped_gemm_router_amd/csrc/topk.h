// Exact top-k (k <= 8) of one token's expert logits inside one wave (gfx950).
//
// diariobitcoin.com, "Perplexity libera Lily, un motor de IA que supera a
// MLX-LM en Apple Silicon", section "Qwen3.6 combina tres cargas de trabajo":
// the router keeps eight of the 256 experts for every token. Selection is on
// the fp32 logits, larger first, equal logits to the lower expert index; -0
// equals +0 and a NaN logit ranks as -inf.
//
// Method: every logit becomes an order-preserving 32-bit key; the k-th
// largest key t is found bit by bit from the top (keep a bit when at least k
// keys are at or above the candidate; one ballot per lane-held key per bit);
// the keys above t and, by ascending index, enough keys equal to t are
// selected and then ranked (a comparison against each other selected key).
#pragma once

#include "device.h"

namespace moe {

__device__ inline uint32_t logit_key(float v) {
  v = v == v ? v : -INFINITY;
  if (v == 0.f) v = 0.f;  // -0 and +0 get the same key
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// key[i] / val[i]: the logit of expert lane + 64 i (key 0 for i >= E / 64;
// real keys are never 0). scratch: 24 words of this wave's LDS. Lane j < k
// returns the expert of rank j and its logit.
__device__ inline void wave_topk(const uint32_t (&key)[4], const float (&val)[4], int k, int lane,
                                 uint32_t* scratch, int& sel_e, float& sel_l) {
  uint32_t t = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = t | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) cnt += __popcll(__ballot(key[i] >= c));
    if (cnt >= k) t = c;
  }
  int need = k;
#pragma unroll
  for (int i = 0; i < 4; ++i) need -= __popcll(__ballot(key[i] > t));
  int base = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint64_t eqm = __ballot(key[i] == t);
    const int before = __popcll(eqm & lanemask_lt());
    const bool sel = key[i] > t || (key[i] == t && before < need);
    need -= min(need, __popcll(eqm));
    const uint64_t sm = __ballot(sel);
    if (sel) {
      const int pos = base + __popcll(sm & lanemask_lt());
      scratch[pos] = key[i];
      scratch[8 + pos] = (uint32_t)(lane + 64 * i);
      scratch[16 + pos] = __float_as_uint(val[i]);
    }
    base += __popcll(sm);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  int rank = -1;
  if (lane < k) {
    const uint32_t my_key = scratch[lane], my_e = scratch[8 + lane];
    rank = 0;
    for (int m = 0; m < k; ++m) {
      const uint32_t km = scratch[m], em = scratch[8 + m];
      rank += (km > my_key) || (km == my_key && em < my_e);
    }
  }
  int src = 0;
  for (int m = 0; m < k; ++m)
    if (__shfl(rank, m) == lane) src = m;
  sel_e = (int)scratch[8 + src];
  sel_l = __uint_as_float(scratch[16 + src]);
}

}  // namespace moe
