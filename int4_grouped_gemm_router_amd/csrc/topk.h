// Exact top-k (k <= 8) of one token's expert logits inside one wave (gfx950).
//
// diariobitcoin.com, "Perplexity libera Lily, un motor de IA que supera a
// MLX-LM en Apple Silicon", section "Qwen3.6 combina tres cargas de trabajo":
// the router keeps eight of the 256 experts for every token. Selection is on
// the fp32 logits, larger first, equal logits to the lower expert index; -0
// equals +0 and a NaN logit ranks as -inf.
//
// Method: every logit becomes an order-preserving 32-bit key and each lane
// sorts its four (key descending, expert ascending). Then k rounds: the
// largest head key of the 64 lanes comes from a cross-lane max (DPP within
// rows of 16, then the four row results); among lanes whose head equals it,
// the lowest expert index wins (a second, min reduction, only when more than
// one lane ties); the winner's lane drops its head.
#pragma once

#include "device.h"

namespace moe {

__device__ inline uint32_t logit_key(float v) {
  v = v == v ? v : -INFINITY;
  if (v == 0.f) v = 0.f;  // -0 and +0 get the same key
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// v from another lane of the same row of 16 (DPP control CTRL).
template <int CTRL>
__device__ inline uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}

// Maximum / minimum of v over the 64 lanes of a fully active wave, returned
// to every lane: lane ^ 1, lane ^ 2, mirror within 8, mirror within 16, then
// the four rows' results.
__device__ inline uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]
  v = max(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]
  v = max(v, dpp<0x141>(v));  // row_half_mirror
  v = max(v, dpp<0x140>(v));  // row_mirror
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}

__device__ inline uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp<0xB1>(v));
  v = min(v, dpp<0x4E>(v));
  v = min(v, dpp<0x141>(v));
  v = min(v, dpp<0x140>(v));
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return min(min(a, b), min(c, d));
}

// key[i] / val[i]: the logit of expert lane + 64 i (key 0 for i >= E / 64;
// real keys are never 0). Every lane of the wave must be active. Lane j < k
// returns the expert of rank j and its logit.
__device__ inline void wave_topk(const uint32_t (&key)[4], const float (&val)[4], int k, int lane,
                                 int& sel_e, float& sel_l) {
  uint32_t hk[4], he[4];
  float hv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hk[i] = key[i];
    he[i] = (uint32_t)(lane + 64 * i);
    hv[i] = val[i];
  }
  auto order = [&](int x, int y) {  // positions x < y: the larger (key, -expert) first
    const bool sw = hk[y] > hk[x] || (hk[y] == hk[x] && he[y] < he[x]);
    const uint32_t k0 = hk[x], e0 = he[x];
    const float v0 = hv[x];
    hk[x] = sw ? hk[y] : k0;
    he[x] = sw ? he[y] : e0;
    hv[x] = sw ? hv[y] : v0;
    hk[y] = sw ? k0 : hk[y];
    he[y] = sw ? e0 : he[y];
    hv[y] = sw ? v0 : hv[y];
  };
  order(0, 1);
  order(2, 3);
  order(0, 2);
  order(1, 3);
  order(1, 2);
  sel_e = -1;
  sel_l = 0.f;
  for (int r = 0; r < k; ++r) {
    const uint32_t m = wave_max_u32(hk[0]);
    const bool at_max = hk[0] == m;
    uint64_t cand = __ballot(at_max);
    if (__popcll(cand) > 1) {  // equal logits in several lanes: lowest expert first
      const uint32_t emin = wave_min_u32(at_max ? he[0] : 0xFFFFFFFFu);
      cand = __ballot(at_max && he[0] == emin);
    }
    const int win = __builtin_ctzll(cand);
    const int we = __builtin_amdgcn_readlane((int)he[0], win);
    const float wv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hv[0]), win));
    if (lane == r) {
      sel_e = we;
      sel_l = wv;
    }
    if (lane == win) {
      hk[0] = hk[1];
      hk[1] = hk[2];
      hk[2] = hk[3];
      hk[3] = 0u;
      he[0] = he[1];
      he[1] = he[2];
      he[2] = he[3];
      hv[0] = hv[1];
      hv[1] = hv[2];
      hv[2] = hv[3];
    }
  }
}

}  // namespace moe
