// Decode-shaped MoE layer for 1..4 tokens (gfx950).
//
// diariobitcoin.com, "Perplexity libera Lily, un motor de IA que supera a
// MLX-LM en Apple Silicon", section "El decode busca mover menos datos": at
// batch 1 there is little weight reuse and memory bandwidth is the ceiling.
// The pass therefore reads only the selected experts' packed weights, once
// each (a token set that picks the same expert twice shares one read), with
// coalesced 16-byte loads spread over many waves, each wave issuing all of
// its loads at once; codes are expanded to exact bf16 (128 + q) and
// multiplied by bf16 dot-product instructions with fp32 accumulation.
//
// Four launches on the caller's stream, no host synchronisation:
//   decode_router   fp32 router logits, one block per expert
//   decode_gateup   top-k of every token (recomputed per block from the
//                   logits), the unique selected experts in ascending order,
//                   then gate/up + SwiGLU for (unique expert or shared expert)
//                   x (64-column wave tile); block 0 also writes the routing
//                   metadata
//   decode_down     down projection per (expert, 64-row tile) into
//                   per-(token, slot) fp32 rows
//   combine         y = bf16(shared + sum over the token's k slots), the same
//                   kernel as the prefill path
#include "kernels.h"
#include "topk.h"

namespace moe {

namespace {

constexpr int kDecWaves = 8;
constexpr int kDecThreads = 64 * kDecWaves;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                         false);
}

// Routing state every decode block needs, rebuilt from the logits.
struct DecodeRoute {
  int sel_e[kDecodeMaxT][8];
  float sel_w[kDecodeMaxT][8];
  int sorted_pair[kDecodeMaxT * 8];
  int pos_of_pair[kDecodeMaxT * 8];
  int uniq[kDecodeMaxT * 8];
  int uniq_first[kDecodeMaxT * 8];  // first sorted position of each unique expert
  int n_uniq;
  uint32_t scratch[kDecodeMaxT][24];
};

// Requires kDecThreads threads; every thread must call it.
__device__ void decode_route(const DecodeArgs& a, DecodeRoute& r) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, k = a.k, P = a.T * k;
  if (wave < a.T) {
    const int t = wave;
    const float* row = a.logits + (int64_t)t * E;
    uint32_t key[4];
    float val[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = i < E / 64 ? row[lane + 64 * i] : -INFINITY;
      val[i] = v == v ? v : -INFINITY;  // a NaN logit ranks as -inf
      key[i] = i < E / 64 ? logit_key(val[i]) : 0u;
    }
    int sel;
    float sel_l;
    wave_topk(key, val, k, lane, r.scratch[t], sel, sel_l);
    const float top = __shfl(sel_l, 0);
    const float p = lane < k ? expf(sel_l - top) : 0.f;
    const float z = wave_sum(p);
    if (lane < k) {
      r.sel_e[t][lane] = sel;
      r.sel_w[t][lane] = p / z;
    }
  }
  __syncthreads();
  if (tid < P) {
    const int e = r.sel_e[tid / k][tid % k];
    int pos = 0;
    for (int q = 0; q < P; ++q) {
      const int eq = r.sel_e[q / k][q % k];
      pos += (eq < e) || (eq == e && q < tid);
    }
    r.sorted_pair[pos] = tid;
    r.pos_of_pair[tid] = pos;
  }
  __syncthreads();
  if (wave == 0) {
    bool first = false;
    int e = -1;
    if (lane < P) {
      const int q = r.sorted_pair[lane];
      e = r.sel_e[q / k][q % k];
      first = lane == 0;
      if (lane > 0) {
        const int q0 = r.sorted_pair[lane - 1];
        first = r.sel_e[q0 / k][q0 % k] != e;
      }
    }
    const uint64_t fm = __ballot(first);
    if (first) {
      const int u = __popcll(fm & lanemask_lt());
      r.uniq[u] = e;
      r.uniq_first[u] = lane;
    }
    if (lane == 0) r.n_uniq = __popcll(fm);
  }
  __syncthreads();
}

// Slot of token t in this block's expert (k for the shared expert), or -1.
__device__ inline void token_slots(const DecodeRoute& r, int expert, int T, int k, int (&jslot)[kDecodeMaxT]) {
#pragma unroll
  for (int t = 0; t < kDecodeMaxT; ++t) {
    jslot[t] = -1;
    if (t < T) {
      if (expert < 0) {
        jslot[t] = k;
      } else {
        for (int j = 0; j < k; ++j)
          if (r.sel_e[t][j] == expert) jslot[t] = j;
      }
    }
  }
}

// Partial dot products of one lane for one group: the lane's 16 inputs of
// the group (x0: k = 8kb.., x1: k = 32 + 8kb..) against its four columns'
// codes; acc[ct] += s * sum(x (128 + q)) + (b - 128 s) * sum(x).
__device__ inline void gemv_group(const u32x4 w0, const u32x4 w1, const u32x4 sbv, const u32x4 x0,
                                  const u32x4 x1, const ExpandConsts xk, float (&acc)[4]) {
  const uint32_t words[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  const uint32_t xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
  const float sc[4] = {bf16lo(sbv.x), bf16hi(sbv.x), bf16lo(sbv.y), bf16hi(sbv.y)};
  const float bi[4] = {bf16lo(sbv.z), bf16hi(sbv.z), bf16lo(sbv.w), bf16hi(sbv.w)};
  constexpr uint32_t kOnes = 0x3F803F80u;
  float xsum = 0.f;
#pragma unroll
  for (int d = 0; d < 8; ++d) xsum = dot2(xs[d], kOnes, xsum);
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const u32x4 b0 = expand_codes(words[2 * ct], xk);
    const u32x4 b1 = expand_codes(words[2 * ct + 1], xk);
    float p = 0.f;
    p = dot2(b0.x, xs[0], p);
    p = dot2(b0.y, xs[1], p);
    p = dot2(b0.z, xs[2], p);
    p = dot2(b0.w, xs[3], p);
    p = dot2(b1.x, xs[4], p);
    p = dot2(b1.y, xs[5], p);
    p = dot2(b1.z, xs[6], p);
    p = dot2(b1.w, xs[7], p);
    acc[ct] = __builtin_fmaf(bi[ct] - 128.0f * sc[ct], xsum, __builtin_fmaf(sc[ct], p, acc[ct]));
  }
}

}  // namespace

// Grid: E blocks of 256 threads; block e computes expert e's logit for every
// token: each thread eight inputs per pass, then a block reduction in a fixed
// order.
__global__ __launch_bounds__(256) void decode_router_kernel(DecodeArgs a) {
  __shared__ float part[4][kDecodeMaxT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e = blockIdx.x;
  const float* wr = a.router_w + (int64_t)e * a.H;
  float acc[kDecodeMaxT] = {0.f, 0.f, 0.f, 0.f};
  for (int h0 = 8 * tid; h0 < a.H; h0 += 8 * 256) {
    const float4 w0 = *reinterpret_cast<const float4*>(wr + h0);
    const float4 w1 = *reinterpret_cast<const float4*>(wr + h0 + 4);
    u32x4 xv[kDecodeMaxT];
#pragma unroll
    for (int t = 0; t < kDecodeMaxT; ++t)
      if (t < a.T) xv[t] = *reinterpret_cast<const u32x4*>(a.x + (int64_t)t * a.H + h0);
#pragma unroll
    for (int t = 0; t < kDecodeMaxT; ++t) {
      if (t < a.T) {
        float v = acc[t];
        v = fmaf(bf16lo(xv[t].x), w0.x, v);
        v = fmaf(bf16hi(xv[t].x), w0.y, v);
        v = fmaf(bf16lo(xv[t].y), w0.z, v);
        v = fmaf(bf16hi(xv[t].y), w0.w, v);
        v = fmaf(bf16lo(xv[t].z), w1.x, v);
        v = fmaf(bf16hi(xv[t].z), w1.y, v);
        v = fmaf(bf16lo(xv[t].w), w1.z, v);
        v = fmaf(bf16hi(xv[t].w), w1.w, v);
        acc[t] = v;
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kDecodeMaxT; ++t) {
    const float v = wave_sum(acc[t]);
    if (lane == 0) part[wave][t] = v;
  }
  __syncthreads();
  if (tid < a.T) {
    float v = ((part[0][tid] + part[1][tid]) + part[2][tid]) + part[3][tid];
    if (a.rbias) v += a.rbias[e];
    a.logits[(int64_t)tid * a.E + e] = v;
    if (a.logits_out) a.logits_out[(int64_t)tid * a.E + e] = v;
  }
}

// Grid: (k*T + 1) slots x n_wt wave tiles; block: 8 waves that split K.
// Slot < k*T: the slot-th unique selected expert (blocks past the number of
// unique experts exit); slot k*T: the shared expert. The tokens' activations
// are staged in LDS while the block recomputes the routing; then each wave
// issues all of its groups' weight loads at once.
template <int GPW>
__global__ __launch_bounds__(kDecThreads) void decode_gateup_kernel(DecodeArgs a) {
  __shared__ DecodeRoute r;
  __shared__ float red[kDecWaves][kDecodeMaxT][kWaveCols];
  __shared__ u32x4 xs_l[kDecodeMaxT * 4096 / 8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, kb = lane >> 4;
  const int T = a.T, k = a.k, P = T * k, H = a.H, I = a.I;
  const PackGeom geom = pack_geom(I, H, 1);
  const int slot = blockIdx.x / geom.n_wt, wt = blockIdx.x % geom.n_wt;
  const int G = geom.G;
  constexpr int gpw = GPW;  // groups per wave (G <= kDecWaves * GPW)

  // activations -> LDS (16 bytes per thread per pass)
  const int n16 = T * H / 8;
  for (int i = tid; i < n16; i += kDecThreads) xs_l[i] = reinterpret_cast<const u32x4*>(a.x)[i];

  decode_route(a, r);

  if (blockIdx.x == 0) {
    if (tid < P) {
      a.topk_idx[tid] = r.sel_e[tid / k][tid % k];
      a.topk_w[tid] = r.sel_w[tid / k][tid % k];
      if (a.perm) {
        a.perm[r.pos_of_pair[tid]] = tid;
        a.inv_perm[tid] = r.pos_of_pair[tid];
      }
    }
    if (a.hist) {
      for (int e = tid; e < a.E; e += blockDim.x) {
        int c = 0, off = 0;
        for (int q = 0; q < P; ++q) {
          const int eq = r.sel_e[q / k][q % k];
          c += eq == e;
          off += eq < e;
        }
        a.hist[e] = c;
        a.offsets[e] = off;
      }
      if (tid == 0) {
        a.offsets[a.E] = P;
        *a.num_blocks = r.n_uniq;
      }
      if (tid < r.n_uniq) {
        const int first = r.uniq_first[tid];
        const int next = tid + 1 < r.n_uniq ? r.uniq_first[tid + 1] : P;
        a.block_map[3 * tid] = r.uniq[tid];
        a.block_map[3 * tid + 1] = first;
        a.block_map[3 * tid + 2] = next - first;
      }
    }
  }

  int expert = -1;
  if (slot < P) {
    if (slot >= r.n_uniq) return;
    expert = r.uniq[slot];
  }
  int jslot[kDecodeMaxT];
  token_slots(r, expert, T, k, jslot);
  const uint8_t* ebase = expert >= 0 ? a.gu_blob + (int64_t)expert * a.gu_expert_bytes : a.gu_shared;

  // all weight loads of this wave's groups first
  u32x4 w0[GPW], w1[GPW], sb[GPW];
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const int g = wave * gpw + gi;
    if (g < G) {
      const uint8_t* nib = ebase + geom.nib_off + (((int64_t)wt * G + g) * 128 + lane) * 16;
      w0[gi] = *reinterpret_cast<const u32x4*>(nib);
      w1[gi] = *reinterpret_cast<const u32x4*>(nib + 1024);
      sb[gi] = *reinterpret_cast<const u32x4*>(ebase + geom.sb_off + (((int64_t)wt * G + g) * 16 + c16) * 16);
    }
  }
  const ExpandConsts xk = expand_consts();
  float acc[kDecodeMaxT][4];
#pragma unroll
  for (int t = 0; t < kDecodeMaxT; ++t)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[t][ct] = 0.f;
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const int g = wave * gpw + gi;
    if (g < G) {
#pragma unroll
      for (int t = 0; t < kDecodeMaxT; ++t) {
        if (t < T && jslot[t] >= 0) {
          const int base16 = (t * H + g * kGroup + 8 * kb) / 8;
          gemv_group(w0[gi], w1[gi], sb[gi], xs_l[base16], xs_l[base16 + 4], xk, acc[t]);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kDecodeMaxT; ++t)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      if (t < T) {
        float v = acc[t][ct];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (kb == 0) red[wave][t][16 * ct + c16] = v;
      }
    }
  __syncthreads();
  if (tid < T * 32) {
    const int t = tid / 32, j = tid % 32;
    if (jslot[t] >= 0) {
      float gv = 0.f, uv = 0.f;
      const int jg = 32 * (j >> 4) + (j & 15);  // gate column of intermediate j; up is 16 later
      for (int w = 0; w < kDecWaves; ++w) {
        gv += red[w][t][jg];
        uv += red[w][t][jg + 16];
      }
      const int row = jslot[t] == k ? k * T + t : t * k + jslot[t];
      a.h[(int64_t)row * I + 32 * wt + j] = f2bf(silu(gv) * uv);
    }
  }
}

// Grid: (k*T + 1) slots x (H/64) wave tiles; block: 8 waves that split K.
template <int GPW>
__global__ __launch_bounds__(kDecThreads) void decode_down_kernel(DecodeArgs a) {
  __shared__ DecodeRoute r;
  __shared__ float red[kDecWaves][kDecodeMaxT][kWaveCols];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, kb = lane >> 4;
  const int T = a.T, k = a.k, P = T * k, H = a.H, I = a.I;
  const PackGeom geom = pack_geom(H, I, 0);
  const int slot = blockIdx.x / geom.n_wt, wt = blockIdx.x % geom.n_wt;
  const int G = geom.G;
  constexpr int gpw = GPW;  // groups per wave (G <= kDecWaves * GPW)
  decode_route(a, r);
  int expert = -1;
  if (slot < P) {
    if (slot >= r.n_uniq) return;
    expert = r.uniq[slot];
  }
  int jslot[kDecodeMaxT];
  token_slots(r, expert, T, k, jslot);
  const uint8_t* ebase = expert >= 0 ? a.dn_blob + (int64_t)expert * a.dn_expert_bytes : a.dn_shared;

  u32x4 w0[GPW], w1[GPW], sb[GPW];
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const int g = wave * gpw + gi;
    if (g < G) {
      const uint8_t* nib = ebase + geom.nib_off + (((int64_t)wt * G + g) * 128 + lane) * 16;
      w0[gi] = *reinterpret_cast<const u32x4*>(nib);
      w1[gi] = *reinterpret_cast<const u32x4*>(nib + 1024);
      sb[gi] = *reinterpret_cast<const u32x4*>(ebase + geom.sb_off + (((int64_t)wt * G + g) * 16 + c16) * 16);
    }
  }
  const ExpandConsts xk = expand_consts();
  float acc[kDecodeMaxT][4];
#pragma unroll
  for (int t = 0; t < kDecodeMaxT; ++t)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[t][ct] = 0.f;
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const int g = wave * gpw + gi;
    if (g < G) {
#pragma unroll
      for (int t = 0; t < kDecodeMaxT; ++t) {
        if (t < T && jslot[t] >= 0) {
          const int row = jslot[t] == k ? k * T + t : t * k + jslot[t];
          const uint16_t* hr = a.h + (int64_t)row * I + g * kGroup + 8 * kb;
          gemv_group(w0[gi], w1[gi], sb[gi], *reinterpret_cast<const u32x4*>(hr),
                     *reinterpret_cast<const u32x4*>(hr + 32), xk, acc[t]);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kDecodeMaxT; ++t)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      if (t < T) {
        float v = acc[t][ct];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (kb == 0) red[wave][t][16 * ct + c16] = v;
      }
    }
  __syncthreads();
  if (tid < T * kWaveCols) {
    const int t = tid / kWaveCols, j = tid % kWaveCols;
    if (jslot[t] >= 0) {
      float d = 0.f;
      for (int w = 0; w < kDecWaves; ++w) d += red[w][t][j];
      a.partial[((int64_t)t * (k + 1) + jslot[t]) * H + 64 * wt + j] = d;
    }
  }
}

namespace {

// Smallest groups-per-wave instantiation that covers G groups with 8 waves.
template <template <int> class KernelSel>
hipError_t launch_gpw(int G, dim3 grid, hipStream_t s, const DecodeArgs& a) {
  if (G <= kDecWaves)
    hipLaunchKernelGGL(KernelSel<1>::fn(), grid, dim3(kDecThreads), 0, s, a);
  else if (G <= 2 * kDecWaves)
    hipLaunchKernelGGL(KernelSel<2>::fn(), grid, dim3(kDecThreads), 0, s, a);
  else if (G <= 4 * kDecWaves)
    hipLaunchKernelGGL(KernelSel<4>::fn(), grid, dim3(kDecThreads), 0, s, a);
  else if (G <= 8 * kDecWaves)
    hipLaunchKernelGGL(KernelSel<8>::fn(), grid, dim3(kDecThreads), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipSuccess;
}

template <int GPW>
struct GateUpSel {
  static auto fn() { return decode_gateup_kernel<GPW>; }
};
template <int GPW>
struct DownSel {
  static auto fn() { return decode_down_kernel<GPW>; }
};

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s, hipEvent_t* ev) {
  const PackGeom gu = pack_geom(a.I, a.H, 1);
  const PackGeom dn = pack_geom(a.H, a.I, 0);
  if (gu.G > kMaxGroups || dn.G > kMaxGroups || a.T > kDecodeMaxT) return hipErrorInvalidValue;
  const int slots = a.k * a.T + 1;
  hipError_t e = hipSuccess;
  if (ev && (e = hipEventRecord(ev[0], s)) != hipSuccess) return e;
  hipLaunchKernelGGL(decode_router_kernel, dim3(a.E), dim3(256), 0, s, a);
  if (ev && (e = hipEventRecord(ev[1], s)) != hipSuccess) return e;
  if ((e = launch_gpw<GateUpSel>(gu.G, dim3(slots * gu.n_wt), s, a)) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[2], s)) != hipSuccess) return e;
  if ((e = launch_gpw<DownSel>(dn.G, dim3(slots * dn.n_wt), s, a)) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[3], s)) != hipSuccess) return e;
  if ((e = launch_combine(a.partial, a.topk_w, a.y, a.T, a.H, a.k, s)) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[4], s)) != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace moe
