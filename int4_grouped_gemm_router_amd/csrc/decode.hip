// Decode-shaped MoE layer for 1..4 tokens (gfx950).
//
// diariobitcoin.com, "Perplexity libera Lily, un motor de IA que supera a
// MLX-LM en Apple Silicon", section "El decode busca mover menos datos": at
// batch 1 there is little weight reuse and memory bandwidth is the ceiling.
// The pass therefore reads only the selected experts' packed weights, once
// each (a token set that picks the same expert twice shares one read), with
// coalesced 16-byte loads spread over many waves so enough bytes are in
// flight; the arithmetic is plain fp32 on the vector ALUs.
//
// Four launches on the caller's stream, no host synchronisation:
//   decode_router   fp32 router logits, one wave per expert
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

namespace moe {

namespace {

constexpr int kDecWaves = 8;

// w = q*s + b applied to a lane's sixteen inputs: returns s * sum(x*q) + b * sum(x)
// through the caller; here only sum(x*q) for one packed word (8 codes).
__device__ inline float dot_codes(uint32_t w, const float* x8) {
  float acc = 0.f;
#pragma unroll
  for (int o = 0; o < 8; ++o) {
    const float q = (float)((w >> (4 * nibble_pos(o))) & 0xFu);
    acc = fmaf(x8[o], q, acc);
  }
  return acc;
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
};

// Requires 256 <= blockDim.x; every thread must call it.
__device__ void decode_route(const DecodeArgs& a, DecodeRoute& r) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, k = a.k, per = E / 64, P = a.T * k;
  if (wave < a.T) {
    const int t = wave;
    float l[4];
    for (int i = 0; i < 4; ++i) {
      const float v = i < per ? a.logits[(int64_t)t * E + lane + 64 * i] : -INFINITY;
      l[i] = v == v ? v : -INFINITY;  // a NaN logit never wins; the selection stays valid
    }
    uint32_t taken = 0;
    int sel = -1;
    float sel_l = 0.f, top = 0.f;
    for (int j = 0; j < k; ++j) {
      float bv = -INFINITY;
      int bi = 0x7FFFFFFF;
      for (int i = 0; i < per; ++i) {
        const int e = lane + 64 * i;
        if (!((taken >> i) & 1u) && (l[i] > bv || (l[i] == bv && e < bi))) {
          bv = l[i];
          bi = e;
        }
      }
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
      if (j == 0) top = bv;
      if (lane == j) {
        sel = bi;
        sel_l = bv;
      }
    }
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

}  // namespace

// Grid: E/4 blocks of 256 threads; wave w computes expert 4*blockIdx.x + w.
__global__ __launch_bounds__(256) void decode_router_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = blockIdx.x * 4 + wave;
  if (e >= a.E) return;
  const float* wr = a.router_w + (int64_t)e * a.H;
  float acc[kDecodeMaxT] = {0.f, 0.f, 0.f, 0.f};
  for (int h0 = lane * 4; h0 < a.H; h0 += 256) {
    const float4 w = *reinterpret_cast<const float4*>(wr + h0);
    for (int t = 0; t < a.T; ++t) {
      const u32x2 xv = *reinterpret_cast<const u32x2*>(a.x + (int64_t)t * a.H + h0);
      acc[t] = fmaf(bf16lo(xv.x), w.x, acc[t]);
      acc[t] = fmaf(bf16hi(xv.x), w.y, acc[t]);
      acc[t] = fmaf(bf16lo(xv.y), w.z, acc[t]);
      acc[t] = fmaf(bf16hi(xv.y), w.w, acc[t]);
    }
  }
  for (int t = 0; t < a.T; ++t) {
    float v = wave_sum(acc[t]);
    if (a.rbias) v += a.rbias[e];
    if (lane == 0) {
      a.logits[(int64_t)t * a.E + e] = v;
      if (a.logits_out) a.logits_out[(int64_t)t * a.E + e] = v;
    }
  }
}

// Grid: (k*T + 1) slots x n_wt wave tiles; block: 512 threads (8 waves split K).
__global__ __launch_bounds__(512) void decode_gateup_kernel(DecodeArgs a) {
  __shared__ DecodeRoute r;
  __shared__ float red[kDecWaves][kDecodeMaxT][kWaveCols];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, kb = lane >> 4;
  const int T = a.T, k = a.k, P = T * k, H = a.H, I = a.I;
  decode_route(a, r);

  const PackGeom geom = pack_geom(I, H, 1);
  const int slot = blockIdx.x / geom.n_wt, wt = blockIdx.x % geom.n_wt;

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
  // tokens of this block: token t uses slot jslot[t] (or -1)
  int jslot[kDecodeMaxT];
  for (int t = 0; t < kDecodeMaxT; ++t) {
    jslot[t] = -1;
    if (t < T) {
      if (expert < 0) {
        jslot[t] = k;  // shared
      } else {
        for (int j = 0; j < k; ++j)
          if (r.sel_e[t][j] == expert) jslot[t] = j;
      }
    }
  }
  const uint8_t* ebase = expert >= 0 ? a.gu_blob + (int64_t)expert * a.gu_expert_bytes : a.gu_shared;
  const int G = geom.G;
  const int gpw = (G + kDecWaves - 1) / kDecWaves;
  float acc[4][kDecodeMaxT];
  for (int ct = 0; ct < 4; ++ct)
    for (int t = 0; t < kDecodeMaxT; ++t) acc[ct][t] = 0.f;
  for (int gi = 0; gi < gpw; ++gi) {
    const int g = wave * gpw + gi;
    if (g >= G) break;
    const uint8_t* nib = ebase + geom.nib_off + (((int64_t)wt * G + g) * 128 + lane) * 16;
    const u32x4 w0 = *reinterpret_cast<const u32x4*>(nib);
    const u32x4 w1 = *reinterpret_cast<const u32x4*>(nib + 1024);
    const u32x4 sbv = *reinterpret_cast<const u32x4*>(
        ebase + geom.sb_off + (((int64_t)wt * G + g) * 16 + c16) * 16);
    const uint32_t words[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    const float s[4] = {bf16lo(sbv.x), bf16hi(sbv.x), bf16lo(sbv.y), bf16hi(sbv.y)};
    const float b[4] = {bf16lo(sbv.z), bf16hi(sbv.z), bf16lo(sbv.w), bf16hi(sbv.w)};
    for (int t = 0; t < T; ++t) {
      if (jslot[t] < 0) continue;
      const uint16_t* xr = a.x + (int64_t)t * H + g * kGroup + 8 * kb;
      const u32x4 v0 = *reinterpret_cast<const u32x4*>(xr);
      const u32x4 v1 = *reinterpret_cast<const u32x4*>(xr + 32);
      const float x0[8] = {bf16lo(v0.x), bf16hi(v0.x), bf16lo(v0.y), bf16hi(v0.y),
                           bf16lo(v0.z), bf16hi(v0.z), bf16lo(v0.w), bf16hi(v0.w)};
      const float x1[8] = {bf16lo(v1.x), bf16hi(v1.x), bf16lo(v1.y), bf16hi(v1.y),
                           bf16lo(v1.z), bf16hi(v1.z), bf16lo(v1.w), bf16hi(v1.w)};
      float xsum = 0.f;
      for (int o = 0; o < 8; ++o) xsum += x0[o] + x1[o];
      for (int ct = 0; ct < 4; ++ct) {
        const float pq = dot_codes(words[2 * ct], x0) + dot_codes(words[2 * ct + 1], x1);
        acc[ct][t] += s[ct] * pq + b[ct] * xsum;
      }
    }
  }
  for (int ct = 0; ct < 4; ++ct)
    for (int t = 0; t < T; ++t) {
      float v = acc[ct][t];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (kb == 0) red[wave][t][16 * ct + c16] = v;
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

// Grid: (k*T + 1) slots x (H/64) wave tiles; block: 512 threads (8 waves split K).
__global__ __launch_bounds__(512) void decode_down_kernel(DecodeArgs a) {
  __shared__ DecodeRoute r;
  __shared__ float red[kDecWaves][kDecodeMaxT][kWaveCols];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, kb = lane >> 4;
  const int T = a.T, k = a.k, P = T * k, H = a.H, I = a.I;
  decode_route(a, r);
  const PackGeom geom = pack_geom(H, I, 0);
  const int slot = blockIdx.x / geom.n_wt, wt = blockIdx.x % geom.n_wt;
  int expert = -1;
  if (slot < P) {
    if (slot >= r.n_uniq) return;
    expert = r.uniq[slot];
  }
  int jslot[kDecodeMaxT];
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
  const uint8_t* ebase = expert >= 0 ? a.dn_blob + (int64_t)expert * a.dn_expert_bytes : a.dn_shared;
  const int G = geom.G;
  const int gpw = (G + kDecWaves - 1) / kDecWaves;
  float acc[4][kDecodeMaxT];
  for (int ct = 0; ct < 4; ++ct)
    for (int t = 0; t < kDecodeMaxT; ++t) acc[ct][t] = 0.f;
  for (int gi = 0; gi < gpw; ++gi) {
    const int g = wave * gpw + gi;
    if (g >= G) break;
    const uint8_t* nib = ebase + geom.nib_off + (((int64_t)wt * G + g) * 128 + lane) * 16;
    const u32x4 w0 = *reinterpret_cast<const u32x4*>(nib);
    const u32x4 w1 = *reinterpret_cast<const u32x4*>(nib + 1024);
    const u32x4 sbv = *reinterpret_cast<const u32x4*>(
        ebase + geom.sb_off + (((int64_t)wt * G + g) * 16 + c16) * 16);
    const uint32_t words[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    const float s[4] = {bf16lo(sbv.x), bf16hi(sbv.x), bf16lo(sbv.y), bf16hi(sbv.y)};
    const float b[4] = {bf16lo(sbv.z), bf16hi(sbv.z), bf16lo(sbv.w), bf16hi(sbv.w)};
    for (int t = 0; t < T; ++t) {
      if (jslot[t] < 0) continue;
      const int row = jslot[t] == k ? k * T + t : t * k + jslot[t];
      const uint16_t* hr = a.h + (int64_t)row * I + g * kGroup + 8 * kb;
      const u32x4 h0 = *reinterpret_cast<const u32x4*>(hr);
      const u32x4 h1 = *reinterpret_cast<const u32x4*>(hr + 32);
      const float x0[8] = {bf16lo(h0.x), bf16hi(h0.x), bf16lo(h0.y), bf16hi(h0.y),
                           bf16lo(h0.z), bf16hi(h0.z), bf16lo(h0.w), bf16hi(h0.w)};
      const float x1[8] = {bf16lo(h1.x), bf16hi(h1.x), bf16lo(h1.y), bf16hi(h1.y),
                           bf16lo(h1.z), bf16hi(h1.z), bf16lo(h1.w), bf16hi(h1.w)};
      float xsum = 0.f;
      for (int o = 0; o < 8; ++o) xsum += x0[o] + x1[o];
      for (int ct = 0; ct < 4; ++ct) {
        const float pq = dot_codes(words[2 * ct], x0) + dot_codes(words[2 * ct + 1], x1);
        acc[ct][t] += s[ct] * pq + b[ct] * xsum;
      }
    }
  }
  for (int ct = 0; ct < 4; ++ct)
    for (int t = 0; t < T; ++t) {
      float v = acc[ct][t];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (kb == 0) red[wave][t][16 * ct + c16] = v;
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

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s, hipEvent_t* ev) {
  const PackGeom gu = pack_geom(a.I, a.H, 1);
  const PackGeom dn = pack_geom(a.H, a.I, 0);
  const int slots = a.k * a.T + 1;
  hipError_t e = hipSuccess;
  if (ev && (e = hipEventRecord(ev[0], s)) != hipSuccess) return e;
  hipLaunchKernelGGL(decode_router_kernel, dim3((a.E + 3) / 4), dim3(256), 0, s, a);
  if (ev && (e = hipEventRecord(ev[1], s)) != hipSuccess) return e;
  hipLaunchKernelGGL(decode_gateup_kernel, dim3(slots * gu.n_wt), dim3(512), 0, s, a);
  if (ev && (e = hipEventRecord(ev[2], s)) != hipSuccess) return e;
  hipLaunchKernelGGL(decode_down_kernel, dim3(slots * dn.n_wt), dim3(512), 0, s, a);
  if (ev && (e = hipEventRecord(ev[3], s)) != hipSuccess) return e;
  if ((e = launch_combine(a.partial, a.topk_w, a.y, a.T, a.H, a.k, s)) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[4], s)) != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace moe
