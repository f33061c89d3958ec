// Decode-shaped MoE layer for 1..4 tokens (gfx950).
//
// diariobitcoin.com, "Perplexity libera Lily, un motor de IA que supera a
// MLX-LM en Apple Silicon", section "El decode busca mover menos datos": at
// batch 1 there is little weight reuse and memory bandwidth is the ceiling.
// The pass therefore reads only the selected experts' packed weights, with
// coalesced 16-byte loads spread over many waves, each wave issuing all of
// its loads at once; codes are expanded to exact bf16 (128 + q) and
// multiplied by bf16 dot-product instructions with fp32 accumulation.
//
// Three launches on the caller's stream, no host synchronisation:
//   decode_router   fp32 router logits, one block per expert
//   decode_gateup   every block recomputes the top-k of every token from the
//                   logits (one wave per token) and the ascending list of
//                   unique selected experts, then computes gate/up + SwiGLU
//                   for (unique expert or shared expert) x (64-column wave
//                   tile); a token set that picks one expert twice shares its
//                   read; block 0 also writes the routing metadata
//   decode_down     per token and 16-column tile (32 from two tokens on) of
//                   the output: the
//                   down projection of the token's (token, slot) pairs, then
//                   y = bf16(shared + sum over the token's k slots of
//                   weight * output) in a fixed order
#include "kernels.h"
#include "topk.h"

namespace moe {

namespace {

constexpr int kDecWaves = 8;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kK = 8;  // experts per token

__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                         false);
}

// Routing state every decode block needs, rebuilt from the logits.
// Pairs are (token t, rank j) -> index t * kK + j.
struct DecodeRoute {
  int sel_e[kDecodeMaxT * kK];
  float sel_w[kDecodeMaxT * kK];
  int sorted_pair[kDecodeMaxT * kK];
  int pos_of_pair[kDecodeMaxT * kK];
  int uniq[kDecodeMaxT * kK];
  int uniq_first[kDecodeMaxT * kK];  // first sorted position of each unique expert
  int n_uniq;
};

// This thread's four logits of token `wave` (waves >= T load token 0's and
// do not use them): issued early so that their latency overlaps other work.
__device__ inline void load_route_logits(const DecodeArgs& a, float (&lv)[4]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* row = a.logits + (int64_t)(wave < a.T ? wave : 0) * a.E;
#pragma unroll
  for (int i = 0; i < 4; ++i) lv[i] = row[min(lane + 64 * i, a.E - 1)];
}

// Requires kDecThreads threads; every thread must call it, with the logits
// from load_route_logits().
__device__ void decode_route(const DecodeArgs& a, const float (&lv)[4], DecodeRoute& r) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, P = a.T * kK;
  if (wave < a.T) {
    const int t = wave;
    uint32_t key[4];
    float val[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = i < E / 64 ? lv[i] : -INFINITY;
      val[i] = v == v ? v : -INFINITY;  // a NaN logit ranks as -inf
      key[i] = i < E / 64 ? logit_key(val[i]) : 0u;
    }
    int sel;
    float sel_l;
    wave_topk(key, val, kK, lane, sel, sel_l);
    const float top = __shfl(sel_l, 0);
    const float p = lane < kK ? expf(sel_l - top) : 0.f;
    const float z = wave_sum(p);
    if (lane < kK) {
      r.sel_e[t * kK + lane] = sel;
      r.sel_w[t * kK + lane] = p / z;
    }
  }
  __syncthreads();
  if (tid < P) {
    const int e = r.sel_e[tid];
    int pos = 0;
    for (int q = 0; q < P; ++q) {
      const int eq = r.sel_e[q];
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
      e = r.sel_e[r.sorted_pair[lane]];
      first = lane == 0 || r.sel_e[r.sorted_pair[lane - 1]] != e;
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

// Slot of token t in this block's expert (kK for the shared expert), or -1.
__device__ inline void token_slots(const DecodeRoute& r, int expert, int T, int (&jslot)[kDecodeMaxT]) {
#pragma unroll
  for (int t = 0; t < kDecodeMaxT; ++t) {
    jslot[t] = -1;
    if (t < T) {
      if (expert < 0) {
        jslot[t] = kK;
      } else {
#pragma unroll
        for (int j = 0; j < kK; ++j)
          if (r.sel_e[t * kK + j] == expert) jslot[t] = j;
      }
    }
  }
}

// Partial dot products of one lane for one group and one half of a 64-column
// wave tile (column tiles 2 half and 2 half + 1): the lane's 16 inputs of the
// group (x0: k = 8kb.., x1: k = 32 + 8kb..) against its two columns' codes
// (w: the half's 16 bytes); acc[c] += s * sum(x (128 + q)) + (b - 128 s) * sum(x).
__device__ inline void gemv_half(const u32x4 w, const u32x4 sbv, int half, const u32x4 x0,
                                 const u32x4 x1, const ExpandConsts xk, float (&acc)[2]) {
  const uint32_t words[4] = {w.x, w.y, w.z, w.w};
  const uint32_t xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
  const uint32_t s2 = half ? sbv.y : sbv.x, b2 = half ? sbv.w : sbv.z;
  const float sc[2] = {bf16lo(s2), bf16hi(s2)};
  const float bi[2] = {bf16lo(b2), bf16hi(b2)};
  constexpr uint32_t kOnes = 0x3F803F80u;
  float xsum = 0.f;
#pragma unroll
  for (int d = 0; d < 8; ++d) xsum = dot2(xs[d], kOnes, xsum);
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const u32x4 b0 = expand_codes(words[2 * c], xk);
    const u32x4 b1 = expand_codes(words[2 * c + 1], xk);
    float p = 0.f;
    p = dot2(b0.x, xs[0], p);
    p = dot2(b0.y, xs[1], p);
    p = dot2(b0.z, xs[2], p);
    p = dot2(b0.w, xs[3], p);
    p = dot2(b1.x, xs[4], p);
    p = dot2(b1.y, xs[5], p);
    p = dot2(b1.z, xs[6], p);
    p = dot2(b1.w, xs[7], p);
    acc[c] = __builtin_fmaf(bi[c] - 128.0f * sc[c], xsum, __builtin_fmaf(sc[c], p, acc[c]));
  }
}

// One column tile ct of a lane's 64-column wave tile for one group: the
// lane's two code words of ct (w) against its 16 inputs; sw / bw are the
// scale and bias words holding ct's pair (odd: the high half).
__device__ inline void gemv_quarter(const u32x2 w, uint32_t sw, uint32_t bw, int odd, const u32x4 x0,
                                    const u32x4 x1, const ExpandConsts xk, float& acc) {
  const uint32_t xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
  constexpr uint32_t kOnes = 0x3F803F80u;
  float xsum = 0.f;
#pragma unroll
  for (int d = 0; d < 8; ++d) xsum = dot2(xs[d], kOnes, xsum);
  const u32x4 b0 = expand_codes(w.x, xk);
  const u32x4 b1 = expand_codes(w.y, xk);
  float p = 0.f;
  p = dot2(b0.x, xs[0], p);
  p = dot2(b0.y, xs[1], p);
  p = dot2(b0.z, xs[2], p);
  p = dot2(b0.w, xs[3], p);
  p = dot2(b1.x, xs[4], p);
  p = dot2(b1.y, xs[5], p);
  p = dot2(b1.z, xs[6], p);
  p = dot2(b1.w, xs[7], p);
  const float sc = odd ? bf16hi(sw) : bf16lo(sw), bi = odd ? bf16hi(bw) : bf16lo(bw);
  acc = __builtin_fmaf(bi - 128.0f * sc, xsum, __builtin_fmaf(sc, p, acc));
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

// Grid: (k*T + 1) slots x n_wt wave tiles x 2 / NH halves; block: 8 waves
// that split K. Slot k*T: the shared expert (the first blocks of the grid);
// slot < k*T: the slot-th unique selected expert (blocks past the number of
// unique experts exit). A half of
// a 64-column wave tile is 16 gate and the matching 16 up columns; a block
// takes NH halves: one at a single token (twice the blocks to spread 16 MB
// over the chip), both from two tokens on (half the blocks, so that every
// block of a step is resident at once and no second round of blocks pays the
// logits -> top-k -> weights latency chain again). The activations and the
// logits are loaded first; the activations are staged in LDS while the
// logits are in flight; after the routing each wave issues all of its
// groups' weight loads at once.
template <int GPW, int NH>
__global__ __launch_bounds__(kDecThreads) void decode_gateup_kernel(DecodeArgs a) {
  __shared__ DecodeRoute r;
  __shared__ float red[kDecWaves][kDecodeMaxT][NH][kWaveCols / 2];
  __shared__ u32x4 xs_l[kDecodeMaxT * 4096 / 8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, kb = lane >> 4;
  const int T = a.T, P = T * kK, H = a.H, I = a.I;
  const PackGeom geom = pack_geom(I, H, 1);
  // NH = 1: the two half blocks of a wave tile (they read the same
  // scale/bias records) are blocks b and b + 8, which run on one XCD (blocks
  // go to XCD b % 8 in turn), so the second finds the records in that XCD's
  // L2; the grid is rounded up to a multiple of 16 and the extra blocks exit
  int half0 = 0, tile = blockIdx.x;
  if (NH == 1) {
    const int xcd = blockIdx.x & 7, l = blockIdx.x >> 3;
    half0 = l & 1;
    tile = ((l >> 1) << 3) | xcd;
    if (tile >= (P + 1) * geom.n_wt) return;
  }
  // the shared expert's tiles first, then the unique routed experts in
  // order: blocks past the unique experts (which exit at once) come last
  const int sraw = tile / geom.n_wt, wt = tile % geom.n_wt;
  const int slot = sraw == 0 ? P : sraw - 1;
  const int G = geom.G;
  constexpr int gpw = GPW;  // groups per wave (G <= kDecWaves * GPW)
  constexpr int kXPer = kDecodeMaxT * 4096 / 8 / kDecThreads;

  const int n16 = T * H / 8;
  {
    u32x4 xv[kXPer];  // (clamped, unconditional loads: no branches between them)
#pragma unroll
    for (int i = 0; i < kXPer; ++i)
      xv[i] = reinterpret_cast<const u32x4*>(a.x)[min(tid + i * kDecThreads, n16 - 1)];
    float lv[4];
    load_route_logits(a, lv);
    // the activations go to LDS while the logits are still in flight
#pragma unroll
    for (int i = 0; i < kXPer; ++i)
      if (tid + i * kDecThreads < n16) xs_l[tid + i * kDecThreads] = xv[i];
    decode_route(a, lv, r);  // its barriers also publish xs_l
  }

  if (blockIdx.x == 0) {
    if (tid < P) {
      a.topk_idx[tid] = r.sel_e[tid];
      a.topk_w[tid] = r.sel_w[tid];
      if (a.perm) {
        a.perm[r.pos_of_pair[tid]] = tid;
        a.inv_perm[tid] = r.pos_of_pair[tid];
      }
    }
    if (a.hist) {
      for (int e = tid; e < a.E; e += kDecThreads) {
        int c = 0, off = 0;
        for (int q = 0; q < P; ++q) {
          const int eq = r.sel_e[q];
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
  token_slots(r, expert, T, jslot);
  const uint8_t* ebase = expert >= 0 ? a.gu_blob + (int64_t)expert * a.gu_expert_bytes : a.gu_shared;

  // (unconditional loads, groups past G clamped to G - 1 and not used: no
  // branches between the loads)
  // (one scale/bias record serves both halves)
  u32x4 wq[GPW][NH], sb[GPW];
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const int g = min(wave * gpw + gi, G - 1);
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
      wq[gi][hh] = *reinterpret_cast<const u32x4*>(
          ebase + geom.nib_off + (((int64_t)wt * G + g) * 128 + 64 * (half0 + hh) + lane) * 16);
    sb[gi] = *reinterpret_cast<const u32x4*>(ebase + geom.sb_off + (((int64_t)wt * G + g) * 16 + c16) * 16);
  }
  // keep every weight load ahead of the arithmetic (one memory round trip)
  __builtin_amdgcn_sched_barrier(0);

  const ExpandConsts xk = expand_consts();
  float acc[kDecodeMaxT][NH][2];
#pragma unroll
  for (int t = 0; t < kDecodeMaxT; ++t)
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) acc[t][hh][0] = acc[t][hh][1] = 0.f;
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const int g = wave * gpw + gi;
    if (g < G) {
#pragma unroll
      for (int t = 0; t < kDecodeMaxT; ++t) {
        if (t < T && jslot[t] >= 0) {
          const int base16 = (t * H + g * kGroup + 8 * kb) / 8;
#pragma unroll
          for (int hh = 0; hh < NH; ++hh)
            gemv_half(wq[gi][hh], sb[gi], half0 + hh, xs_l[base16], xs_l[base16 + 4], xk, acc[t][hh]);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kDecodeMaxT; ++t)
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        if (t < T) {
          float v = acc[t][hh][c];
          v += __shfl_xor(v, 16);
          v += __shfl_xor(v, 32);
          if (kb == 0) red[wave][t][hh][16 * c + c16] = v;  // c = 0: gate, c = 1: up
        }
      }
  __syncthreads();
  if (tid < T * 16 * NH) {
    const int t = tid / (16 * NH), hh = (tid / 16) % NH, j = tid % 16;
    if (jslot[t] >= 0) {
      float gv = 0.f, uv = 0.f;
      for (int w = 0; w < kDecWaves; ++w) {
        gv += red[w][t][hh][j];
        uv += red[w][t][hh][16 + j];
      }
      const int row = jslot[t] == kK ? kK * T + t : t * kK + jslot[t];
      a.h[(int64_t)row * I + 32 * wt + 16 * (half0 + hh) + j] = f2bf(silu(gv) * uv);
    }
  }
}

// Down projection and combine. Grid: T tokens x H/64 wave tiles x 4 / CT
// blocks of CT column tiles (16 columns each): CT = 1 at one token (128
// blocks, each moving half the bytes of a 32-column block), CT = 2 from two
// tokens on (enough blocks already). Block: 8 waves. A block owns the k + 1
// (token, slot) pairs of its token, slot k being the shared expert. Per
// round of eight groups, wave w takes group w of the round: all the pairs'
// weight loads and, at the same time, the block's copy of the pairs'
// activation rows into LDS, one barrier, and the arithmetic; the column sums
// of each pair stay in registers over the rounds. The expert ids and routing
// weights are read once, up front. Then per pair d[j] = sum over the eight
// waves in order, and y[t] = bf16(d[k] + sum_{j<k} w[t][j] * d[j]), j
// ascending.
constexpr int kDecPairs = kK + 1;

template <int CT>
__global__ __launch_bounds__(kDecThreads) void decode_down_kernel(DecodeArgs a) {
  static_assert(CT == 1 || CT == 2, "one or two column tiles per block");
  constexpr int kSub = 4 / CT;  // blocks per 64-column wave tile
  __shared__ float red[kDecWaves][kDecPairs][16 * CT];
  __shared__ u32x4 hs[kDecPairs][kDecWaves * kGroup / 8];  // [pair][group in round][8 inputs]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, kb = lane >> 4;
  const int T = a.T, H = a.H, I = a.I;
  const PackGeom geom = pack_geom(H, I, 0);
  // CT = 1: the two blocks of one packed half (column tiles 2h and 2h + 1
  // read the same 16-byte code vectors) are blocks b and b + 8, which run on
  // one XCD (blocks go to XCD b % 8 in turn), so the second finds the codes
  // in that XCD's L2 instead of fetching them again (the grid is a multiple
  // of 16: H % 256 == 0)
  int sub, wt, t;
  if (CT == 1) {
    const int xcd = blockIdx.x & 7, l = blockIdx.x >> 3;
    const int m = ((l >> 1) << 3) | xcd;  // (token, wave tile, half)
    sub = 2 * (m & 1) + (l & 1);
    wt = (m >> 1) % geom.n_wt;
    t = (m >> 1) / geom.n_wt;
  } else {
    sub = blockIdx.x % kSub;
    wt = (blockIdx.x / kSub) % geom.n_wt;
    t = (blockIdx.x / kSub) / geom.n_wt;
  }
  const int G = geom.G;
  const int ct0 = CT * sub;  // first column tile of the block
  const int half = ct0 >> 1, odd = ct0 & 1;
  const ExpandConsts xk = expand_consts();
  int ex[kDecPairs];
  float wj[kK];
#pragma unroll
  for (int j = 0; j < kK; ++j) {
    ex[j] = a.topk_idx[t * kK + j];
    wj[j] = a.topk_w[t * kK + j];
  }
  ex[kK] = -1;  // the shared expert
  float acc[kDecPairs][CT];
#pragma unroll
  for (int j = 0; j < kDecPairs; ++j)
#pragma unroll
    for (int c = 0; c < CT; ++c) acc[j][c] = 0.f;
  for (int r0 = 0; r0 < G; r0 += kDecWaves) {
    const int ng = min(kDecWaves, G - r0), g = r0 + wave;
    static_assert(kDecWaves * kGroup / 8 == 64, "LDS row of the round: 64 chunks of 8 inputs");
    // activation rows of this round (independent of the expert ids)
    constexpr int kHsPer = (kDecPairs * kDecWaves * kGroup / 8 + kDecThreads - 1) / kDecThreads;
    // (unconditional, clamped loads: no branches between the loads)
    u32x4 hv[kHsPer];
#pragma unroll
    for (int q = 0; q < kHsPer; ++q) {
      const int i = tid + q * kDecThreads;
      const int j = min(i >> 6, kDecPairs - 1), c = min(i & 63, 8 * ng - 1);
      const int row = j < kK ? t * kK + j : kK * T + t;
      hv[q] = *reinterpret_cast<const u32x4*>(a.h + (int64_t)row * I + r0 * kGroup + 8 * c);
    }
    // per pair: the lane's code words of the block's column tiles (16 bytes
    // of the half, or 8 of them) and its scale / bias record
    u32x4 wq[kDecPairs], sb[kDecPairs];
    const int gl = min(g, G - 1);  // waves past G load group G - 1 and do not use it
#pragma unroll
    for (int j = 0; j < kDecPairs; ++j) {
      const int e = __builtin_amdgcn_readfirstlane(ex[j]);
      const uint8_t* eb = e >= 0 ? a.dn_blob + (int64_t)e * a.dn_expert_bytes : a.dn_shared;
      const uint8_t* np = eb + geom.nib_off + (((int64_t)wt * G + gl) * 128 + 64 * half + lane) * 16;
      if constexpr (CT == 2) {
        wq[j] = *reinterpret_cast<const u32x4*>(np);
      } else {
        const u32x2 v = *reinterpret_cast<const u32x2*>(np + 8 * odd);
        wq[j] = u32x4{v.x, v.y, 0u, 0u};
      }
      sb[j] = *reinterpret_cast<const u32x4*>(eb + geom.sb_off + (((int64_t)wt * G + gl) * 16 + c16) * 16);
    }
    // keep every load of the round ahead of the LDS copy and the arithmetic
    __builtin_amdgcn_sched_barrier(0);
    if (r0 > 0) __syncthreads();  // every wave is done with the previous rows
#pragma unroll
    for (int q = 0; q < kHsPer; ++q) {
      const int i = tid + q * kDecThreads;
      if ((i >> 6) < kDecPairs && (i & 63) < 8 * ng) hs[i >> 6][i & 63] = hv[q];
    }
    __syncthreads();
    if (g < G) {
      const int c = 8 * wave + kb;
#pragma unroll
      for (int j = 0; j < kDecPairs; ++j) {
        if constexpr (CT == 2)  // both column tiles of the half share the row sums
          gemv_half(wq[j], sb[j], half, hs[j][c], hs[j][c + 4], xk, acc[j]);
        else
          gemv_quarter(u32x2{wq[j][0], wq[j][1]}, half ? sb[j].y : sb[j].x, half ? sb[j].w : sb[j].z, odd,
                       hs[j][c], hs[j][c + 4], xk, acc[j][0]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kDecPairs; ++j) {
#pragma unroll
    for (int cc = 0; cc < CT; ++cc) {
      float v = acc[j][cc];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (kb == 0) red[wave][j][16 * cc + c16] = v;
    }
  }
  __syncthreads();
  if (tid < 16 * CT) {
    const int n = tid;
    float d[kK + 1];
#pragma unroll
    for (int j = 0; j <= kK; ++j) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) v += red[w][j][n];
      d[j] = v;
    }
    float s = d[kK];
#pragma unroll
    for (int j = 0; j < kK; ++j) s = __builtin_fmaf(wj[j], d[j], s);
    a.y[(int64_t)t * H + 64 * wt + 16 * ct0 + n] = f2bf(s);
  }
}

namespace {

// Smallest groups-per-wave instantiation that covers G groups with 8 waves.
template <int NH>
hipError_t launch_gateup_nh(int G, dim3 grid, hipStream_t s, const DecodeArgs& a) {
  if (G <= kDecWaves)
    hipLaunchKernelGGL((decode_gateup_kernel<1, NH>), grid, dim3(kDecThreads), 0, s, a);
  else if (G <= 2 * kDecWaves)
    hipLaunchKernelGGL((decode_gateup_kernel<2, NH>), grid, dim3(kDecThreads), 0, s, a);
  else if (G <= 4 * kDecWaves)
    hipLaunchKernelGGL((decode_gateup_kernel<4, NH>), grid, dim3(kDecThreads), 0, s, a);
  else if (G <= 8 * kDecWaves)
    hipLaunchKernelGGL((decode_gateup_kernel<8, NH>), grid, dim3(kDecThreads), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipSuccess;
}

// Half-tile blocks at one token, whole wave tiles from two tokens on.
hipError_t launch_gateup(int G, int slots, int n_wt, int T, hipStream_t s, const DecodeArgs& a) {
  if (T == 1) return launch_gateup_nh<1>(G, dim3((slots * n_wt * 2 + 15) / 16 * 16), s, a);
  return launch_gateup_nh<2>(G, dim3(slots * n_wt), s, a);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s, hipEvent_t* ev) {
  const PackGeom gu = pack_geom(a.I, a.H, 1);
  const PackGeom dn = pack_geom(a.H, a.I, 0);
  if (gu.G > kMaxGroups || dn.G > kMaxGroups || a.T > kDecodeMaxT || a.k != kK)
    return hipErrorInvalidValue;
  const int slots = kK * a.T + 1;  // unique routed experts (at most k*T), then the shared expert
  hipError_t e = hipSuccess;
  if (ev && (e = hipEventRecord(ev[0], s)) != hipSuccess) return e;
  hipLaunchKernelGGL(decode_router_kernel, dim3(a.E), dim3(256), 0, s, a);
  if (ev && (e = hipEventRecord(ev[1], s)) != hipSuccess) return e;
  if ((e = launch_gateup(gu.G, slots, gu.n_wt, a.T, s, a)) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[2], s)) != hipSuccess) return e;
  if (a.T == 1)
    hipLaunchKernelGGL(decode_down_kernel<1>, dim3(a.T * dn.n_wt * 4), dim3(kDecThreads), 0, s, a);  // (a multiple of 16)
  else
    hipLaunchKernelGGL(decode_down_kernel<2>, dim3(a.T * dn.n_wt * 2), dim3(kDecThreads), 0, s, a);
  if (ev && (e = hipEventRecord(ev[3], s)) != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace moe
