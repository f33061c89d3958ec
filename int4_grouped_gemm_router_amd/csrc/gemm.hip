// Grouped expert GEMMs with fused int4 expansion (gfx950, bf16 matrix cores).
//
// diariobitcoin.com, "Perplexity libera Lily, un motor de IA que supera a
// MLX-LM en Apple Silicon", section "Las optimizaciones en el prefill": the
// grouped expert GEMM reconstructs the 4-bit weights block by block in on-chip
// memory with fp32 accumulation and never writes expanded weights back; the
// expert GEMMs are about 90% of prefill time.
//
// One work item is up to 64 rows of one expert (rows are (token, slot) pairs
// in expert-sorted order, or tokens for the shared expert) and one 256-column
// tile of the output; four waves each own 64 columns. Per 64-input group:
//   - five groups are in flight per wave: the activation rows of a group,
//     gathered through the routing permutation, arrive in an LDS ring by
//     asynchronous global -> LDS copies; each wave's 2 KB of packed codes and
//     128 B of scales arrive in a register ring as contiguous 1 KB wave loads;
//     one barrier per group;
//   - each code is expanded to the exact bf16 value 128 + q with two bit
//     operations (no arithmetic);
//   - the matrix cores form P = x . (128 + q) for the group in fp32 and the
//     group's scale is applied on the accumulator: acc += s * P.
// The bias term sum_g (b - 128 s) * sum_{c in g} x_c is added at the end by
// three more matrix-core K-steps over precomputed per-group sums of the
// activations (hi/lo bf16 halves) and the per-group (b - 128 s) (hi/lo).
// Algebraically this is x . (q*s + b) with the weights used exactly.
//
// The operands of the bias term are fetched in the prologue (so the
// epilogue issues no global load): the (bias, scale) words of the lane's
// groups into registers, the per-row group sums into LDS.
//
// Epilogues: gate/up -> h = silu(gate) * up rounded to bf16, plus the per-64
// column sums of h for the down GEMM's bias term; down -> the output in fp32
// at [token][slot]; the combine kernel then forms y = bf16(shared + sum over
// the k slots of weight * output) in a fixed order, so the result is
// deterministic.
#include "kernels.h"

namespace moe {

// Groups in flight: the packed codes and scales of a wave are private to it,
// so they land in a register ring; the gathered activation rows are shared by
// the block and land in an LDS ring through asynchronous global -> LDS copies.
// kStages - 1 groups are in flight per wave (about 90 KB per CU at two blocks
// per CU), which is what the memory system needs to stream near its peak.
constexpr int kStages = 6;
constexpr int kXStage = kItemRows * 128;        // gathered activations per group: 4 KB
constexpr int kSub = kItemRows / 16;            // 16-row MFMA subtiles per item

typedef __attribute__((address_space(3))) void lds_void;

// Asynchronous 16-byte global -> LDS copy; lane l writes dst + 16 l.
__device__ inline void dma16(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, 0);
}

// Wait until at most `groups` later load groups (XI + 3 loads each) are pending.
template <int XI>
__device__ inline void wait_groups(int groups) {
  constexpr int per = XI + 3;
  static_assert(kStages - 2 <= 4, "wait_groups covers up to four pending groups");
  if (groups >= 4) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * per) : "memory");
  } else if (groups == 3) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * per) : "memory");
  } else if (groups == 2) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * per) : "memory");
  } else if (groups == 1) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(per) : "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

constexpr int kMaxX3 = 96;                      // extra-K entries staged in LDS (fast path)

struct Lds {
  u32x4 x[kStages][kXStage / 16];               // [stage][ms][c 8][row 16]
  u32x4 x3[kMaxX3 / 8][64];                     // per-row group sums: [chunk][row]
  int rowidx[kItemRows];
  int outrow[kItemRows];
  float red[4][kItemRows];
};

// Main K loop, one 64-input group per step: wait for the group's loads, one
// barrier (the activation stage is shared), issue the loads of the group
// kStages - 1 ahead, expand the codes to bf16 and run the matrix cores.
// XI = activation copies per wave per group (1 for items of up to 32 rows,
// 2 for up to 64).
template <int XI>
__device__ inline void main_loop(const GemmArgs& a, Lds& L, int rows, int nsub,
                                 const uint8_t* nib, const uint8_t* scl, f32x4 (&acc)[kSub][4]) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, kb = lane >> 4;
  const int K = a.K, G = K / kGroup;
  // activation copies: instruction i of this wave covers units u = 64 (wave + 4 i) + lane
  const uint16_t* xsrc[XI];
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int u = 64 * (wave + 4 * i) + lane;
    const int m = (u >> 7) * 16 + (u & 15);
    xsrc[i] = a.act + (int64_t)L.rowidx[m < rows ? m : 0] * K + 8 * ((u >> 4) & 7);
  }
  const uint8_t* nsrc = nib + lane * 16;
  const uint8_t* ssrc = scl + c16 * 8;
  const ExpandConsts xk = expand_consts();
  u32x4 wq[kStages][2];
  u32x2 sq[kStages];
  auto issue = [&](int g, int slot) {
#pragma unroll
    for (int i = 0; i < XI; ++i) dma16(xsrc[i] + g * kGroup, &L.x[slot][64 * (wave + 4 * i)]);
    wq[slot][0] = *reinterpret_cast<const u32x4*>(nsrc + (int64_t)g * kNibBytes);
    wq[slot][1] = *reinterpret_cast<const u32x4*>(nsrc + (int64_t)g * kNibBytes + 1024);
    sq[slot] = *reinterpret_cast<const u32x2*>(ssrc + (int64_t)g * kSclBytes);
  };
#pragma unroll
  for (int d = 0; d < kStages - 1; ++d)
    if (d < G) issue(d, d);

  for (int g0 = 0; g0 < G; g0 += kStages) {
#pragma unroll
    for (int d = 0; d < kStages; ++d) {
      const int g = g0 + d;
      if (g >= G) break;
      wait_groups<XI>(min(kStages - 2, G - 1 - g));
      // Barrier that is also a compiler memory barrier: no LDS read of this
      // stage may move above it and no copy into the stage freed by the
      // previous step may move above it (a bare s_barrier builtin allows both).
      lds_barrier();
      if (g + kStages - 1 < G) issue(g + kStages - 1, (d + kStages - 1) % kStages);
      const uint32_t words[8] = {wq[d][0].x, wq[d][0].y, wq[d][0].z, wq[d][0].w,
                                 wq[d][1].x, wq[d][1].y, wq[d][1].z, wq[d][1].w};
      const float s[4] = {bf16lo(sq[d].x), bf16hi(sq[d].x), bf16lo(sq[d].y), bf16hi(sq[d].y)};
      u32x4 ax[2 * XI][2];
#pragma unroll
      for (int ms = 0; ms < 2 * XI; ++ms) {
        ax[ms][0] = L.x[d][(ms * 8 + kb) * 16 + c16];
        ax[ms][1] = L.x[d][(ms * 8 + 4 + kb) * 16 + c16];
      }
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const u32x4 b0 = expand_codes(words[2 * ct], xk);
        const u32x4 b1 = expand_codes(words[2 * ct + 1], xk);
#pragma unroll
        for (int ms = 0; ms < 2 * XI; ++ms) {
          if (ms < nsub) {
            f32x4 p = mfma16(ax[ms][0], b0, f32x4{0.f, 0.f, 0.f, 0.f});
            p = mfma16(ax[ms][1], b1, p);
            acc[ms][ct] += s[ct] * p;
          }
        }
      }
    }
  }
}

// B operand of the bias term for one lane: eight consecutive groups g0.. of
// (b - 128 s) for its four columns, as truncated-bf16 heads (hi) and the bf16
// of the remainders (lo).
__device__ inline void bias_operands(const u32x4 (&bv)[4], const u32x2 (&sv)[8], u32x4 (&hi)[4],
                                     u32x4 (&lo)[4]) {
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const uint32_t bw[4] = {bv[ct].x, bv[ct].y, bv[ct].z, bv[ct].w};
    uint32_t h[4], l[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint16_t hh[2], ll[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int o = 2 * d + e;
        const float b = e ? bf16hi(bw[d]) : bf16lo(bw[d]);
        const uint32_t sw = (ct < 2) ? sv[o].x : sv[o].y;
        const float sc = (ct & 1) ? bf16hi(sw) : bf16lo(sw);
        split_hi_lo(b - 128.0f * sc, hh[e], ll[e]);
      }
      h[d] = hh[0] | ((uint32_t)hh[1] << 16);
      l[d] = ll[0] | ((uint32_t)ll[1] << 16);
    }
    hi[ct] = u32x4{h[0], h[1], h[2], h[3]};
    lo[ct] = u32x4{l[0], l[1], l[2], l[3]};
  }
}

template <int MODE>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, kb = lane >> 4;

  // Block ids are dispatched round-robin over the 8 XCDs; keep the column
  // tiles of one item on one XCD so its gathered rows are shared in L2.
  const int bid = blockIdx.x;
  const int q8 = bid >> 3;
  const int slot = (q8 / a.n_tiles) * 8 + (bid & 7);
  const int nt = q8 % a.n_tiles;

  int expert = -1, row0 = 0, rows = 0, token0 = 0;
  if (slot < a.routed_slots) {
    if (slot >= *a.num_items) return;
    expert = a.items[3 * slot];
    row0 = a.items[3 * slot + 1];
    rows = a.items[3 * slot + 2];
  } else if (slot < a.routed_slots + a.shared_slots) {
    token0 = (slot - a.routed_slots) * kItemRows;
    rows = min(kItemRows, a.T - token0);
    row0 = a.k * a.T + token0;
  } else {
    return;
  }
  if (rows <= 0) return;

  const int K = a.K, G = K / kGroup;
  const PackGeom geom = pack_geom(a.N, K, a.paired);
  const int Gp = geom.Gp;
  const int wt = nt * 4 + wave;
  const uint8_t* ebase = expert >= 0 ? a.blob + (int64_t)expert * a.expert_bytes : a.shared_blob;
  const uint8_t* nib = ebase + geom.nib_off + (int64_t)wt * G * kNibBytes;
  const uint8_t* scl = ebase + geom.scl_off + (int64_t)wt * G * kSclBytes;
  const uint8_t* bia = ebase + geom.bia_off;

  __shared__ Lds L;

  // Row bookkeeping. The down GEMM's output row (token, slot) comes from the
  // permutation; it is only needed by the epilogue, so its load stays in
  // flight through the main loop.
  int perm_p = 0;
  if (tid < kItemRows) {
    int ri = 0;
    if (tid < rows) {
      if (MODE == kGateUp) {
        ri = expert >= 0 ? a.perm[row0 + tid] / a.k : token0 + tid;
      } else {
        ri = row0 + tid;
        if (expert >= 0) perm_p = a.perm[row0 + tid];
      }
    }
    L.rowidx[tid] = ri;
  }
  __syncthreads();

  // Bias-term operands (fast path: every lane uses one run of eight groups,
  // true for Gp <= 32 and Kx <= kMaxX3): the raw bias and scale loads are
  // issued here and consumed after the main loop, and the per-row group
  // sums of the activations are copied into LDS.
  const bool fast = Gp <= 32 && a.Kx <= kMaxX3;
  const int g0 = (8 * kb) % Gp;
  u32x4 bv[4];
  u32x2 sv[8];
  if (fast) {
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
      bv[ct] = *reinterpret_cast<const u32x4*>(bia + (((int64_t)wt * kWaveCols + 16 * ct + c16) * Gp + g0) * 2);
#pragma unroll
    for (int o = 0; o < 8; ++o)
      sv[o] = g0 + o < G ? *reinterpret_cast<const u32x2*>(scl + ((int64_t)(g0 + o) * 16 + c16) * 8)
                         : u32x2{0u, 0u};
    const int row = lane < rows ? lane : 0;  // lanes past the item copy row 0 (unused)
    for (int c = wave; c < a.Kx / 8; c += 4)
      dma16(a.act3 + (int64_t)L.rowidx[row] * a.Kx + 8 * c, &L.x3[c][0]);
  }

  const int nsub = (rows + 15) >> 4;
  f32x4 acc[kSub][4];
  for (int ms = 0; ms < kSub; ++ms)
    for (int ct = 0; ct < 4; ++ct) acc[ms][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  main_loop<kItemRows / 32>(a, L, rows, nsub, nib, scl, acc);

  // bias term: sum_g (b - 128 s)[col][g] * xsum[row][g], as extra K-steps
  // (three segments of Gp entries: hi*hi, hi*lo, lo*hi; zero padding after)
  if (fast) {
    u32x4 hi[4], lo[4];
    bias_operands(bv, sv, hi, lo);
    for (int k0s = 0; k0s < a.Kx; k0s += 32) {
      const int seg = (k0s + 8 * kb) / Gp;
      u32x4 be[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        be[ct] = seg == 1 ? lo[ct] : (seg < 3 ? hi[ct] : u32x4{0u, 0u, 0u, 0u});
#pragma unroll
      for (int ms = 0; ms < kSub; ++ms) {
        if (ms < nsub) {
          const u32x4 ax = L.x3[k0s / 8 + kb][ms * 16 + c16];
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) acc[ms][ct] = mfma16(ax, be[ct], acc[ms][ct]);
        }
      }
    }
  } else {
    for (int k0s = 0; k0s < a.Kx; k0s += 32) {
      const int k0 = k0s + 8 * kb;
      const int seg = k0 / Gp, gg0 = k0 % Gp;
      u32x4 be[4];
      for (int ct = 0; ct < 4; ++ct) be[ct] = u32x4{0u, 0u, 0u, 0u};
      if (seg < 3) {
        u32x4 b8[4];
        u32x2 s8[8];
        for (int ct = 0; ct < 4; ++ct)
          b8[ct] = *reinterpret_cast<const u32x4*>(bia + (((int64_t)wt * kWaveCols + 16 * ct + c16) * Gp + gg0) * 2);
        for (int o = 0; o < 8; ++o)
          s8[o] = gg0 + o < G ? *reinterpret_cast<const u32x2*>(scl + ((int64_t)(gg0 + o) * 16 + c16) * 8)
                              : u32x2{0u, 0u};
        u32x4 hi[4], lo[4];
        bias_operands(b8, s8, hi, lo);
        for (int ct = 0; ct < 4; ++ct) be[ct] = seg == 1 ? lo[ct] : hi[ct];
      }
#pragma unroll
      for (int ms = 0; ms < kSub; ++ms) {
        if (ms < nsub) {
          const int m = ms * 16 + c16;
          u32x4 ax = u32x4{0u, 0u, 0u, 0u};
          if (m < rows)
            ax = *reinterpret_cast<const u32x4*>(a.act3 + (int64_t)L.rowidx[m] * a.Kx + k0);
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) acc[ms][ct] = mfma16(ax, be[ct], acc[ms][ct]);
        }
      }
    }
  }

  if (MODE == kGateUp) {
    const int I = a.N;
    float hs[kSub][4];
#pragma unroll
    for (int ms = 0; ms < kSub; ++ms) {
      for (int i = 0; i < 4; ++i) hs[ms][i] = 0.f;
      if (ms < nsub) {
        for (int ct = 0; ct < 2; ++ct) {
          const int hc = 32 * wt + 16 * ct + c16;
          for (int i = 0; i < 4; ++i) {
            const int r = ms * 16 + 4 * kb + i;
            const uint16_t hb = f2bf(silu(acc[ms][ct][i]) * acc[ms][ct + 2][i]);
            if (r < rows) {
              a.h_out[(int64_t)(row0 + r) * I + hc] = hb;
              hs[ms][i] += bf16f(hb);
            }
          }
        }
      }
      for (int i = 0; i < 4; ++i) {
        float v = hs[ms][i];
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        v += __shfl_xor(v, 4);
        v += __shfl_xor(v, 8);
        if (c16 == 0) L.red[wave][ms * 16 + 4 * kb + i] = v;
      }
    }
    __syncthreads();
    const int Gd = I / kGroup, Gpd = round_up(Gd, 8);
    if (tid < 128) {
      const int w2 = tid >> 6, r = tid & 63;
      if (r < rows) {
        const float v = L.red[2 * w2][r] + L.red[2 * w2 + 1][r];
        const int gh = nt * 2 + w2;
        uint16_t hi, lo;
        split_hi_lo(v, hi, lo);
        uint16_t* o = a.hs3_out + (int64_t)(row0 + r) * a.Kx_down;
        o[gh] = hi;
        o[Gpd + gh] = hi;
        o[2 * Gpd + gh] = lo;
      }
    }
    if (nt == 0) {
      for (int e = tid; e < rows * a.Kx_down; e += 256) {
        const int r = e / a.Kx_down, kk = e % a.Kx_down;
        const int seg = kk / Gpd, g = kk % Gpd;
        if (seg >= 3 || g >= Gd) a.hs3_out[(int64_t)(row0 + r) * a.Kx_down + kk] = 0;
      }
    }
  } else {
    if (tid < kItemRows)
      L.outrow[tid] = expert >= 0 ? perm_p + perm_p / a.k  // row t*(k+1) + j
                                  : (token0 + tid) * (a.k + 1) + a.k;
    __syncthreads();
#pragma unroll
    for (int ms = 0; ms < kSub; ++ms) {
      if (ms < nsub) {
        for (int i = 0; i < 4; ++i) {
          const int r = ms * 16 + 4 * kb + i;
          if (r < rows) {
            float* o = a.partial + (int64_t)L.outrow[r] * a.N + 64 * wt + c16;
            for (int ct = 0; ct < 4; ++ct) o[16 * ct] = acc[ms][ct][i];
          }
        }
      }
    }
  }
}

// y[t][n] = bf16(partial[t][k][n] + sum_{j<k} w[t][j] * partial[t][j][n]):
// slot k holds the shared expert, slots j < k the routed experts; each thread
// owns eight consecutive n of one token and issues all its loads up front.
template <int K>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ partial,
                                                      const float* __restrict__ topk_w,
                                                      uint16_t* __restrict__ y, int T, int N) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int per_row = N / 8;
  if (i >= (int64_t)T * per_row) return;
  const int64_t t = i / per_row;
  const int n = (int)(i % per_row) * 8;
  const float* p = partial + t * (K + 1) * (int64_t)N + n;
  f32x4 v[K + 1][2];
#pragma unroll
  for (int j = 0; j <= K; ++j) {
    v[j][0] = *reinterpret_cast<const f32x4*>(p + (int64_t)j * N);
    v[j][1] = *reinterpret_cast<const f32x4*>(p + (int64_t)j * N + 4);
  }
  float w[K];
#pragma unroll
  for (int j = 0; j < K; ++j) w[j] = topk_w[t * K + j];
  f32x4 s0 = v[K][0], s1 = v[K][1];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    s0 += w[j] * v[j][0];
    s1 += w[j] * v[j][1];
  }
  u32x4 o;
  o.x = f2bf(s0.x) | ((uint32_t)f2bf(s0.y) << 16);
  o.y = f2bf(s0.z) | ((uint32_t)f2bf(s0.w) << 16);
  o.z = f2bf(s1.x) | ((uint32_t)f2bf(s1.y) << 16);
  o.w = f2bf(s1.z) | ((uint32_t)f2bf(s1.w) << 16);
  *reinterpret_cast<u32x4*>(y + t * N + n) = o;
}

// Test hook: expand one expert's packed matrices with the GEMM's own loads and
// code expansion. Grid: (n_wt, G); block: 64 threads (one wave).
__global__ void test_dequant_kernel(const uint8_t* ebase, int N, int K, int paired, float* out) {
  const int lane = threadIdx.x, c16 = lane & 15, kb = lane >> 4;
  const int wt = blockIdx.x, g = blockIdx.y;
  const PackGeom geom = pack_geom(N, K, paired);
  const int G = geom.G;
  const uint8_t* nib = ebase + geom.nib_off + ((int64_t)wt * G + g) * kNibBytes + lane * 16;
  const uint8_t* scl = ebase + geom.scl_off + (((int64_t)wt * G + g) * 16 + c16) * 8;
  const u32x4 w0 = *reinterpret_cast<const u32x4*>(nib);
  const u32x4 w1 = *reinterpret_cast<const u32x4*>(nib + 1024);
  const u32x2 sc = *reinterpret_cast<const u32x2*>(scl);
  const uint32_t words[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  const float s[4] = {bf16lo(sc.x), bf16hi(sc.x), bf16lo(sc.y), bf16hi(sc.y)};
  const uint16_t* bia = reinterpret_cast<const uint16_t*>(ebase + geom.bia_off);
  const ExpandConsts xk = expand_consts();
  for (int ct = 0; ct < 4; ++ct) {
    const int j = 16 * ct + c16;
    const float b = bf16f(bia[((int64_t)wt * kWaveCols + j) * geom.Gp + g]);
    int mat = 0, row = 64 * wt + j;
    if (paired) {
      mat = j >> 5;
      row = 32 * wt + (j & 31);
    }
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4 v = expand_codes(words[2 * ct + ks], xk);
      const uint32_t pairs[4] = {v.x, v.y, v.z, v.w};
      for (int d = 0; d < 4; ++d)
        for (int hlf = 0; hlf < 2; ++hlf) {
          const float e128 = hlf ? bf16hi(pairs[d]) : bf16lo(pairs[d]);
          const int kk = g * kGroup + 32 * ks + 8 * kb + 2 * d + hlf;
          out[((int64_t)mat * N + row) * K + kk] = (e128 - 128.0f) * s[ct] + b;
        }
    }
  }
}

hipError_t launch_gemm(GemmMode mode, const GemmArgs& a, hipStream_t s) {
  const dim3 grid(a.total_slots * a.n_tiles), block(256);
  if (mode == kGateUp)
    hipLaunchKernelGGL(gemm_kernel<kGateUp>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(gemm_kernel<kDown>, grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_combine(const float* partial, const float* topk_w, uint16_t* y, int T, int N,
                          int k, hipStream_t s) {
  if (k != 8) return hipErrorInvalidValue;
  const int64_t threads = (int64_t)T * (N / 8);
  hipLaunchKernelGGL(combine_kernel<8>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                     partial, topk_w, y, T, N);
  return hipGetLastError();
}

hipError_t launch_test_dequant(const uint8_t* expert_base, int N, int K, int paired, float* out,
                               hipStream_t s) {
  const PackGeom g = pack_geom(N, K, paired);
  hipLaunchKernelGGL(test_dequant_kernel, dim3(g.n_wt, g.G), dim3(64), 0, s, expert_base, N, K,
                     paired, out);
  return hipGetLastError();
}

}  // namespace moe
