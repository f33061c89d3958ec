// Grouped expert GEMMs with fused int4 expansion (gfx950, bf16 matrix cores).
//
// diariobitcoin.com, "Perplexity libera Lily, un motor de IA que supera a
// MLX-LM en Apple Silicon", section "Las optimizaciones en el prefill": the
// grouped expert GEMM reconstructs the 4-bit weights block by block in on-chip
// memory with fp32 accumulation and never writes expanded weights back; the
// expert GEMMs are about 90% of prefill time.
//
// A unit of work is one work item (up to 32 rows of one expert: (token, slot)
// pairs in expert-sorted order, or 32 tokens of the shared expert) times one
// column tile of the output; each wave owns 64 columns. The grid is
// persistent: every block streams its units back to back and starts loading
// the next unit while the current one finishes, so the memory pipeline does
// not drain between units (gemm_ring_kernel: a register ring of plain loads,
// one group ahead, see below; K a multiple of 128).
//
// Per group and 16x16 output tile, with the codes expanded to the exact bf16
// values 128 + q by two bit operations:
//   P    = x . (128 + q)                      (matrix cores, fp32)
//   xsum = x . 1                               (matrix cores: the rows' sums)
//   acc += s * P + (b - 128 s) * xsum          (fp32 VALU)
// Algebraically this is x . (q s + b) with the weights used exactly.
//
// Epilogues: gate/up -> h = silu(gate) * up rounded to bf16; down -> a routed
// row rounded to bf16 at its (token, slot) pair index, a shared-expert row in
// fp32 at its token; the combine kernel then forms
// y = bf16(shared + sum over the k slots of weight * output) in a fixed order,
// so the result is deterministic.
#include <atomic>

#include "kernels.h"

namespace moe {

constexpr int kBatch = 16;                       // units whose row tables a block stages at once
constexpr int kXBytes = kItemRows * kGroup * 2;  // gathered activations per group: 4 KB
// Keeps the compiler from moving LDS accesses across this point (the
// epilogue transposes through LDS with differently typed accesses).
__device__ inline void compiler_fence() { asm volatile("" ::: "memory"); }

struct UnitInfo {
  int expert;  // -1: shared expert
  int row0;    // first row (sorted pair position, or k*T + first token for the shared expert)
  int rows;    // 1..item_rows
  int nt;      // column tile
};

// Down output of one row and four consecutive columns: a routed row (pair p)
// rounded to bf16 at [p][N] (it enters the combine with a routing weight of
// about 1/k), a shared-expert row (token t) kept in fp32 at [t][N].
__device__ inline void store_down(const GemmArgs& a, bool routed, int orow, int col, f32x4 v) {
  if (routed) {
    u32x2 o;
    o.x = pack_bf16x2(v.x, v.y);
    o.y = pack_bf16x2(v.z, v.w);
    *reinterpret_cast<u32x2*>(a.partial_r + (int64_t)orow * a.N + col) = o;
  } else {
    *reinterpret_cast<f32x4*>(a.partial_s + (int64_t)orow * a.N + col) = v;
  }
}

// bf16 pairs (1.0, 1.0): the B operand that turns an MFMA into row sums.
constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;

// One 64-input group for NS 16-row subtiles: the rows' group sums come from
// the matrix cores (x . 1), then acc += s * P + (b - 128 s) * xsum.
template <int NS>
__device__ __forceinline__ void ring_step(const u32x4 w0, const u32x4 w1, const u32x4 sbv,
                                          const u32x4* xst, int kb, int c16,
                                          const ExpandConsts xk, f32x4 (&acc)[2][4]) {
  const uint32_t words[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  const float sc[4] = {bf16lo(sbv.x), bf16hi(sbv.x), bf16lo(sbv.y), bf16hi(sbv.y)};
  const float bi[4] = {bf16lo(sbv.z), bf16hi(sbv.z), bf16lo(sbv.w), bf16hi(sbv.w)};
  const u32x4 ones = {kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2};
  u32x4 ax[NS][2];
  f32x4 xsv[NS];
#pragma unroll
  for (int ms = 0; ms < NS; ++ms) {
    ax[ms][0] = xst[(ms * 8 + kb) * 16 + c16];
    ax[ms][1] = xst[(ms * 8 + 4 + kb) * 16 + c16];
    xsv[ms] = mfma16(ax[ms][0], ones, f32x4{0.f, 0.f, 0.f, 0.f});
    xsv[ms] = mfma16(ax[ms][1], ones, xsv[ms]);
  }
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const u32x4 b0 = expand_codes(words[2 * ct], xk);
    const u32x4 b1 = expand_codes(words[2 * ct + 1], xk);
    const float bp = bi[ct] - 128.0f * sc[ct];
#pragma unroll
    for (int ms = 0; ms < NS; ++ms) {
      f32x4 p = mfma16(ax[ms][0], b0, f32x4{0.f, 0.f, 0.f, 0.f});
      p = mfma16(ax[ms][1], b1, p);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[ms][ct][i] = __builtin_fmaf(bp, xsv[ms][i], __builtin_fmaf(sc[ct], p[i], acc[ms][ct][i]));
    }
  }
}

// One group with bf16 weights already expanded in memory: w[2 ct + ks] is the
// B operand of column tile ct and k half ks; plain MFMA accumulation.
template <int NS>
__device__ __forceinline__ void ring_step_bf16(const u32x4 (&w)[8], const u32x4* xst, int kb, int c16,
                                               f32x4 (&acc)[2][4]) {
#pragma unroll
  for (int ms = 0; ms < NS; ++ms) {
    const u32x4 a0 = xst[(ms * 8 + kb) * 16 + c16];
    const u32x4 a1 = xst[(ms * 8 + 4 + kb) * 16 + c16];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      acc[ms][ct] = mfma16(a0, w[2 * ct], acc[ms][ct]);
      acc[ms][ct] = mfma16(a1, w[2 * ct + 1], acc[ms][ct]);
    }
  }
}

// ------------------------------------------------------------------ register-ring kernel
//
// The main path for K a multiple of 128 (G % 2 == 0). Three blocks of four
// waves per compute unit (three waves per SIMD, so one wave's waits are
// covered by the others); each wave owns 64 columns. Every load of the loop
// is a plain register load: per wave and group the packed codes (2 KB), a
// 1 KB share of the gathered activation rows and a 256-byte share of the
// scale/bias words are loaded into a two-deep register ring one group ahead
// (about 40 KB per compute unit in flight, some 10 MB on the chip: what HBM
// needs at its loaded latency; three groups ahead, 30 MB in flight, made the
// 512-token gate/up 5% and down 3% slower). At its turn a group's activation
// and scale/bias shares are written to a two-stage LDS buffer, one barrier,
// and all four waves read them. Unit boundaries fall on multiples of two
// groups, so every ring slot index is static and the loads for the next
// unit start while the current one finishes. Loads of one kind complete in
// order, so the compiler's own wait counts keep a group in flight (no
// asynchronous LDS copies are mixed in, which would force full drains).

constexpr int kRWaves = 4;
constexpr int kRThreads = kRWaves * 64;
constexpr int kRS = 2;         // ring depth in groups (K / 64 must be a multiple)
constexpr int kRBlocksPerCU = 3;

struct RingLds {
  u32x4 x[2][kXBytes / 16];      // [stage][ms 2][c 8][row 16]
  u32x4 sb[2][kRWaves][16];      // [stage][wave][c16]: 4 scales, 4 biases
  UnitInfo unit[kBatch];
  int rowidx[kBatch][kItemRows];
  int outrow[kBatch][kItemRows];
  u32x4 tr[kRWaves][64];
};

// BF16W: the weights come as bf16 values already expanded in memory (the
// unfused comparison path, see bf16 expansion below) instead of int4 codes:
// per wave and group 8 x 16 bytes per lane, a two-deep ring, no scale, bias
// or row sums.
template <int MODE, bool BF16W>
__global__ __launch_bounds__(kRThreads, kRBlocksPerCU) void gemm_ring_kernel(GemmArgs a) {
  constexpr int RS = BF16W ? 2 : kRS;  // ring depth in groups
  constexpr int NW = BF16W ? 8 : 2;    // weight vectors per lane and group
  __shared__ RingLds L;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, kb = lane >> 4;
  const int K = a.K, G = K / kGroup;
  const PackGeom geom = pack_geom(a.N, K, a.paired);
  const int n_wt = geom.n_wt;
  const int n_tiles = (n_wt + kRWaves - 1) / kRWaves;

  const int xcd = blockIdx.x & 7, lb = blockIdx.x >> 3, nbx = gridDim.x >> 3;
  const int ni = *a.num_items;
  const int n_slots = ni + a.shared_slots;
  // XCD x owns the contiguous unit range [u0, u1) (units are slot-major), so
  // the column tiles of one item, and the items of one expert, share an L2
  const int n_units = n_slots * n_tiles;
  const int u0 = (int)((int64_t)n_units * xcd / 8), u1 = (int)((int64_t)n_units * (xcd + 1) / 8);
  const int my_units = u1 - u0 > lb ? (u1 - u0 - lb + nbx - 1) / nbx : 0;
  const ExpandConsts xk = expand_consts();

  const int xu = 64 * wave + lane;                                 // 16-byte unit of the x stage
  const int xm = (xu >> 7) * 16 + (xu & 15), xc = (xu >> 4) & 7;

  for (int base = 0; base < my_units; base += kBatch) {
    const int nb = min(kBatch, my_units - base);
    lds_barrier();
    if (tid < nb) {
      const int v = u0 + lb + (base + tid) * nbx;
      const int slot = v / n_tiles;
      UnitInfo u;
      u.nt = v % n_tiles;
      if (slot < ni) {
        u.expert = a.items[3 * slot];
        u.row0 = a.items[3 * slot + 1];
        u.rows = a.items[3 * slot + 2];
      } else {
        const int t0 = (slot - ni) * a.item_rows;
        u.expert = -1;
        u.row0 = a.k * a.T + t0;
        u.rows = min(a.item_rows, a.T - t0);
      }
      L.unit[tid] = u;
    }
    lds_barrier();
    for (int e = tid; e < nb * kItemRows; e += kRThreads) {
      const int j = e / kItemRows, m = e % kItemRows;
      const UnitInfo u = L.unit[j];
      const int mm = m < u.rows ? m : 0;
      if (MODE == kGateUp) {
        L.rowidx[j][m] = u.expert >= 0 ? a.perm[u.row0 + mm] / a.k : u.row0 - a.k * a.T + mm;
      } else {
        L.rowidx[j][m] = u.row0 + mm;
        int orow;
        if (u.expert >= 0) {
          const int p = a.perm[u.row0 + mm];
          orow = p;
        } else {
          orow = u.row0 - a.k * a.T + mm;  // shared output row: the token
        }
        L.outrow[j][m] = orow;
      }
    }
    lds_barrier();

    // ---- load side: unit iu, group ig (stays on the last group once every
    // group is issued, so each step issues the same four loads)
    const int total = nb * G;  // a multiple of RS
    int iu = 0, ig = 0, issued = 0;
    const uint16_t* xsrc = nullptr;
    const uint8_t* nsrc = nullptr;
    const uint8_t* bsrc = nullptr;
    auto set_load_unit = [&](int j) {
      const int expert = __builtin_amdgcn_readfirstlane(L.unit[j].expert);
      const int nt = __builtin_amdgcn_readfirstlane(L.unit[j].nt);
      const int wt = min(nt * kRWaves + wave, n_wt - 1);
      const uint8_t* eb = expert >= 0 ? a.blob + (int64_t)expert * a.expert_bytes : a.shared_blob;
      nsrc = BF16W ? eb + (int64_t)wt * G * kBf16GroupBytes + lane * 16
                   : eb + geom.nib_off + (int64_t)wt * G * kNibBytes + lane * 16;
      bsrc = eb + geom.sb_off + (int64_t)wt * G * kSbBytes + lane * 4;
      xsrc = a.act + (int64_t)L.rowidx[j][xm] * K + 8 * xc;
    };
    u32x4 rc[RS][NW], rx[RS];
    uint32_t rb[RS];
    auto load = [&](u32x4 (&cw)[NW], u32x4& xv, uint32_t& bv) {
      if constexpr (BF16W) {
#pragma unroll
        for (int h = 0; h < NW; ++h)
          cw[h] = *reinterpret_cast<const u32x4*>(nsrc + (int64_t)ig * kBf16GroupBytes + 1024 * h);
        bv = 0;
      } else {
        cw[0] = *reinterpret_cast<const u32x4*>(nsrc + (int64_t)ig * kNibBytes);
        cw[1] = *reinterpret_cast<const u32x4*>(nsrc + (int64_t)ig * kNibBytes + 1024);
        bv = *reinterpret_cast<const uint32_t*>(bsrc + (int64_t)ig * kSbBytes);
      }
      xv = *reinterpret_cast<const u32x4*>(xsrc + ig * kGroup);
      if (++issued < total) {
        if (++ig == G) {
          ig = 0;
          set_load_unit(++iu);
        }
      }
    };
    set_load_unit(0);
#pragma unroll
    for (int d = 0; d < RS - 1; ++d) load(rc[d], rx[d], rb[d]);

    f32x4 acc[2][4];
    int rows = 0, nsub = 0, nt = 0, row0 = 0;
    bool routed = true;
    bool active = false;
    for (int s0 = 0; s0 < total; s0 += RS) {
      const int cu = s0 / G, cg0 = s0 % G;
      if (cg0 == 0) {
        rows = __builtin_amdgcn_readfirstlane(L.unit[cu].rows);
        routed = __builtin_amdgcn_readfirstlane(L.unit[cu].expert) >= 0;
        row0 = __builtin_amdgcn_readfirstlane(L.unit[cu].row0);
        nt = __builtin_amdgcn_readfirstlane(L.unit[cu].nt);
        nsub = (rows + 15) >> 4;
        active = nt * kRWaves + wave < n_wt;
#pragma unroll
        for (int ms = 0; ms < 2; ++ms)
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) acc[ms][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int d = 0; d < RS; ++d) {
        const int nx = (d + RS - 1) % RS;
        load(rc[nx], rx[nx], rb[nx]);  // group s0 + d + RS - 1 (or a repeat of the last)
        L.x[d & 1][xu] = rx[d];
        if constexpr (!BF16W) reinterpret_cast<uint32_t*>(&L.sb[d & 1][wave][0])[lane] = rb[d];
        // this group's shares are in LDS, and every wave is done with the
        // stage these writes replaced (read two groups ago)
        lds_barrier();
        if (active) {
          if constexpr (BF16W) {
            if (nsub == 2)
              ring_step_bf16<2>(rc[d], &L.x[d & 1][0], kb, c16, acc);
            else
              ring_step_bf16<1>(rc[d], &L.x[d & 1][0], kb, c16, acc);
          } else {
            const u32x4 sbv = L.sb[d & 1][wave][c16];
            if (nsub == 2)
              ring_step<2>(rc[d][0], rc[d][1], sbv, &L.x[d & 1][0], kb, c16, xk, acc);
            else
              ring_step<1>(rc[d][0], rc[d][1], sbv, &L.x[d & 1][0], kb, c16, xk, acc);
          }
        }
      }
      if (cg0 + RS < G) continue;

      // ---- epilogue of unit cu
      const int wt = nt * kRWaves + wave;
      if (!active) continue;
      if (MODE == kGateUp) {
        const int I = a.N;
        uint16_t* trb = reinterpret_cast<uint16_t*>(&L.tr[wave][0]);
        const int rr = lane >> 2, ch = lane & 3;
#pragma unroll
        for (int ms = 0; ms < 2; ++ms) {
          if (ms < nsub) {
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                trb[(4 * kb + i) * 32 + 16 * ct + c16] =
                    f2bf(silu(acc[ms][2 * ct][i]) * acc[ms][2 * ct + 1][i]);
            compiler_fence();
            const u32x4 v = L.tr[wave][rr * 4 + ch];
            compiler_fence();
            if (16 * ms + rr < rows)
              *reinterpret_cast<u32x4*>(a.h_out + (int64_t)(row0 + 16 * ms + rr) * I + 32 * wt + 8 * ch) = v;
          }
        }
      } else {
        float* trf = reinterpret_cast<float*>(&L.tr[wave][0]);
        const int rr = lane >> 2, c4 = lane & 3;
#pragma unroll
        for (int ms = 0; ms < 2; ++ms) {
          if (ms < nsub) {
            const int r = 16 * ms + rr;
            const int orow = L.outrow[cu][r < rows ? r : 0];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
              for (int i = 0; i < 4; ++i) trf[(4 * kb + i) * 16 + c16] = acc[ms][ct][i];
              compiler_fence();
              const f32x4 v = *reinterpret_cast<const f32x4*>(&trf[rr * 16 + 4 * c4]);
              compiler_fence();
              if (r < rows) store_down(a, routed, orow, 64 * wt + 16 * ct + 4 * c4, v);
            }
          }
        }
      }
    }
  }
}

// y[t][n] = bf16(shared[t][n] + sum_{j<k} w[t][j] * routed[t k + j][n]), j
// ascending: the shared expert's fp32 row plus the k routed bf16 rows; each
// thread owns eight consecutive n of one token and issues all its loads up
// front.
template <int K>
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ routed,
                                                      const float* __restrict__ shared,
                                                      const float* __restrict__ topk_w,
                                                      uint16_t* __restrict__ y, int T, int N) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int per_row = N / 8;
  if (i >= (int64_t)T * per_row) return;
  const int64_t t = i / per_row;
  const int n = (int)(i % per_row) * 8;
  const uint16_t* pr = routed + t * K * (int64_t)N + n;
  u32x4 v[K];
#pragma unroll
  for (int j = 0; j < K; ++j) v[j] = *reinterpret_cast<const u32x4*>(pr + (int64_t)j * N);
  f32x4 s0 = *reinterpret_cast<const f32x4*>(shared + t * N + n);
  f32x4 s1 = *reinterpret_cast<const f32x4*>(shared + t * N + n + 4);
  float w[K];
#pragma unroll
  for (int j = 0; j < K; ++j) w[j] = topk_w[t * K + j];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const f32x4 d0 = {bf16lo(v[j].x), bf16hi(v[j].x), bf16lo(v[j].y), bf16hi(v[j].y)};
    const f32x4 d1 = {bf16lo(v[j].z), bf16hi(v[j].z), bf16lo(v[j].w), bf16hi(v[j].w)};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      s0[q] = __builtin_fmaf(w[j], d0[q], s0[q]);
      s1[q] = __builtin_fmaf(w[j], d1[q], s1[q]);
    }
  }
  u32x4 o;
  o.x = pack_bf16x2(s0.x, s0.y);
  o.y = pack_bf16x2(s0.z, s0.w);
  o.z = pack_bf16x2(s1.x, s1.y);
  o.w = pack_bf16x2(s1.z, s1.w);
  *reinterpret_cast<u32x4*>(y + t * N + n) = o;
}

// Unfused comparison path: expand packed experts to bf16 in memory. Grid:
// (count + 1 experts, n_wt * G / 4); block: 4 waves, one (wave tile, group)
// each; the last expert index is the shared expert.
__global__ __launch_bounds__(256) void expand_bf16_kernel(const uint8_t* blob, int64_t expert_bytes,
                                                          const uint8_t* shared_blob, int count,
                                                          const int32_t* hist, int N, int K,
                                                          int paired, uint8_t* out,
                                                          uint8_t* out_shared) {
  const int e = blockIdx.x;
  if (e < count && hist && hist[e] == 0) return;  // expert without rows
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, c16 = lane & 15;
  const PackGeom geom = pack_geom(N, K, paired);
  const int G = geom.G, q = blockIdx.y * 4 + wave;
  if (q >= geom.n_wt * G) return;
  const uint8_t* eb = e < count ? blob + (int64_t)e * expert_bytes : shared_blob;
  uint8_t* ob = e < count ? out + (int64_t)e * geom.n_wt * G * kBf16GroupBytes : out_shared;
  const uint8_t* nib = eb + geom.nib_off + ((int64_t)q * 128 + lane) * 16;
  const u32x4 w0 = *reinterpret_cast<const u32x4*>(nib);
  const u32x4 w1 = *reinterpret_cast<const u32x4*>(nib + 1024);
  const u32x4 sbv = *reinterpret_cast<const u32x4*>(eb + geom.sb_off + ((int64_t)q * 16 + c16) * 16);
  const uint32_t words[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  const float sc[4] = {bf16lo(sbv.x), bf16hi(sbv.x), bf16lo(sbv.y), bf16hi(sbv.y)};
  const float bi[4] = {bf16lo(sbv.z), bf16hi(sbv.z), bf16lo(sbv.w), bf16hi(sbv.w)};
  const ExpandConsts xk = expand_consts();
#pragma unroll
  for (int wd = 0; wd < 8; ++wd) {
    const int ct = wd >> 1;
    const u32x4 v = expand_codes(words[wd], xk);
    const uint32_t pr[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const float lo = __builtin_fmaf(bf16lo(pr[d]) - 128.0f, sc[ct], bi[ct]);
      const float hi = __builtin_fmaf(bf16hi(pr[d]) - 128.0f, sc[ct], bi[ct]);
      o[d] = pack_bf16x2(lo, hi);
    }
    *reinterpret_cast<u32x4*>(ob + ((int64_t)q * 8 + wd) * 1024 + lane * 16) = u32x4{o[0], o[1], o[2], o[3]};
  }
}

// Test hook: expand one expert's packed matrices with the GEMM's own loads and
// code expansion. Grid: (n_wt, G); block: 64 threads (one wave).
__global__ void test_dequant_kernel(const uint8_t* ebase, int N, int K, int paired, float* out) {
  const int lane = threadIdx.x, c16 = lane & 15, kb = lane >> 4;
  const int wt = blockIdx.x, g = blockIdx.y;
  const PackGeom geom = pack_geom(N, K, paired);
  const int G = geom.G;
  const uint8_t* nib = ebase + geom.nib_off + ((int64_t)wt * G + g) * kNibBytes + lane * 16;
  const u32x4 w0 = *reinterpret_cast<const u32x4*>(nib);
  const u32x4 w1 = *reinterpret_cast<const u32x4*>(nib + 1024);
  const u32x4 sbv =
      *reinterpret_cast<const u32x4*>(ebase + geom.sb_off + ((int64_t)wt * G + g) * kSbBytes + c16 * 16);
  const uint32_t words[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  const float s[4] = {bf16lo(sbv.x), bf16hi(sbv.x), bf16lo(sbv.y), bf16hi(sbv.y)};
  const float bi[4] = {bf16lo(sbv.z), bf16hi(sbv.z), bf16lo(sbv.w), bf16hi(sbv.w)};
  const ExpandConsts xk = expand_consts();
  for (int ct = 0; ct < 4; ++ct) {
    const int j = 16 * ct + c16;
    int mat = 0, row = 64 * wt + j;
    if (paired) {
      mat = (j >> 4) & 1;
      row = 32 * wt + 16 * (j >> 5) + (j & 15);
    }
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4 v = expand_codes(words[2 * ct + ks], xk);
      const uint32_t pairs[4] = {v.x, v.y, v.z, v.w};
      for (int d = 0; d < 4; ++d)
        for (int hlf = 0; hlf < 2; ++hlf) {
          const float e128 = hlf ? bf16hi(pairs[d]) : bf16lo(pairs[d]);
          const int kk = g * kGroup + 32 * ks + 8 * kb + 2 * d + hlf;
          out[((int64_t)mat * N + row) * K + kk] = (e128 - 128.0f) * s[ct] + bi[ct];
        }
    }
  }
}

// Persistent grids: one block per compute unit (a multiple of 8 for the XCD
// mapping). The per-device count is cached; concurrent first calls may both
// query it and store the same value (relaxed atomics, no lock needed).
int compute_units() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (!v) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 8)
      cus = 256;
    v = cus / 8 * 8;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

namespace {

template <int MODE>
hipError_t launch_mode(const GemmArgs& a, hipStream_t s, int grid_blocks) {
  if (a.bf16_weights) {
    const int G = a.K / kGroup;
    if (G % 2) return hipErrorInvalidValue;
    const int exact = (grid_blocks + 7) / 8 * 8;
    hipLaunchKernelGGL((gemm_ring_kernel<MODE, true>),
                       dim3(grid_blocks > 0 ? exact : kRBlocksPerCU * compute_units()),
                       dim3(kRThreads), 0, s, a);
    return hipGetLastError();
  }
  const int G = a.K / kGroup;
  if (G < 2 || G > kMaxGroups) return hipErrorInvalidValue;
  // every supported shape has an even group count (H % 256 == 0, I % 128 == 0)
  if (G % kRS) return hipErrorInvalidValue;
  const int exact = (grid_blocks + 7) / 8 * 8;
  const dim3 grid(grid_blocks > 0 ? exact : kRBlocksPerCU * compute_units()), block(kRThreads);
  hipLaunchKernelGGL((gemm_ring_kernel<MODE, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(GemmMode mode, const GemmArgs& a, hipStream_t s, int grid_blocks) {
  return mode == kGateUp ? launch_mode<kGateUp>(a, s, grid_blocks) : launch_mode<kDown>(a, s, grid_blocks);
}

hipError_t launch_combine(const uint16_t* routed, const float* shared, const float* topk_w, uint16_t* y,
                          int T, int N, int k, hipStream_t s) {
  if (k != 8) return hipErrorInvalidValue;
  const int64_t threads = (int64_t)T * (N / 8);
  hipLaunchKernelGGL(combine_kernel<8>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                     routed, shared, topk_w, y, T, N);
  return hipGetLastError();
}

hipError_t launch_expand_bf16(const uint8_t* blob, int64_t expert_bytes, const uint8_t* shared_blob,
                              int count, const int32_t* hist, int N, int K, int paired, uint8_t* out,
                              uint8_t* out_shared, hipStream_t s) {
  const PackGeom g = pack_geom(N, K, paired);
  const dim3 grid(count + 1, (g.n_wt * g.G + 3) / 4);
  hipLaunchKernelGGL(expand_bf16_kernel, grid, dim3(256), 0, s, blob, expert_bytes, shared_blob, count,
                     hist, N, K, paired, out, out_shared);
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
