// Grouped expert GEMMs for long chunks: int4 weights expanded once to bf16
// per (expert, 512-column tile, 64-input group) and shared by up to 144 rows
// of that expert (gfx950, bf16 matrix cores, fp32 accumulation).
//
// diariobitcoin.com, "Perplexity libera Lily, un motor de IA que supera a
// MLX-LM en Apple Silicon", section "Las optimizaciones en el prefill": the
// grouped expert GEMM reconstructs the 4-bit weights block by block on chip
// with fp32 accumulation and never writes expanded weights back to memory;
// section "Qwen3.6 combina tres cargas de trabajo": weights are affine 4-bit
// in groups of 64 with a bf16 scale and bias, w = q * scale + bias.
//
// A work unit is one work item (up to 144 rows of one expert in
// expert-sorted order, or 144 tokens of the shared expert) times a 512-column
// tile of the output. A block of eight waves takes one unit; wave w owns the
// 64 columns of packed wave tile 8 nt + w for all of the item's rows (up to
// nine 16-row subtiles, 144 fp32 accumulators per lane: 144 rows rather than
// 128 so that an expert a little above 128 rows in a chunk, common when the
// chunk averages 128 rows per expert, does not pay a second expansion of its
// weights for a few rows). Per 64-input group:
//   * the gathered activation rows (144 x 64 bf16 = 18 KB) are loaded by all
//     512 threads into registers during the previous group's step, then
//     written to a two-stage LDS buffer in the matrix-core A-operand order,
//     and all eight waves read them;
//   * each lane loads the packed codes of its own B-operand positions (the
//     packed layout puts them there) and their scale/bias record about one
//     and a half groups ahead, and expands them to bf16 w = q s + b in
//     registers: each pair of codes becomes the exact fp16 pair
//     (1024 + q, 1024 + q') by a shift and one AND-OR (no shift for the
//     lowest pair), one mixed-precision FMA per weight forms fp32 q s + b
//     with a single
//     rounding ((1024 + q) s + (b - 1024 s), the product exact), and one
//     conversion rounds two weights to bf16 (nearest even);
//   * the matrix cores accumulate x . w directly (v_mfma_f32_16x16x32_bf16).
// The expansion costs about two vector instructions per weight, shared by
// the item's rows; there is no per-output scale step.
//
// Epilogues as in the 32-row GEMMs: gate/up writes h = bf16(silu(gate) * up)
// at the row's sorted position; down writes a routed row rounded to bf16 at
// its (token, slot) pair index and a shared-expert row in fp32 at its token,
// for the deterministic combine kernel.
#include <type_traits>

#include "kernels.h"

namespace moe {

namespace {

constexpr int kWRows = kWideRows;       // rows per work item
constexpr int kWSub = kWRows / 16;      // 16-row subtiles
constexpr int kWWaves = 8;
constexpr int kWThreads = kWWaves * 64;
constexpr int kWSubPerChunk = kWThreads / 128;                   // subtiles one chunk index covers
constexpr int kWChunks = (kWSub + kWSubPerChunk - 1) / kWSubPerChunk;  // 16-byte activation chunks per thread and group
constexpr int kWStaged = kWChunks * kWSubPerChunk;                // subtiles the staging covers (>= kWSub)
constexpr int kWTabRows = 16 * kWStaged;                          // rows of the row tables

struct WideLds {
  union {
    // [stage][subtile][k half][lane]: the A fragments of one group
    u32x4 a[2][kWStaged][2][64];
    // epilogue: one 8 KB transpose buffer per wave
    uint8_t tr[kWWaves][kWRows * 64];
  };
  uint32_t rowoff[kWTabRows];  // byte offset of each row's activations from the unit's base
  int outrow[kWTabRows];   // down: output row (pair index, or token of a shared row)
};

struct WideExpand {
  uint32_t mask_lo, magic;  // 0x000F000F, fp16 1024 | 1024
};

// Hidden from the optimiser so that (w & mask) | magic is selected as one
// bitwise three-input op with register operands.
__device__ inline WideExpand wide_expand_consts() {
  WideExpand k;
  asm volatile("v_mov_b32 %0, 0x000F000F" : "=v"(k.mask_lo));
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(k.magic));
  return k;
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Keeps the compiler from moving LDS accesses across this point (the
// epilogue transposes through LDS with differently typed accesses).
__device__ inline void wide_fence() { asm volatile("" ::: "memory"); }

// Per column and group: the scale s and the offset b - 1024 s (exact in fp32
// for the bf16 inputs' exponent spans).
struct ColAffine {
  float s, c;
};

__device__ inline ColAffine col_affine(float s, float b) {
  return ColAffine{s, __builtin_fmaf(-1024.0f, s, b)};
}

// One packed word (eight codes of one column, k = 8 consecutive inputs, code
// o at nibble (o & 1) * 4 + (o >> 1)) -> the eight bf16 weights in k order:
// ((w >> 4d) & 0x000F000F) | 0x64006400 is the fp16 pair (1024 + q_2d,
// 1024 + q_2d+1), and (1024 + q) s + (b - 1024 s) = q s + b with one rounding.
__device__ inline u32x4 expand_bf16(uint32_t w, const ColAffine& c, const WideExpand& k) {
  u32x4 r;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const f16x2 h = __builtin_bit_cast(f16x2, ((w >> (4 * d)) & k.mask_lo) | k.magic);
    r[d] = pack_bf16x2(__builtin_fmaf((float)h.x, c.s, c.c), __builtin_fmaf((float)h.y, c.s, c.c));
  }
  return r;
}

// Buffer resources: 32-bit offsets from a uniform base, and reads past
// `bytes` return zero instead of touching memory.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ inline u32x4 bload(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

}  // namespace

// Grid: 8 * n_tiles * ceil(max_slots / 8) blocks of 512 threads. Block b
// runs on XCD b & 7; with l = b >> 3, it takes slot 8 (l / n_tiles) + (b & 7)
// and column tile l % n_tiles, so the column tiles of one item run on one XCD
// (their activation rows shared in its L2). Blocks are handed out in index
// order, so the work list's longest-first order makes the launch a greedy
// longest-first schedule per XCD. Slots past the work list exit at once.
//
// Column halves (gate/up): one block per compute unit runs at a time, so V
// units take about V / cus rounds, and a last round of rem = V mod cus units
// leaves the other compute units idle for a whole unit time. When
// rem <= cus / 2, the last rem units in dispatch order run as two
// 256-column halves instead (half 0 in the unit's own block, half 1 in one
// of the blocks past the work list): the last round then takes about half a
// unit time. A half computes each of its outputs by the same operations in
// the same order as the whole unit, so results do not depend on the split.
template <int MODE>
__global__ __launch_bounds__(kWThreads, 1) void gemm_wide_kernel(GemmArgs a) {
  __shared__ WideLds L;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, kb = lane >> 4;
  const int K = a.K, G = K / kGroup;
  const PackGeom geom = pack_geom(a.N, K, a.paired);
  const int n_tiles = (geom.n_wt + kWWaves - 1) / kWWaves;
  const int ni = *a.num_items;
  const int n_slots = ni + a.shared_slots;
  const int n_units = n_slots * n_tiles;
  // dispatch rank of unit block (slot 8 r + x, tile t): rows of 8 slots,
  // tile-major within a row; the last row holds n_slots & 7 slots
  const int full_rows = n_slots >> 3, last_row = n_slots & 7;
  const int full_units = 8 * n_tiles * full_rows;
  // blocks from first_free on have no unit (the grid is sized for the most
  // work items); the first of them take the second column halves
  const int first_free = 8 * n_tiles * (full_rows + (last_row > 0 ? 1 : 0));
  const int rem = n_units % a.cus;
  int split = MODE == kGateUp && rem <= a.cus / 2 ? rem : 0;  // units run as column halves
  split = min(split, max(0, (int)gridDim.x - first_free));
  int slot, nt, hsel = -1;  // hsel: -1 the whole unit, 0 / 1 its column half
  if ((int)blockIdx.x < first_free) {
    const int x = blockIdx.x & 7, l = blockIdx.x >> 3;
    const int r = l / n_tiles, t = l % n_tiles;
    slot = 8 * r + x;
    nt = t;
    if (slot >= n_slots) return;
    const int rank = r < full_rows ? 8 * n_tiles * r + 8 * t + x : full_units + last_row * t + x;
    if (rank >= n_units - split) hsel = 0;
  } else {
    const int i = (int)blockIdx.x - first_free;
    if (i >= split) return;
    const int v = n_units - split + i;  // rank of the unit whose half 1 this is
    if (v < full_units) {
      const int r = v / (8 * n_tiles), q = v % (8 * n_tiles);
      nt = q >> 3;
      slot = 8 * r + (q & 7);
    } else {
      const int q = v - full_units;  // last_row > 0 here
      nt = q / last_row;
      slot = 8 * full_rows + q % last_row;
    }
    hsel = 1;
  }

  // slots: the shared expert's items (full ones first), then the work list
  // (full items, then partial ones, larger first)
  int expert, row0, rows;
  if (slot >= a.shared_slots) {
    const int it = slot - a.shared_slots;
    expert = a.items[3 * it];
    row0 = a.items[3 * it + 1];
    rows = a.items[3 * it + 2];
  } else {
    const int t0 = slot * kWRows;
    expert = -1;
    row0 = a.k * a.T + t0;
    rows = min(kWRows, a.T - t0);
  }
  const bool routed = expert >= 0;
  const int nsub = (rows + 15) >> 4;

  // activation base of the unit: the chunk's x (gate/up: rows gathered by
  // token) or the item's first h row (down: rows contiguous)
  const uint16_t* abase = MODE == kGateUp ? a.act : a.act + (int64_t)row0 * K;
  const uint32_t abytes = MODE == kGateUp ? (uint32_t)((int64_t)a.T * K * 2) : (uint32_t)(rows * K * 2);
  // row tables: byte offset of each row's activations from abase (rows past
  // the item repeat row 0) and, for down, the output row
  if (tid < kWTabRows) {
    const int m = tid < rows ? tid : 0;
    int orow = 0;
    uint32_t aoff;
    if (MODE == kGateUp) {
      const int tok = routed ? a.perm[row0 + m] / a.k : row0 - a.k * a.T + m;
      aoff = (uint32_t)tok * (uint32_t)(2 * K);
    } else {
      aoff = (uint32_t)m * (uint32_t)(2 * K);
      orow = routed ? a.perm[row0 + m] : row0 - a.k * a.T + m;
    }
    L.rowoff[tid] = aoff;
    L.outrow[tid] = orow;
  }
  __syncthreads();

  // activation staging: thread (c16, chunk j of the 128-byte group row, sp)
  // copies rows 16 (kWSubPerChunk i + sp) + c16, i = 0 .. kWChunks - 1
  const int sj = (tid >> 4) & 7, spar = tid >> 7;
  const rsrc_t ares = make_rsrc(abase, abytes);
  uint32_t aoffs[kWChunks];
#pragma unroll
  for (int i = 0; i < kWChunks; ++i) aoffs[i] = L.rowoff[16 * (kWSubPerChunk * i + spar) + c16] + 16 * sj;
  const int sks = sj >> 2, slane = (sj & 3) * 16 + c16;

  // this lane's codes and scale/bias records: a whole unit's wave w takes
  // wave tile 8 nt + w (16-column tiles 0-3); in a column half, wave w takes
  // tiles 2 (w & 1) and 2 (w & 1) + 1 of wave tile 8 nt + 4 hsel + w / 2. The
  // waves past the matrix's last wave tile repeat it and store nothing.
  const int wt_raw = hsel < 0 ? nt * kWWaves + wave : nt * kWWaves + 4 * hsel + (wave >> 1);
  const int ch = hsel < 0 ? 0 : (wave & 1);  // which pair of 16-column tiles (halves)
  const bool wt_active = wt_raw < geom.n_wt;
  const int wt = wt_active ? wt_raw : geom.n_wt - 1;
  const uint8_t* eb = routed ? a.blob + (int64_t)expert * a.expert_bytes : a.shared_blob;
  const rsrc_t wres = make_rsrc(eb, (uint32_t)geom.expert_bytes);
  const uint32_t nbase = (uint32_t)(geom.nib_off + (int64_t)wt * G * kNibBytes);
  const uint32_t sbase = (uint32_t)(geom.sb_off + (int64_t)wt * G * kSbBytes);

  u32x4 ax[kWChunks];      // activation chunks of group g + 1 (to LDS at the end of step g)
  u32x4 cw[2][2], sbv[2];  // codes and scale/bias of groups g and g + 1
  // loads past the last group repeat it (unconditional loads keep the wait
  // counts exact; the repeats hit in cache and are not used); only the chunks
  // of the NS computed subtiles are staged
  auto load_act = [&](int g, u32x4 (&dst)[kWChunks], int ns) {
    g = min(g, G - 1);
#pragma unroll
    for (int i = 0; i < kWChunks; ++i)
      if (kWSubPerChunk * i < ns) dst[i] = bload(ares, aoffs[i], (uint32_t)g * (kGroup * 2));
  };
  // CT 16-column tiles per wave: 4 (whole units: both 16-byte halves of the
  // lane's codes) or 2 (column halves: the half holding tiles 2 ch, 2 ch + 1)
  auto load_w = [&](int g, u32x4 (&c)[2], u32x4& sv, auto CT_) {
    constexpr int CT = decltype(CT_)::value;
    g = min(g, G - 1);
    if constexpr (CT == 4) {
      c[0] = bload(wres, lane * 16, nbase + (uint32_t)g * kNibBytes);
      c[1] = bload(wres, lane * 16, nbase + (uint32_t)g * kNibBytes + 1024);
    } else {
      c[0] = bload(wres, lane * 16, nbase + (uint32_t)g * kNibBytes + 1024 * ch);
    }
    sv = bload(wres, c16 * 16, sbase + (uint32_t)g * kSbBytes);
  };
  auto store_act = [&](int st, const u32x4 (&src)[kWChunks], int ns) {
#pragma unroll
    for (int i = 0; i < kWChunks; ++i)
      if (kWSubPerChunk * i < ns) L.a[st][kWSubPerChunk * i + spar][sks][slane] = src[i];
  };

  f32x4 acc[kWSub][4];
#pragma unroll
  for (int ms = 0; ms < kWSub; ++ms)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[ms][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  const WideExpand xk = wide_expand_consts();

  auto word = [&](const u32x4 (&c)[2], int i) -> uint32_t { return c[i >> 2][i & 3]; };

  // The main loop for NS computed 16-row subtiles (NS * 16 >= rows; the
  // extra rows repeat row 0 and are not stored), straight-line per NS. One
  // step is one group: its 2 NS A fragments f = (k half, subtile) stream from
  // LDS one ahead of the matrix-core ops that use them (scheduling fences
  // keep each read ahead), and each k half's four B operands are expanded
  // just before its 4 NS matrix-core ops. The activations of group g + 1 are
  // loaded at the start of step g and written to LDS at its end; the codes
  // of group g + 2 are loaded once step g has expanded group g's. S = g % 2
  // (register slot, LDS stage) is a compile-time constant so the rings stay
  // in registers.
  auto run = [&](auto NS_, auto CT_) {
    constexpr int NS = decltype(NS_)::value;
    constexpr int CT = decltype(CT_)::value;
    auto frag = [&](int S, int f) -> u32x4 { return L.a[S][f % NS][f / NS][lane]; };
    // prologue: codes of groups 0 and 1 in flight, group 0's activations in LDS
    load_act(0, ax, NS);
    load_w(0, cw[0], sbv[0], CT_);
    load_w(1, cw[1], sbv[1], CT_);
    store_act(0, ax, NS);
    __syncthreads();
    auto step = [&](int g, auto S_) {
      constexpr int S = decltype(S_)::value;
      load_act(g + 1, ax, NS);  // to LDS at the end of this step
      u32x4 af[2];
      af[0] = frag(S, 0);
      ColAffine ca[CT];
      {
        const u32x4 sb = sbv[S];
        if constexpr (CT == 4) {
          const float sc[4] = {bf16lo(sb.x), bf16hi(sb.x), bf16lo(sb.y), bf16hi(sb.y)};
          const float bi[4] = {bf16lo(sb.z), bf16hi(sb.z), bf16lo(sb.w), bf16hi(sb.w)};
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) ca[ct] = col_affine(sc[ct], bi[ct]);
        } else {
          const uint32_t sp = ch ? sb.y : sb.x, bp = ch ? sb.w : sb.z;
          ca[0] = col_affine(bf16lo(sp), bf16lo(bp));
          ca[1] = col_affine(bf16hi(sp), bf16hi(bp));
        }
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4 bw[CT];  // this k half's B operands
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) bw[ct] = expand_bf16(word(cw[S], 2 * ct + ks), ca[ct], xk);
        // every word of slot S is expanded: its registers take group g + 2
        if (ks == 1) load_w(g + 2, cw[S], sbv[S], CT_);
#pragma unroll
        for (int ms = 0; ms < NS; ++ms) {
          const int f = ks * NS + ms;
          if (f + 1 < 2 * NS) af[(f + 1) % 2] = frag(S, f + 1);
          __builtin_amdgcn_sched_barrier(0);
          const u32x4 av = af[f % 2];
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) acc[ms][ct] = mfma16(av, bw[ct], acc[ms][ct]);
        }
      }
      store_act(1 - S, ax, NS);  // group g + 1
      // the next group's activations are in LDS and every wave is done with
      // this group's stage (written again in the next step)
      lds_barrier();
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    for (int g = 0; g < G; g += 2) {  // G is even for every supported shape
      step(g, I0{});
      step(g + 1, I1{});
    }
  };
  auto run_ns = [&](auto CT_) {
    if (nsub <= 1)
      run(std::integral_constant<int, 1>{}, CT_);
    else if (nsub <= 2)
      run(std::integral_constant<int, 2>{}, CT_);
    else if (nsub <= 4)
      run(std::integral_constant<int, 4>{}, CT_);
    else if (nsub <= 6)
      run(std::integral_constant<int, 6>{}, CT_);
    else if (nsub <= 8)
      run(std::integral_constant<int, 8>{}, CT_);
    else
      run(std::integral_constant<int, kWSub>{}, CT_);
  };
  if constexpr (MODE == kGateUp) {
    if (hsel >= 0) {
      run_ns(std::integral_constant<int, 2>{});
    } else {
      run_ns(std::integral_constant<int, 4>{});
    }
  } else {
    run_ns(std::integral_constant<int, 4>{});
  }

  // ---- epilogue: per-wave transpose through this wave's 9 KB of LDS (the
  // last step's barrier ended every read of the activation stages)
  uint8_t* tb = &L.tr[wave][0];
  if (!wt_active) return;
  if (MODE == kGateUp) {
    // h = bf16(silu(gate) * up), gate/up in 16-column tile pairs (2 j, 2 j + 1):
    // up to 144 rows x CW intermediate columns (CW = 32 whole, 16 in a half)
    const int I = a.N;
    uint16_t* trb = reinterpret_cast<uint16_t*>(tb);
    auto store_h = [&](auto CW_) {
      constexpr int CW = decltype(CW_)::value;
#pragma unroll
      for (int ms = 0; ms < kWSub; ++ms) {
        if (ms < nsub) {
#pragma unroll
          for (int j = 0; j < CW / 16; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              trb[(16 * ms + 4 * kb + i) * CW + 16 * j + c16] =
                  f2bf(silu(acc[ms][2 * j][i]) * acc[ms][2 * j + 1][i]);
        }
      }
      // (a wave's LDS accesses execute in order: no wait between its writes
      // and its reads of the other lanes' values)
      wide_fence();
      constexpr int kChunks = CW / 8;  // 16-byte pieces per row
      constexpr int kQ = (kWRows * kChunks + 63) / 64;
      const int col0 = 32 * wt + 16 * ch;
      // all of the lane's reads first, then the stores (one LDS wait, not
      // one per store); rows past the item read this wave's own buffer
      // (kWRows rows) and are not stored
      u32x4 v[kQ];
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        const int c = lane + 64 * q, r = min(c / kChunks, kWRows - 1), pc = c % kChunks;
        v[q] = *reinterpret_cast<const u32x4*>(trb + r * CW + 8 * pc);
      }
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        const int c = lane + 64 * q, r = c / kChunks, pc = c % kChunks;
        if (r < rows) *reinterpret_cast<u32x4*>(a.h_out + (int64_t)(row0 + r) * I + col0 + 8 * pc) = v[q];
      }
    };
    if (hsel < 0)
      store_h(std::integral_constant<int, 32>{});
    else
      store_h(std::integral_constant<int, 16>{});
  } else {
    // 32 rows x 64 columns of fp32 per round (down has no column halves)
    float* trf = reinterpret_cast<float*>(tb);
#pragma unroll
    for (int mp = 0; mp < (kWSub + 1) / 2; ++mp) {
      if (2 * mp < nsub) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
          if (2 * mp + h2 < kWSub)
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) trf[(16 * h2 + 4 * kb + i) * 64 + 16 * ct + c16] = acc[2 * mp + h2][ct][i];
        wide_fence();
        // the round's eight values and output rows read first (one LDS wait,
        // not one per store; the output-row table covers every row read)
        f32x4 v[8];
        int orow[8];
        const int col = 64 * wt + 4 * (lane & 15);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int r = (lane >> 4) + 4 * q;
          v[q] = *reinterpret_cast<const f32x4*>(trf + r * 64 + 4 * (lane & 15));
          orow[q] = L.outrow[32 * mp + r];
        }
        if (routed) {
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            if (32 * mp + (lane >> 4) + 4 * q < rows) {
              u32x2 o;
              o.x = pack_bf16x2(v[q].x, v[q].y);
              o.y = pack_bf16x2(v[q].z, v[q].w);
              *reinterpret_cast<u32x2*>(a.partial_r + (int64_t)orow[q] * a.N + col) = o;
            }
          }
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q)
            if (32 * mp + (lane >> 4) + 4 * q < rows)
              *reinterpret_cast<f32x4*>(a.partial_s + (int64_t)orow[q] * a.N + col) = v[q];
        }
        wide_fence();
      }
    }
  }
}

hipError_t launch_gemm_wide(GemmMode mode, const GemmArgs& a_in, int max_slots, hipStream_t s) {
  GemmArgs a = a_in;
  const PackGeom geom = pack_geom(a.N, a.K, a.paired);
  if (a.K % (2 * kGroup) || max_slots <= 0) return hipErrorInvalidValue;
  a.cus = compute_units();
  const int n_tiles = (geom.n_wt + kWWaves - 1) / kWWaves;
  const int64_t blocks = 8LL * n_tiles * ((max_slots + 7) / 8);
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (mode == kGateUp)
    hipLaunchKernelGGL(gemm_wide_kernel<kGateUp>, dim3((unsigned)blocks), dim3(kWThreads), 0, s, a);
  else
    hipLaunchKernelGGL(gemm_wide_kernel<kDown>, dim3((unsigned)blocks), dim3(kWThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
