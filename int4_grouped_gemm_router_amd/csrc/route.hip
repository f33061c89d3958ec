// Router and GPU-resident routing for the int4 MoE layer (gfx950).
//
// diariobitcoin.com, "Perplexity libera Lily, un motor de IA que supera a
// MLX-LM en Apple Silicon": section "Qwen3.6 combina tres cargas de trabajo"
// (a router scores the experts and keeps eight per token) and section "Las
// optimizaciones en el prefill" (routing histogram, prefix scan, scatter and
// block map stay on the GPU, with no CPU synchronisation inside the layer).
//
// Kernels, all enqueued on one stream with grids sized from host-known upper
// bounds so that nothing is read back:
//   router_mfma   logits partials: x (bf16) * Wr (three exact bf16 planes)
//                 on the matrix cores, fp32 accumulation, split along H
//   topk          per token: sum of the partials (+ router bias), top-k with
//                 ties to the lower index, renormalised softmax weights and
//                 per-chunk expert counts
//   scan_scatter  per chunk of 1024 pairs: expert offsets (exclusive scan),
//                 the chunk's base per expert, a stable scatter of the pairs
//                 (wave ballot peer matching), and, in block 0, the histogram,
//                 offsets, the 32-row block map and the GEMM work list.
#include "kernels.h"
#include "topk.h"

namespace moe {

// ---------------------------------------------------------------- router

// Grid: (ceil(T/(16 NW)), E/(16 CT), KS). Block: NW waves (4, or 8 for long
// chunks, which halves how often the weight tile is re-read); wave w owns
// tokens [16 NW bx + 16w, +16) and all 16 CT experts of the block's tile (CT
// MFMA tiles: 2 below 1024 tokens, which doubles the blocks, else 4).
// The three bf16 planes of the weight tile (6 CT KB per 64-input group) are
// shared by the waves: they arrive in a three-stage LDS ring by asynchronous
// global -> LDS copies, 6 CT / NW 1 KB copies per wave per group; the
// activation fragments arrive in a register ring alongside.
constexpr int kRStages = 3;

template <int LOADS>
__device__ inline void router_wait(int groups) {
  // LOADS loads per group per wave: the plane copies and two activation loads
  static_assert(LOADS == 5 || LOADS == 8, "wait counts of the instantiated tilings");
  if (groups >= 1) {
    if constexpr (LOADS == 5)
      asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

template <int NW, int CT>
__global__ __launch_bounds__(NW * 64) void router_mfma_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ planes,
                                                          float* __restrict__ partial, int T,
                                                          int H, int E, int groups_per_split,
                                                          int* __restrict__ zero_buf,
                                                          int zero_count) {
  // CT of the four 16-expert column tiles of a 64-expert plane tile per block
  __shared__ u32x4 bt[kRStages][3 * 2 * CT * 64];  // [stage][plane][ct][ks 2][lane 64]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15, kb = lane >> 4;
  const int tt = blockIdx.x, split = blockIdx.z;
  const int et = blockIdx.y / (4 / CT), ct0 = CT * (blockIdx.y % (4 / CT));
  const int G = H / kGroup, n_et = E / 64;
  if (zero_buf && tt == 0 && blockIdx.y == 0 && split == 0)
    for (int i = threadIdx.x; i < zero_count; i += blockDim.x) zero_buf[i] = 0;

  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  static_assert(CT == 2 || CT == 4, "half or whole plane tiles");
  constexpr int kChunks = 3 * 2 * CT;       // 1 KB plane chunks per group
  constexpr int kCopies = kChunks / NW;     // per wave
  static_assert(kCopies * NW == kChunks, "chunks split evenly over the waves");
  const int row = tt * 16 * NW + wave * 16 + c16;
  const bool row_ok = row < T;
  const uint16_t* xr = x + (int64_t)(row_ok ? row : 0) * H + 8 * kb;
  const uint8_t* pl = reinterpret_cast<const uint8_t*>(planes);
  const int g0 = split * groups_per_split, ng = groups_per_split;
  u32x4 aq[kRStages][2];
  auto issue = [&](int gi, int st) {
    const int g = g0 + gi;
#pragma unroll
    for (int i = 0; i < kCopies; ++i) {
      const int q = wave * kCopies + i;      // 1 KB chunk of the block's share
      const int p = q / (2 * CT), part = q % (2 * CT);
      const uint8_t* src =
          pl + ((((int64_t)p * n_et + et) * G + g) * 8 + 2 * ct0 + part) * 1024 + lane * 16;
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)&bt[st][(p * 2 * CT + part) * 64],
                                       16, 0, 0);
    }
    aq[st][0] = *reinterpret_cast<const u32x4*>(xr + g * kGroup);
    aq[st][1] = *reinterpret_cast<const u32x4*>(xr + g * kGroup + 32);
  };
  f32x4 acc[CT];
  for (int ct = 0; ct < CT; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int d = 0; d < kRStages - 1; ++d)
    if (d < ng) issue(d, d);
  for (int gb = 0; gb < ng; gb += kRStages) {
#pragma unroll
    for (int d = 0; d < kRStages; ++d) {
      const int gi = gb + d;
      if (gi >= ng) break;
      router_wait<kCopies + 2>(min(kRStages - 2, ng - 1 - gi));
      lds_barrier();
      if (gi + kRStages - 1 < ng) issue(gi + kRStages - 1, (d + kRStages - 1) % kRStages);
      const u32x4 a0 = row_ok ? aq[d][0] : u32x4{0u, 0u, 0u, 0u};
      const u32x4 a1 = row_ok ? aq[d][1] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          acc[ct] = mfma16(a0, bt[d][(p * 2 * CT + 2 * ct) * 64 + lane], acc[ct]);
          acc[ct] = mfma16(a1, bt[d][(p * 2 * CT + 2 * ct + 1) * 64 + lane], acc[ct]);
        }
    }
  }
  float* out = partial + (int64_t)split * T * E;
  for (int ct = 0; ct < CT; ++ct)
    for (int i = 0; i < 4; ++i) {
      const int t = tt * 16 * NW + wave * 16 + 4 * kb + i;
      if (t < T) out[(int64_t)t * E + et * 64 + (ct0 + ct) * 16 + c16] = acc[ct][i];
    }
}

// ---------------------------------------------------------------- top-k

// Grid: ceil(T/4); one wave per token.
__global__ __launch_bounds__(256) void topk_kernel(TopkArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= a.T) return;
  const int E = a.E, k = a.k, per = E / 64;
  // all partial and bias loads first (splits <= kMaxSplits; unconditional,
  // clamped loads, so that no branch separates them and they share one
  // memory round trip), then a fixed-order sum
  float pv[kMaxSplits][4], rb[4];
  const float* rbias = a.rbias ? a.rbias : a.partial;  // read but unused without a bias
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      pv[sp][i] = a.partial[((int64_t)min(sp, a.splits - 1) * a.T + t) * E + lane + 64 * min(i, per - 1)];
#pragma unroll
  for (int i = 0; i < 4; ++i) rb[i] = rbias[lane + 64 * min(i, per - 1)];
  __builtin_amdgcn_sched_barrier(0);
  float l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    l[i] = -INFINITY;
    if (i < per) {
      const int e = lane + 64 * i;
      float v = 0.f;
#pragma unroll
      for (int sp = 0; sp < kMaxSplits; ++sp) v += sp < a.splits ? pv[sp][i] : 0.f;
      if (a.rbias) v += rb[i];
      if (a.logits_out) a.logits_out[(int64_t)t * E + e] = v;
      l[i] = v == v ? v : -INFINITY;  // a NaN logit ranks as -inf
    }
  }
  // top-k: value descending, index ascending
  uint32_t key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) key[i] = i < per ? logit_key(l[i]) : 0u;
  int sel_e;
  float sel_l;
  wave_topk(key, l, k, lane, sel_e, sel_l);
  const float top = __shfl(sel_l, 0);
  // weights: exp(l_j - l_0) / sum over the k selected
  const float p = lane < k ? expf(sel_l - top) : 0.f;
  const float z = wave_sum(p);
  if (lane < k) {
    const int64_t pair = (int64_t)t * k + lane;
    a.topk_idx[pair] = sel_e;
    a.topk_w[pair] = p / z;
    if (a.chunk_hist) atomicAdd(&a.chunk_hist[(pair / kChunkPairs) * E + sel_e], 1);
  }
}

// ---------------------------------------------------------------- scan + scatter

__device__ inline int block_exclusive_scan(int v, int* scratch /* >= 4 ints */, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(inc, o);
    if (lane >= o) inc += n;
  }
  if (lane == 63) scratch[wave] = inc;
  __syncthreads();
  int base = 0;
  total = 0;
  for (int w = 0; w < 4; ++w) {
    if (w < wave) base += scratch[w];
    total += scratch[w];
  }
  __syncthreads();
  return base + inc - v;
}

// Grid: number of 1024-pair chunks. Block: 256 threads (one per expert).
__global__ __launch_bounds__(256) void scan_scatter_kernel(ScatterArgs a) {
  __shared__ int off_s[256];
  __shared__ int wbase[4][256];
  __shared__ int scratch[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, P = a.T * a.k;
  const int chunk = blockIdx.x;
  const int n_chunks = (P + kChunkPairs - 1) / kChunkPairs;
  // this wave's pair ids, loaded before the scan so both round trips overlap
  const int p0 = chunk * kChunkPairs + wave * 256;
  // (clamped, unconditional loads: no branch separates them)
  int pe[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) pe[r] = a.topk_idx[min(p0 + r * 64 + lane, P - 1)];
  // totals and this chunk's base per expert, eight chunk counts per round trip
  int tot = 0, before = 0;
  const int te = min(tid, E - 1);
  for (int c0 = 0; c0 < n_chunks; c0 += 8) {
    int v[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = a.chunk_hist[min(c0 + c, n_chunks - 1) * E + te];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int cc = c0 + c;
      if (cc < n_chunks && tid < E) {
        tot += v[c];
        if (cc < chunk) before += v[c];
      }
    }
  }
  int total;
  const int off = block_exclusive_scan(tid < E ? tot : 0, scratch, total);
  if (tid < E) off_s[tid] = off;
  if (chunk == 0) {
    if (tid < E) {
      a.hist[tid] = tot;
      a.offsets[tid] = off;
    }
    if (tid == 0) a.offsets[E] = total;
    // 32-row routing blocks
    int nb_total;
    const int nb = tid < E ? (tot + a.block_m - 1) / a.block_m : 0;
    const int boff = block_exclusive_scan(nb, scratch, nb_total);
    for (int i = 0; i < nb; ++i) {
      int* bm = a.block_map + 3 * (int64_t)(boff + i);
      bm[0] = tid;
      bm[1] = off + i * a.block_m;
      bm[2] = min(a.block_m, tot - i * a.block_m);
    }
    if (tid == 0) *a.num_blocks = nb_total;
    // GEMM work items: up to item_rows rows of one expert
    if (a.items && !a.longest_first) {
      int ni_total;
      const int ir = a.item_rows;
      const int ni = tid < E ? (tot + ir - 1) / ir : 0;
      const int ioff = block_exclusive_scan(ni, scratch, ni_total);
      for (int i = 0; i < ni; ++i) {
        int* it = a.items + 3 * (int64_t)(ioff + i);
        it[0] = tid;
        it[1] = off + i * ir;
        it[2] = min(ir, tot - i * ir);
      }
      if (tid == 0) *a.num_items = ni_total;
    } else if (a.items) {
      // full items first, then each expert's partial last item, larger
      // first: blocks are handed out in work-list order, so the short items
      // fill the end of the launch (longest-processing-time-first order)
      int nf_total;
      const int ir = a.item_rows;
      const int nf = tid < E ? tot / ir : 0;
      const int rem = tid < E ? tot - nf * ir : 0;
      const int foff = block_exclusive_scan(nf, scratch, nf_total);
      for (int i = 0; i < nf; ++i) {
        int* it = a.items + 3 * (int64_t)(foff + i);
        it[0] = tid;
        it[1] = off + i * ir;
        it[2] = ir;
      }
      // rank among the partial items (remainder sizes 1 .. ir - 1 < 256):
      // a counting sort, larger first, equal sizes by expert index. Per wave,
      // ballot matching finds the lanes with the same size; wbase (not yet in
      // use) holds each wave's count per size, then the counts of all sizes
      // above each size.
      int* rcnt = &wbase[0][0];                 // [4 waves][256 sizes]
      for (int i = tid; i < 4 * 256; i += 256) rcnt[i] = 0;
      __syncthreads();
      const uint64_t peers = match_any((uint32_t)rem, 8);
      const int wrank = __popcll(peers & lanemask_lt());
      if (rem > 0 && wrank == 0) rcnt[wave * 256 + rem] = __popcll(peers);
      __syncthreads();
      int before_w = 0;
      for (int w = 0; w < 4; ++w) before_w += w < wave ? rcnt[w * 256 + rem] : 0;
      const int b = 255 - tid;                  // sizes in descending order
      const int cb = b >= 1 ? rcnt[b] + rcnt[256 + b] + rcnt[512 + b] + rcnt[768 + b] : 0;
      int nrem;
      const int above = block_exclusive_scan(cb, scratch, nrem);
      off_s[b] = above;                         // items of sizes larger than b
      __syncthreads();
      if (rem > 0) {
        const int rank = off_s[rem] + before_w + wrank;
        int* it = a.items + 3 * (int64_t)(nf_total + rank);
        it[0] = tid;
        it[1] = off + nf * ir;
        it[2] = rem;
      }
      if (tid == 0) *a.num_items = nf_total + nrem;
      __syncthreads();
      if (tid < E) off_s[tid] = off;
    }
  }
  // wave-level counts of this chunk's pairs: wave w owns 256 consecutive pairs
  for (int i = tid; i < 4 * 256; i += 256) (&wbase[0][0])[i] = 0;
  __syncthreads();
  for (int r = 0; r < 4; ++r) {
    const int p = p0 + r * 64 + lane;
    if (p < P) atomicAdd(&wbase[wave][pe[r]], 1);
  }
  __syncthreads();
  if (tid < E) {
    int run = off_s[tid] + before;
    for (int w = 0; w < 4; ++w) {
      const int c = wbase[w][tid];
      wbase[w][tid] = run;
      run += c;
    }
  }
  __syncthreads();
  // stable scatter: rank among equal experts inside each 64-pair round
  for (int r = 0; r < 4; ++r) {
    const int p = p0 + r * 64 + lane;
    if (p < P) {
      const int e = pe[r];
      const uint64_t peers = match_any((uint32_t)e, 8);
      const int rank = __popcll(peers & lanemask_lt());
      const int pos = wbase[wave][e] + rank;
      a.perm[pos] = p;
      a.inv_perm[p] = pos;
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      if (rank == 0) wbase[wave][e] += __popcll(peers);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  }
}

__global__ void fill_zero_kernel(int* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// ---------------------------------------------------------------- launchers

// From this many tokens the router takes 128-token tiles (8 waves per block;
// below it, 64-token tiles keep enough blocks to fill the chip).
constexpr int kRouterWideMinT = 1024;

hipError_t launch_router(const uint16_t* x, const uint16_t* planes, float* partial, int T, int H,
                         int E, int splits, int* zero_buf, int zero_count, hipStream_t s) {
  const int G = H / kGroup;
  if (T >= kRouterWideMinT) {
    const dim3 grid((T + 127) / 128, E / 64, splits);
    hipLaunchKernelGGL((router_mfma_kernel<8, 4>), grid, dim3(512), 0, s, x, planes, partial, T, H, E,
                       G / splits, zero_buf, zero_count);
  } else {
    const dim3 grid((T + 63) / 64, E / 32, splits);
    hipLaunchKernelGGL((router_mfma_kernel<4, 2>), grid, dim3(256), 0, s, x, planes, partial, T, H, E,
                       G / splits, zero_buf, zero_count);
  }
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(topk_kernel, dim3((a.T + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_scan_scatter(const ScatterArgs& a, hipStream_t s) {
  const int P = a.T * a.k;
  hipLaunchKernelGGL(scan_scatter_kernel, dim3((P + kChunkPairs - 1) / kChunkPairs), dim3(256),
                     0, s, a);
  return hipGetLastError();
}

hipError_t launch_fill_zero(int* p, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace moe
