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
//   - the activation rows of the group are gathered through the routing
//     permutation into LDS (double buffered, one barrier per group);
//   - each wave loads its 2 KB of packed codes and 128 B of scales with
//     coalesced 16-byte loads (one group ahead) and expands each code to the
//     exact bf16 value 128 + q with two bit operations (no arithmetic);
//   - the matrix cores form P = x . (128 + q) for the group in fp32 and the
//     group's scale is applied on the accumulator: acc += s * P.
// The bias term sum_g (b - 128 s) * sum_{c in g} x_c is added at the end by
// three more matrix-core K-steps over precomputed per-group sums of the
// activations (hi/lo bf16 halves) and the per-group (b - 128 s) (hi/lo).
// Algebraically this is x . (q*s + b) with the weights used exactly.
//
// Epilogues: gate/up -> h = silu(gate) * up rounded to bf16, plus the per-64
// column sums of h for the down GEMM's bias term; routed down -> the output
// times the pair's routing weight, stored in fp32 per pair; shared down ->
// y = bf16(shared + sum over the k pairs of the token), in a fixed order.
#include "kernels.h"

namespace moe {

template <int MODE>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  const int wt = nt * 4 + wave;
  const uint8_t* ebase = expert >= 0 ? a.blob + (int64_t)expert * a.expert_bytes : a.shared_blob;
  const uint8_t* nib = ebase + geom.nib_off + ((int64_t)wt * G * 64 + lane) * 32;
  const uint8_t* scl = ebase + geom.scl_off + ((int64_t)wt * G * 16 + c16) * 8;

  __shared__ u32x4 lds_a[2][512];        // [buf][ms 4][c 8][row 16] x 16 B
  __shared__ int rowidx[kItemRows];      // activation row of each item row
  __shared__ int pair_s[kItemRows];
  __shared__ float wgt_s[kItemRows];
  __shared__ float red[4][kItemRows];

  if (tid < kItemRows) {
    int ri = 0, pr = 0;
    float wv = 0.f;
    if (tid < rows) {
      if (MODE == kGateUp) {
        ri = expert >= 0 ? a.perm[row0 + tid] / a.k : token0 + tid;
      } else {
        ri = row0 + tid;
        if (MODE == kDownRouted) {
          pr = a.perm[row0 + tid];
          wv = a.topk_w[pr];
        }
      }
    }
    rowidx[tid] = ri;
    pair_s[tid] = pr;
    wgt_s[tid] = wv;
  }
  __syncthreads();

  const int nsub = (rows + 15) >> 4;
  // staging units: u = tid + 256 i -> (ms = u >> 7, chunk c = (u >> 4) & 7, row r16 = u & 15)
  const uint16_t* src[2];
  bool live[2];
  for (int i = 0; i < 2; ++i) {
    const int u = tid + 256 * i;
    const int m = (u >> 7) * 16 + (u & 15);
    live[i] = m < rows;
    src[i] = a.act + (int64_t)rowidx[live[i] ? m : 0] * K + 8 * ((u >> 4) & 7);
  }
  u32x4 stage[2];
  auto stage_load = [&](int g) {
    for (int i = 0; i < 2; ++i)
      if (live[i]) stage[i] = *reinterpret_cast<const u32x4*>(src[i] + g * kGroup);
  };
  auto stage_store = [&](int buf) {
    for (int i = 0; i < 2; ++i)
      if (live[i]) lds_a[buf][tid + 256 * i] = stage[i];
  };

  f32x4 acc[4][4];
  for (int ms = 0; ms < 4; ++ms)
    for (int ct = 0; ct < 4; ++ct) acc[ms][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 w0 = *reinterpret_cast<const u32x4*>(nib);
  u32x4 w1 = *reinterpret_cast<const u32x4*>(nib + 16);
  u32x2 sc = *reinterpret_cast<const u32x2*>(scl);
  stage_load(0);
  stage_store(0);
  lds_barrier();

  for (int g = 0; g < G; ++g) {
    const int buf = g & 1;
    const bool more = g + 1 < G;
    u32x4 nw0 = w0, nw1 = w1;
    u32x2 nsc = sc;
    if (more) {
      stage_load(g + 1);
      nw0 = *reinterpret_cast<const u32x4*>(nib + (int64_t)(g + 1) * 64 * 32);
      nw1 = *reinterpret_cast<const u32x4*>(nib + (int64_t)(g + 1) * 64 * 32 + 16);
      nsc = *reinterpret_cast<const u32x2*>(scl + (int64_t)(g + 1) * 16 * 8);
    }
    u32x4 bq[4][2];
    bq[0][0] = expand_codes(w0.x);
    bq[0][1] = expand_codes(w0.y);
    bq[1][0] = expand_codes(w0.z);
    bq[1][1] = expand_codes(w0.w);
    bq[2][0] = expand_codes(w1.x);
    bq[2][1] = expand_codes(w1.y);
    bq[3][0] = expand_codes(w1.z);
    bq[3][1] = expand_codes(w1.w);
    const float s[4] = {bf16lo(sc.x), bf16hi(sc.x), bf16lo(sc.y), bf16hi(sc.y)};
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) {
      if (ms < nsub) {
        const u32x4 a0 = lds_a[buf][(ms * 8 + kb) * 16 + c16];
        const u32x4 a1 = lds_a[buf][(ms * 8 + 4 + kb) * 16 + c16];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          f32x4 p = mfma16(a0, bq[ct][0], f32x4{0.f, 0.f, 0.f, 0.f});
          p = mfma16(a1, bq[ct][1], p);
          acc[ms][ct] += s[ct] * p;
        }
      }
    }
    if (more) stage_store(buf ^ 1);
    lds_barrier();
    w0 = nw0;
    w1 = nw1;
    sc = nsc;
  }

  // bias term: sum_g (b - 128 s)[col][g] * xsum[row][g] over three K-steps
  {
    const int Gp = geom.Gp;
    const uint8_t* bia = ebase + geom.bia_off;
    const uint8_t* sclb = ebase + geom.scl_off;
    for (int k0s = 0; k0s < a.Kx; k0s += 32) {
      const int k0 = k0s + 8 * kb;
      const int seg = k0 / Gp, gg0 = k0 % Gp;
      u32x4 be[4];
      for (int ct = 0; ct < 4; ++ct) be[ct] = u32x4{0u, 0u, 0u, 0u};
      if (seg < 3) {
        float bv[4][8], sv[4][8];
        for (int ct = 0; ct < 4; ++ct) {
          const int j = 16 * ct + c16;
          const u32x4 b8 = *reinterpret_cast<const u32x4*>(bia + (((int64_t)wt * kWaveCols + j) * Gp + gg0) * 2);
          bv[ct][0] = bf16lo(b8.x); bv[ct][1] = bf16hi(b8.x);
          bv[ct][2] = bf16lo(b8.y); bv[ct][3] = bf16hi(b8.y);
          bv[ct][4] = bf16lo(b8.z); bv[ct][5] = bf16hi(b8.z);
          bv[ct][6] = bf16lo(b8.w); bv[ct][7] = bf16hi(b8.w);
        }
        for (int o = 0; o < 8; ++o) {
          const int g = gg0 + o;
          u32x2 s4 = u32x2{0u, 0u};
          if (g < G) s4 = *reinterpret_cast<const u32x2*>(sclb + (((int64_t)wt * G + g) * 16 + c16) * 8);
          sv[0][o] = bf16lo(s4.x); sv[1][o] = bf16hi(s4.x);
          sv[2][o] = bf16lo(s4.y); sv[3][o] = bf16hi(s4.y);
        }
        for (int ct = 0; ct < 4; ++ct) {
          uint16_t h16[8];
          for (int o = 0; o < 8; ++o) {
            uint16_t hi, lo;
            split_hi_lo(bv[ct][o] - 128.0f * sv[ct][o], hi, lo);
            h16[o] = seg == 1 ? lo : hi;
          }
          be[ct] = u32x4{h16[0] | ((uint32_t)h16[1] << 16), h16[2] | ((uint32_t)h16[3] << 16),
                         h16[4] | ((uint32_t)h16[5] << 16), h16[6] | ((uint32_t)h16[7] << 16)};
        }
      }
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) {
        if (ms < nsub) {
          const int m = ms * 16 + c16;
          u32x4 ax = u32x4{0u, 0u, 0u, 0u};
          if (m < rows)
            ax = *reinterpret_cast<const u32x4*>(a.act3 + (int64_t)rowidx[m] * a.Kx + k0);
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) acc[ms][ct] = mfma16(ax, be[ct], acc[ms][ct]);
        }
      }
    }
  }

  if (MODE == kGateUp) {
    const int I = a.N;
    float hs[4][4];
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) {
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
        if (c16 == 0) red[wave][ms * 16 + 4 * kb + i] = v;
      }
    }
    __syncthreads();
    const int Gd = I / kGroup, Gpd = round_up(Gd, 8);
    if (tid < 128) {
      const int w2 = tid >> 6, r = tid & 63;
      if (r < rows) {
        const float v = red[2 * w2][r] + red[2 * w2 + 1][r];
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
  } else if (MODE == kDownRouted) {
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) {
      if (ms < nsub) {
        for (int i = 0; i < 4; ++i) {
          const int r = ms * 16 + 4 * kb + i;
          if (r < rows) {
            float* o = a.partial + (int64_t)pair_s[r] * a.N + 64 * wt + c16;
            const float wv = wgt_s[r];
            for (int ct = 0; ct < 4; ++ct) o[16 * ct] = wv * acc[ms][ct][i];
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) {
      if (ms < nsub) {
        for (int i = 0; i < 4; ++i) {
          const int r = ms * 16 + 4 * kb + i;
          if (r < rows) {
            const int t = token0 + r;
            const float* pp = a.partial + (int64_t)t * a.k * a.N + 64 * wt + c16;
            uint16_t* o = a.y + (int64_t)t * a.N + 64 * wt + c16;
            for (int ct = 0; ct < 4; ++ct) {
              float v = acc[ms][ct][i];
              for (int j = 0; j < a.k; ++j) v += pp[(int64_t)j * a.N + 16 * ct];
              o[16 * ct] = f2bf(v);
            }
          }
        }
      }
    }
  }
}

// Test hook: expand one expert's packed matrices with the GEMM's own loads and
// code expansion. Grid: (n_wt, G); block: 64 threads (one wave).
__global__ void test_dequant_kernel(const uint8_t* ebase, int N, int K, int paired, float* out) {
  const int lane = threadIdx.x, c16 = lane & 15, kb = lane >> 4;
  const int wt = blockIdx.x, g = blockIdx.y;
  const PackGeom geom = pack_geom(N, K, paired);
  const int G = geom.G;
  const uint8_t* nib = ebase + geom.nib_off + (((int64_t)wt * G + g) * 64 + lane) * 32;
  const uint8_t* scl = ebase + geom.scl_off + (((int64_t)wt * G + g) * 16 + c16) * 8;
  const u32x4 w0 = *reinterpret_cast<const u32x4*>(nib);
  const u32x4 w1 = *reinterpret_cast<const u32x4*>(nib + 16);
  const u32x2 sc = *reinterpret_cast<const u32x2*>(scl);
  const uint32_t words[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  const float s[4] = {bf16lo(sc.x), bf16hi(sc.x), bf16lo(sc.y), bf16hi(sc.y)};
  const uint16_t* bia = reinterpret_cast<const uint16_t*>(ebase + geom.bia_off);
  for (int ct = 0; ct < 4; ++ct) {
    const int j = 16 * ct + c16;
    const float b = bf16f(bia[((int64_t)wt * kWaveCols + j) * geom.Gp + g]);
    int mat = 0, row = 64 * wt + j;
    if (paired) {
      mat = j >> 5;
      row = 32 * wt + (j & 31);
    }
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4 v = expand_codes(words[2 * ct + ks]);
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
  else if (mode == kDownRouted)
    hipLaunchKernelGGL(gemm_kernel<kDownRouted>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(gemm_kernel<kDownShared>, grid, block, 0, s, a);
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
