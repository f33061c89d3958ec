// Packed-weight geometry shared by the host packer and the gfx950 kernels.
//
// Expert matrices are stored for the 16x16x32 bf16 matrix-core instruction.
// A "wave tile" is 64 output columns of one expert (16 columns per MFMA tile,
// four tiles per wave) and the unit of K is one quantisation group of 64
// inputs (two MFMA K-steps of 32). For lane l of a wave, c16 = l & 15 picks
// the column inside a 16-column tile and kb = l >> 4 picks eight consecutive
// inputs inside a 32-input K-step; the A (activation) and B (weight) operands
// use the same (kb, element) -> k assignment, so the contraction is exact
// whatever order the hardware walks K in.
//
// Per expert, two regions (byte offsets from the expert base):
//   nib  [wt][g][half 2][lane 64][16 B]  eight u32 words per lane, words
//        0..3 in half 0 and 4..7 in half 1 (so each half is one contiguous
//        1 KB wave load): word 2*ct + ks holds the codes of column 16*ct + c16
//        for k = 64g + 32ks + 8kb + o, o = 0..7, code o at nibble position
//        (o & 1) * 4 + (o >> 1); with that order ((w >> 4d) & 0x000F000F) |
//        0x43004300 is the bf16 pair (128 + q[2d], 128 + q[2d+1]), d = 0..3.
//   sb   [wt][g][c16 16][8 bf16]  entries 0..3: scale of column 16*ct + c16
//        (ct = 0..3), entries 4..7: bias of the same columns, group g; one
//        16-byte word per (column slot, group), 256 B per (wave tile, group).
// Column j = 16*ct + c16 of wave tile wt is matrix row 64*wt + j (one
// matrix), or, with two matrices (gate, up) per expert, row
// 32*wt + 16*(ct >> 1) + c16 of gate (ct even) or up (ct odd): each 16-column
// tile of gate is followed by the up tile of the same 16 intermediate columns,
// so any half wave tile (1 KB of codes per group) carries a complete SwiGLU
// pair.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace moe {

constexpr int kGroup = 64;          // inputs per quantisation group
constexpr int kWaveCols = 64;       // output columns per wave tile
constexpr int kNibBytes = 2048;     // packed codes per (wave tile, group)
constexpr int kSbBytes = 256;       // scales + biases per (wave tile, group)
// The same weights expanded to bf16 (the unfused comparison path): per (wave
// tile, group) 8 words x 64 lanes x 16 bytes, word w = 2 ct + ks holding the
// B operand that code word w expands to.
constexpr int kBf16GroupBytes = 8 * 64 * 16;
constexpr int kHeaderBytes = 256;   // blob header
constexpr uint32_t kMagic = 0x4734494Du;  // "MI4G"
constexpr uint32_t kRouterMagic = 0x3346424Du;  // "MBF3"
constexpr int kVersion = 3;

__host__ __device__ inline int round_up(int v, int m) { return (v + m - 1) / m * m; }

struct PackGeom {
  int N, K, paired;
  int n_eff;   // output columns per expert (2N when paired)
  int n_wt;    // wave tiles per expert
  int G;       // groups along K
  int64_t nib_off, sb_off, expert_bytes;
};

__host__ __device__ inline PackGeom pack_geom(int N, int K, int paired) {
  PackGeom g;
  g.N = N;
  g.K = K;
  g.paired = paired ? 1 : 0;
  g.n_eff = paired ? 2 * N : N;
  g.n_wt = g.n_eff / kWaveCols;
  g.G = K / kGroup;
  g.nib_off = 0;
  g.sb_off = (int64_t)g.n_wt * g.G * kNibBytes;
  int64_t end = g.sb_off + (int64_t)g.n_wt * g.G * kSbBytes;
  g.expert_bytes = (end + 255) / 256 * 256;
  return g;
}

// u32 index (from the expert's nib base) of word u (0..7) of `lane`.
__host__ __device__ inline int64_t nib_word(int wt, int g, int lane, int u, int G) {
  return ((((int64_t)wt * G + g) * 2 + (u >> 2)) * 64 + lane) * 4 + (u & 3);
}

// Nibble position of code o (0..7) inside its 32-bit word.
__host__ __device__ inline int nibble_pos(int o) { return (o & 1) * 4 + (o >> 1); }

// Router planes: [plane 3][et E/64][g H/64][ct 4][ks 2][lane 64][8 bf16].
__host__ __device__ inline int64_t router_index(int plane, int et, int g, int ct, int ks, int lane,
                                                int n_et, int G) {
  return ((((((int64_t)plane * n_et + et) * G + g) * 4 + ct) * 2 + ks) * 64 + lane) * 8;
}

}  // namespace moe
