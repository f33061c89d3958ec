// Internal kernel interfaces of the int4 MoE library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "device.h"
#include "layout.h"

namespace moe {

constexpr int kChunkPairs = 1024;  // (token, slot) pairs per scatter block
constexpr int kItemRows = 32;      // most rows of one expert per GEMM work item (one routing block)
constexpr int kWideRows = 144;     // rows per work item of the wide GEMMs
constexpr int kMaxGroups = 64;     // K / 64 upper bound of the expert GEMMs
constexpr int kDecodeMaxT = 4;
constexpr int kMaxSplits = 8;      // router K splits summed by the top-k kernel

struct TopkArgs {
  const float* partial;   // [splits][T][E]
  int splits;
  const float* rbias;     // [E] or null
  float* logits_out;      // [T][E] or null
  int32_t* topk_idx;      // [T][k]
  float* topk_w;          // [T][k]
  int32_t* chunk_hist;    // [chunks][E] (zeroed beforehand) or null
  int T, E, k;
};

struct ScatterArgs {
  const int32_t* topk_idx;
  const int32_t* chunk_hist;
  int32_t *hist, *offsets, *perm, *inv_perm, *block_map, *num_blocks;
  int32_t *items, *num_items;  // GEMM work list or null
  int T, E, k, block_m;
  int item_rows;               // rows per GEMM work item
  int longest_first;           // 1: the work list holds every expert's full items
                               // (expert order), then the experts' last partial
                               // items, larger first (ties: lower expert)
};

// Which GEMM: gate/up with SwiGLU, or down (routed and shared items) writing
// per-(token, slot) fp32 rows that the combine kernel sums into y.
enum GemmMode { kGateUp = 0, kDown = 1 };

struct GemmArgs {
  const int32_t* items;      // routed work list [max][3] (expert, first row, rows)
  const int32_t* num_items;  // device scalar
  int shared_slots;          // shared-expert items (item_rows tokens each)
  int item_rows;             // rows per work item, <= kItemRows (the routing block size)
  const uint8_t* blob;       // routed experts (past the header)
  const uint8_t* shared_blob;
  int64_t expert_bytes;
  int N, K, paired;          // packed geometry of this matrix set
  int bf16_weights;          // 1: blob / shared_blob hold bf16-expanded weights (no header)
  int T;                     // tokens in this chunk
  int k;                     // experts per token
  // activations
  const uint16_t* act;       // gate/up: x [T][K]; down: h [(k+1)T][K]
  const int32_t* perm;       // [kT]
  // outputs
  uint16_t* h_out;           // gate/up: h [(k+1)T][N] bf16
  uint16_t* partial_r;       // down, routed rows: [T*k][N] bf16 at pair p = t*k + j
  float* partial_s;          // down, shared-expert rows: [T][N] fp32
  int cus;                   // wide GEMMs: compute units (set by the launcher)
};

// Compute units of the current device, rounded down to a multiple of 8 (the
// XCD count); cached per device.
int compute_units();

hipError_t launch_router(const uint16_t* x, const uint16_t* planes, float* partial, int T, int H,
                         int E, int splits, int* zero_buf, int zero_count, hipStream_t s);
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);
hipError_t launch_scan_scatter(const ScatterArgs& a, hipStream_t s);
hipError_t launch_fill_zero(int* p, int n, hipStream_t s);
// grid_blocks > 0: that many blocks (rounded up to a multiple of 8) instead
// of the persistent grid (used when the host knows the exact unit count).
hipError_t launch_gemm(GemmMode mode, const GemmArgs& a, hipStream_t s, int grid_blocks = 0);
// The wide GEMMs (items of up to kWideRows rows, weights expanded to bf16
// once per item): a.items / a.num_items hold kWideRows-row items and
// a.shared_slots counts kWideRows-token shared items; max_slots bounds
// items + shared items (the grid is sized from it, extra blocks exit).
hipError_t launch_gemm_wide(GemmMode mode, const GemmArgs& a, int max_slots, hipStream_t s);
// y[t][n] = bf16(shared[t][n] + sum_{j<k} topk_w[t][j] * routed[t*k + j][n]) (j ascending).
hipError_t launch_combine(const uint16_t* routed, const float* shared, const float* topk_w, uint16_t* y,
                          int T, int N, int k, hipStream_t s);
// The unfused comparison path: every expert of a packed blob with rows (hist
// null or hist[e] > 0), and the shared expert, expanded to bf16 w = q s + b
// (one rounding) into `out` / `out_shared` in the kBf16GroupBytes layout.
hipError_t launch_expand_bf16(const uint8_t* blob, int64_t expert_bytes, const uint8_t* shared_blob,
                              int count, const int32_t* hist, int N, int K, int paired, uint8_t* out,
                              uint8_t* out_shared, hipStream_t s);
hipError_t launch_test_dequant(const uint8_t* expert_base, int N, int K, int paired, float* out,
                               hipStream_t s);

struct DecodeArgs {
  const uint16_t* x;          // [T][H]
  const float* router_w;      // [E][H]
  const float* rbias;         // [E] or null
  float* logits;              // [T][E]
  float* logits_out;          // [T][E] or null
  int32_t* topk_idx;          // [T][k]
  float* topk_w;              // [T][k]
  int32_t *hist, *offsets, *perm, *inv_perm, *block_map, *num_blocks;  // optional route_out
  const uint8_t* gu_blob;     // routed gate/up experts (past header)
  const uint8_t* gu_shared;
  int64_t gu_expert_bytes;
  const uint8_t* dn_blob;
  const uint8_t* dn_shared;
  int64_t dn_expert_bytes;
  uint16_t* h;                // [k*T + T][I] bf16 (slot order: pairs, then shared)
  uint16_t* y;                // [T][H]
  int T, H, I, E, k, block_m;
};

// ev (optional): four events recorded before each of the three launches and after the last.
// Requires k == 8.
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s, hipEvent_t* ev = nullptr);

}  // namespace moe
