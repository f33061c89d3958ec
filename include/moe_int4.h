/*
 * moe_int4.h — C ABI of the MI355X (gfx950) int4 mixture-of-experts layer.
 *
 * The layer: a router scores E experts per token and keeps the top k, a
 * shared expert sees every token, and each expert is a SwiGLU MLP whose three
 * matrices are stored as affine 4-bit integers in groups of 64 with a bf16
 * scale and bias per group. The routing metadata (histogram, prefix scan,
 * scatter, block map) is built on the GPU on the caller's stream with no host
 * synchronisation, and the expert GEMMs read the packed weights and expand
 * them tile by tile on chip with fp32 accumulation.
 *   Sources: diariobitcoin.com, "Perplexity libera Lily, un motor de IA que
 *   supera a MLX-LM en Apple Silicon", sections "Qwen3.6 combina tres cargas de
 *   trabajo" (256 experts, eight per token, shared expert; 4-bit affine g64
 *   format), "Las optimizaciones en el prefill" (dequant fused in the grouped
 *   GEMM, fp32 accumulation; routing histogram, prefix scan, scatter and block
 *   map kept on the GPU; 32-row blocks; bounded prefill chunks) and "El decode
 *   busca mover menos datos" (batch-1 decode is bandwidth bound).
 *
 * Conventions for every entry point:
 *  - Pointers marked "device" are HIP device pointers; "host" are host memory.
 *    bf16 values are passed as uint16_t bit patterns.
 *  - The caller owns every buffer. The library never allocates, frees or keeps
 *    pointers after a call returns; device buffers must stay valid until the
 *    work enqueued on `stream` completes.
 *  - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *    asynchronously; no entry point synchronises the host. Device faults
 *    surface at the caller's next synchronisation.
 *  - Return value: MOE_OK (0) or a negative MOE_E* code. Arguments are checked
 *    before anything is enqueued, so on error nothing has been launched.
 *  - Alignment: x, y, the workspace, the unfused weight buffer, router_w and
 *    the packed blobs must be 16-byte aligned (the kernels move them in
 *    16-byte vectors); logits, logits_out, router_bias and the route_out
 *    arrays 4-byte aligned. Misaligned pointers give MOE_EINVAL. (Fresh
 *    torch / hipMalloc allocations are 256-byte aligned.)
 *  - Supported dims: E <= 256 and E % 64 == 0, top_k == 8, gemm one of
 *    MOE_GEMM_*, block_m 32 or 16
 *    (the routing block size, which is also the row count of the exact
 *    grouped GEMMs' work items; diariobitcoin.com, "Perplexity libera Lily...",
 *    section "Las optimizaciones en el prefill": 32-row blocks replaced
 *    16-row ones), H % 256 == 0 (H <= 4096), I % 128 == 0
 *    (I <= 4096), and T * top_k < 2^30 tokens x slots per call (pair
 *    indices are 32-bit).
 */
#ifndef MOE_INT4_H
#define MOE_INT4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_EINVAL (-1)       /* null or misaligned pointer, negative size, bad enum */
#define MOE_EUNSUPPORTED (-2) /* dims outside the supported set above         */
#define MOE_EWORKSPACE (-3)   /* workspace smaller than moe_workspace_bytes   */
#define MOE_EHIP (-4)         /* a HIP launch reported an error               */
#define MOE_EBUFFER (-5)      /* host output buffer too small (packers)       */
#define MOE_EFORMAT (-6)      /* int4 code outside 0..15                      */
#define MOE_ESCRATCH (-7)     /* request exceeds the library's static scratch  */

/* Layer dimensions: hidden size H, expert intermediate size I, routed experts
 * E, experts per token top_k, rows per routing block block_m, and which
 * grouped-GEMM kernels the prefill uses (gemm, one of MOE_GEMM_*):
 *   MOE_GEMM_EXACT  work items of block_m rows; the int4 codes enter the
 *                   matrix cores as exact bf16 values 128 + q and scale and
 *                   bias are applied per output and group in fp32 (weights
 *                   used exactly); suited to short chunks, where few rows
 *                   share an expert and the layer streams weights from HBM;
 *   MOE_GEMM_WIDE   work items of up to 144 rows of one expert; each weight
 *                   is expanded once per item to bf16 w = q*scale + bias
 *                   (fp32 value rounded once to bf16) and the matrix cores
 *                   accumulate x.w in fp32; suited to long chunks, where many
 *                   rows share each expanded weight;
 *   MOE_GEMM_AUTO   (0) WIDE for chunks whose pairs average at least 36 rows
 *                   per expert (top_k * T_chunk >= 36 * E), else EXACT.
 * (diariobitcoin.com, "Perplexity libera Lily...", section "Las
 * optimizaciones en el prefill": the grouped GEMM reconstructs the 4-bit
 * weights block by block on chip with fp32 accumulation.) Decode ignores
 * gemm. */
#define MOE_GEMM_AUTO 0
#define MOE_GEMM_EXACT 1
#define MOE_GEMM_WIDE 2
typedef struct {
  int32_t H, I, E, top_k, block_m, gemm;
} moe_dims;

/* Device weights of one layer. Every pointer is a device pointer. The blobs
 * must have been packed for the dims passed with them (E, H, I): their
 * headers are not read at call time, since that would need a device read
 * and a host synchronisation, so blobs of another shape give wrong results,
 * not an error code. The caller keeps them alive until the stream work that
 * uses them completes. */
typedef struct {
  const void* router_w3;       /* pack_router_bf16x3 blob of Wr (prefill router)     */
  const float* router_w;       /* [E][H] fp32 Wr, row-major (decode router)           */
  const float* router_bias;    /* [E] fp32 added to the logits, or NULL                */
  const void* experts_gate_up; /* pack_int4_g64 blob: E experts, gate and up paired   */
  const void* experts_down;    /* pack_int4_g64 blob: E experts, down                  */
  const void* shared_gate_up;  /* pack_int4_g64 blob: 1 expert, gate and up paired    */
  const void* shared_down;     /* pack_int4_g64 blob: 1 expert, down                   */
} moe_layer_weights;

/* Routing metadata (device buffers the caller provides). For T tokens:
 *   topk_idx [T][k] int32  selected experts, larger logit first, ties to the
 *                          lower expert index; slot j of token t is pair t*k+j
 *   topk_w   [T][k] fp32   softmax over all E logits restricted to the k
 *                          selected experts and renormalised to sum to one
 *   hist     [E]    int32  pairs routed to each expert (sums to k*T)
 *   offsets  [E+1]  int32  exclusive prefix sum of hist; offsets[E] = k*T
 *   perm     [k*T]  int32  perm[pos] = pair placed at row pos; the pairs of one
 *                          expert are contiguous, in ascending pair order
 *   inv_perm [k*T]  int32  inv_perm[pair] = pos
 *   block_map [moe_max_blocks(T)][3] int32  for each expert in ascending order,
 *                          ceil(hist[e]/block_m) entries (expert, first row,
 *                          rows in 1..block_m); entries past num_blocks are
 *                          not written
 *   num_blocks [1] int32
 * (diariobitcoin.com, "Perplexity libera Lily...", section "Las optimizaciones
 * en el prefill": histogram, prefix scan, scatter and block map; 32-row blocks.)
 */
typedef struct {
  int32_t* topk_idx;
  float* topk_w;
  int32_t* hist;
  int32_t* offsets;
  int32_t* perm;
  int32_t* inv_perm;
  int32_t* block_map;
  int32_t* num_blocks;
} moe_route_out;

/* Upper bound on the routing blocks of T tokens: ceil(k*T/block_m) + E.
 * Returns a negative code for invalid dims. */
int64_t moe_max_blocks(const moe_dims* dims, int32_t T);

/* Bytes of a pack_int4_g64 blob holding `count` experts of [N][K] matrices
 * (paired != 0: two matrices, gate and up, per expert). 0 if unsupported. */
size_t moe_packed_bytes(int32_t count, int32_t N, int32_t K, int32_t paired);

/* Pack affine int4 weights (host -> host) into the device layout the kernels
 * read. Logical input per matrix, row-major: q [count][N][K] uint8 in 0..15,
 * scale and bias [count][N][K/64] bf16 bits; weight w[n][c] =
 * q[n][c]*scale[n][c/64] + bias[n][c/64] (diariobitcoin.com, "Perplexity
 * libera Lily...", section "Qwen3.6 combina tres cargas de trabajo": 4-bit
 * affine, groups of 64, bf16 scale and bias). With q1/s1/b1 non-null the
 * expert holds two matrices of the same shape (gate = 0, up = 1) interleaved
 * in 32-row slices; with them null, one matrix. The blob is a 256-byte header
 * (magic "MI4G", version 1, count, N, K, paired) followed by one region per
 * expert; the layout is internal to this library and only read by it.
 * K % 64 == 0; N % 32 == 0 (paired) or N % 64 == 0. Returns MOE_EBUFFER if
 * out_bytes < moe_packed_bytes(...), MOE_EFORMAT if a code exceeds 15. */
int pack_int4_g64(const uint8_t* q0, const uint16_t* s0, const uint16_t* b0,
                  const uint8_t* q1, const uint16_t* s1, const uint16_t* b1,
                  int32_t count, int32_t N, int32_t K, void* out, size_t out_bytes);

/* Bytes of a pack_router_bf16x3 blob for an [E][H] router matrix. */
size_t moe_router_packed_bytes(int32_t E, int32_t H);

/* Pack the fp32 router matrix Wr [E][H] (host) into three bf16 planes with
 * Wr = hi + mid + lo exactly (each plane the next 8 significant bits), laid
 * out for the matrix cores (host -> host). E % 64 == 0, H % 64 == 0. */
int pack_router_bf16x3(const float* wr, int32_t E, int32_t H, void* out, size_t out_bytes);

/* Workspace bytes for a call. mode 0: moe_prefill_layer with chunks of at
 * most T_chunk tokens; mode 1: moe_decode_layer with up to T_chunk (<= 4)
 * tokens; mode 2: moe_route of up to T_chunk tokens. */
int moe_workspace_bytes(const moe_dims* dims, int32_t T_chunk, int32_t mode, size_t* bytes);

/* Routing only: from fp32 logits [T][E] (device) fill every field of `out`
 * (device buffers sized for T) on `stream`. T = 0 is a no-op. */
int moe_route(const moe_dims* dims, const float* logits, int32_t T, const moe_route_out* out,
              void* ws, size_t ws_bytes, void* stream);

/* The prefill MoE layer: y [T][H] bf16 = shared(x) + sum_j topk_w * expert(x)
 * for x [T][H] bf16 (both device). Tokens are processed in consecutive chunks
 * of at most chunk_T tokens (chunk_T <= 0: one chunk) reusing one workspace
 * (diariobitcoin.com, "Perplexity libera Lily...", section "Las optimizaciones
 * en el prefill": long prompts run in bounded chunks). logits_out (device
 * [T][E] fp32) receives the router logits when non-null. route_out, when
 * non-null, receives the routing metadata of the LAST chunk (sized for that
 * chunk's token count). Numerics: fp32 router logits; int4 weights expanded
 * on chip as dims->gemm states (exact codes with fp32 scale and bias, or
 * bf16 weights rounded once); fp32 accumulation;
 * the SwiGLU product h is rounded to bf16 before the down projection; each
 * of the k routed down outputs is rounded to bf16 (it enters with a routing
 * weight of about 1/k), the shared expert's stays fp32, and they are summed
 * in fp32 in a fixed order; y is rounded once to bf16. T = 0 is a no-op. */
int moe_prefill_layer(const moe_dims* dims, const moe_layer_weights* w, const uint16_t* x,
                      uint16_t* y, int32_t T, int32_t chunk_T, float* logits_out,
                      const moe_route_out* route_out, void* ws, size_t ws_bytes, void* stream);

/* The same layer for 1 <= T <= 4 tokens (decode), organised as matrix-vector
 * passes over only the selected experts' packed weights (diariobitcoin.com,
 * "Perplexity libera Lily...", section "El decode busca mover menos datos":
 * batch-1 decode is bandwidth bound). logits_out / route_out as above
 * (route_out: topk_idx, topk_w, hist, offsets, perm, inv_perm, block_map and
 * num_blocks are all filled). */
int moe_decode_layer(const moe_dims* dims, const moe_layer_weights* w, const uint16_t* x,
                     uint16_t* y, int32_t T, float* logits_out, const moe_route_out* route_out,
                     void* ws, size_t ws_bytes, void* stream);

/* moe_decode_layer for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments and results as moe_decode_layer without the workspace: the
 * decode kernels' scratch (router logits, top-k, SwiGLU rows) lives in a
 * static device array of MOE_NOALLOC_SCRATCH_BYTES bytes inside the library,
 * one copy per GPU, held until the process ends. The call allocates and
 * frees nothing (its first call on a device resolves that device's array
 * address once with hipGetSymbolAddress; make that first call outside graph
 * capture). Nothing in the array needs to start at zero: every call writes
 * what it reads. Calls that overlap on one GPU (several streams, or several
 * host threads) share the array and race: serialise them. Returns
 * MOE_ESCRATCH if the request needs more scratch than the array holds (the
 * supported dims with T <= 4 need at most 299,520 bytes), otherwise the
 * codes of moe_decode_layer (MOE_EHIP also if the array's address cannot be
 * resolved). */
#define MOE_NOALLOC_SCRATCH_BYTES (320 * 1024)
int moe_decode_layer_noalloc(const moe_dims* dims, const moe_layer_weights* w, const uint16_t* x,
                             uint16_t* y, int32_t T, float* logits_out,
                             const moe_route_out* route_out, void* stream);

/* The prefill layer with host-synchronised routing, for measuring what
 * GPU-resident routing saves (diariobitcoin.com, "Perplexity libera Lily...",
 * section "Las optimizaciones en el prefill": keeping histogram, scan,
 * scatter and block map on the GPU, with no CPU round trip, sped prefill
 * up). Same arguments and results as moe_prefill_layer (no logits or
 * metadata outputs), but per chunk the calling thread waits for the routing
 * kernels, reads the work-item count back (4 bytes, device -> host) and
 * launches the grouped GEMMs with grids of exactly one block per work unit
 * instead of the persistent grids. It synchronises the host once per chunk,
 * so it cannot be captured in a graph. */
int moe_prefill_layer_host_routed(const moe_dims* dims, const moe_layer_weights* w,
                                  const uint16_t* x, uint16_t* y, int32_t T, int32_t chunk_T,
                                  void* ws, size_t ws_bytes, void* stream);

/* The prefill layer without fused dequantisation, for measuring what the
 * fusion saves (diariobitcoin.com, "Perplexity libera Lily...", section "Las
 * optimizaciones en el prefill": reconstructing the weights inside the
 * grouped GEMM, never writing them back, sped prefill up). Per chunk, after
 * the routing, every expert with rows and the shared expert are expanded to
 * bf16 w = q*s + b (one rounding) into wbuf (device, caller-owned,
 * moe_unfused_weight_bytes bytes), then the grouped GEMMs read those bf16
 * weights. Same results as moe_prefill_layer up to the bf16 rounding of the
 * weights (no logits or metadata outputs). MOE_EBUFFER if wbuf is too
 * small. */
int moe_unfused_weight_bytes(const moe_dims* dims, size_t* bytes);
int moe_prefill_layer_unfused(const moe_dims* dims, const moe_layer_weights* w, const uint16_t* x,
                              uint16_t* y, int32_t T, int32_t chunk_T, void* wbuf, size_t wbuf_bytes,
                              void* ws, size_t ws_bytes, void* stream);

/* Timing variants for benchmarks: identical to moe_prefill_layer /
 * moe_decode_layer, and in addition record the caller's events (hipEvent_t
 * handles created by the caller) on `stream`: events[i] just before the i-th
 * kernel launch and one more after the last launch, so consecutive events
 * bracket one kernel each. Prefill launches 6 kernels per chunk (router,
 * top-k, scan/scatter, gate/up, down, combine) and needs
 * n_events >= 6 * chunks + 1; decode launches 3 (router, top-k + gate/up,
 * down + combine) and needs n_events >= 4. MOE_EINVAL if too few events. */
int moe_prefill_layer_profiled(const moe_dims* dims, const moe_layer_weights* w,
                               const uint16_t* x, uint16_t* y, int32_t T, int32_t chunk_T,
                               float* logits_out, const moe_route_out* route_out, void* ws,
                               size_t ws_bytes, void* stream, void* const* events,
                               int32_t n_events);
int moe_decode_layer_profiled(const moe_dims* dims, const moe_layer_weights* w, const uint16_t* x,
                              uint16_t* y, int32_t T, float* logits_out,
                              const moe_route_out* route_out, void* ws, size_t ws_bytes,
                              void* stream, void* const* events, int32_t n_events);

/* Static description of an error code. */
const char* moe_strerror(int code);

/* Test hook: expand expert `expert` of a pack_int4_g64 blob (device) on the
 * GPU with the same load-and-convert code the GEMM kernels use, writing fp32
 * w[n][c] = q*scale + bias to out (device) as [N][K] (paired: [2][N][K], gate
 * then up). */
int moe_test_dequant(const void* blob, int32_t count, int32_t N, int32_t K, int32_t paired,
                     int32_t expert, float* out, void* stream);

/* Measurement helpers, not part of the layer: achievable ceilings of the
 * device, for roofline fractions against measured as well as published peaks.
 *
 * moe_ceiling_read enqueues one streaming read of `bytes` (a multiple of 16,
 * >= 16) of device memory at `buf` by 2048 blocks of 256 threads, each block
 * one contiguous 1/2048 of the buffer (16-byte vector loads, eight in flight
 * per thread). `sink` (device, 4 bytes) is
 * written only if the XOR of a thread's data equals a fixed constant, which
 * keeps the loads live; callers ignore its value. Time it with events; for
 * HBM bandwidth use a buffer much larger than the 256 MB last-level cache.
 *
 * moe_ceiling_mfma enqueues 1024 blocks of four waves, each wave running
 * eight independent chains of 4 * `iters` (iters > 0) 16x16x32 bf16
 * matrix-core operations on register operands, and stores the flop count of
 * the launch in *flops (host). `random` nonzero: the operands are random bf16
 * values (magnitude in [0.5, 1), random sign) that change from one operation
 * to the next, as layer data does; zero: nearly constant operands. The
 * device sustains a lower clock on the first. `clocks` (device, may be null):
 * 2048 unsigned 64-bit values that receive, per block, the real-time ticks
 * (100 MHz) and the shader-clock ticks over its loop; their sums give the
 * clock the launch ran at. `sink` as above.
 *
 * Both return MOE_EINVAL for null pointers or bad sizes, MOE_EHIP if the
 * launch fails; they allocate nothing and do not synchronise. */
int moe_ceiling_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);
int moe_ceiling_mfma(int32_t iters, int32_t random, float* sink, unsigned long long* clocks,
                     double* flops, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_INT4_H */
