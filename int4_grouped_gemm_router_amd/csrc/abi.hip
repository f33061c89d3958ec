// C ABI of the int4 MoE library: argument checks, workspace carve-up, the
// chunk loop, and the launches on the caller's stream (include/moe_int4.h).
#include <algorithm>
#include <atomic>
#include <cstdint>

#include "../../include/moe_int4.h"
#include "kernels.h"

using namespace moe;

namespace {

bool dims_ok(const moe_dims* d) {
  return d && d->E > 0 && d->E <= 256 && d->E % 64 == 0 && d->top_k == 8 && (d->block_m == 32 || d->block_m == 16) &&
         d->H > 0 && d->H % 256 == 0 && d->H <= 4096 && d->I > 0 && d->I % 128 == 0 &&
         d->I <= 4096 && d->gemm >= MOE_GEMM_AUTO && d->gemm <= MOE_GEMM_WIDE;
}

// Wide GEMMs (items of up to kWideRows rows, bf16 weights expanded once per
// item) when the chunk's pairs average at least kWideMinRows rows per expert:
// then enough rows share each expanded weight for the matrix cores to set
// the pace; below it the layer streams weights and the exact kernels' short
// items spread them over more compute units.
constexpr int kWideMinRows = 36;  // the measured crossover lies between 32 and 36 (E = 256)
bool use_wide(const moe_dims* d, int Tn) {
  if (d->gemm == MOE_GEMM_EXACT) return false;
  if (d->gemm == MOE_GEMM_WIDE) return true;
  return (int64_t)d->top_k * Tn >= (int64_t)kWideMinRows * d->E;
}

int64_t max_blocks(const moe_dims* d, int T) {
  return ((int64_t)d->top_k * T + d->block_m - 1) / d->block_m + d->E;
}

int max_items(const moe_dims* d, int T) {
  return (int)(((int64_t)d->top_k * T + d->block_m - 1) / d->block_m + d->E);
}

int n_chunks(const moe_dims* d, int T) {
  return (int)(((int64_t)d->top_k * T + kChunkPairs - 1) / kChunkPairs);
}

// Split the router's K dimension into the largest power of two <= kMaxSplits
// that divides K / 64, whatever T is: the blocks stay short (each holds a
// 72 KB LDS ring, so at most two run on a compute unit) and every logit is
// the same fixed-order sum of the same partial sums for any chunking of the
// tokens, so chunked and unchunked prompts get identical logits.
int router_splits(const moe_dims* d, int /*T*/) {
  const int G = d->H / kGroup;
  int s = kMaxSplits;
  while (G % s) s /= 2;
  return s;
}

// Bump allocator over the caller's workspace (256-byte aligned pieces).
struct Carve {
  uint8_t* base;
  size_t used = 0;
  template <class P>
  P* take(size_t count) {
    P* p = base ? reinterpret_cast<P*>(base + used) : nullptr;
    used += (count * sizeof(P) + 255) / 256 * 256;
    return p;
  }
};

struct PrefillWs {
  float* logit_partial;
  int32_t *topk_idx, *chunk_hist, *hist, *offsets, *perm, *inv_perm, *block_map, *num_blocks;
  int32_t *items, *num_items;
  float* topk_w;
  uint16_t* h;  // [(k+1)Tc][I]
  uint16_t* partial_r;  // routed down rows, bf16 [k*Tc][H]
  float* partial_s;     // shared-expert down rows, fp32 [Tc][H]
};

PrefillWs carve_prefill(const moe_dims* d, int Tc, void* ws, size_t* bytes) {
  Carve c{static_cast<uint8_t*>(ws)};
  PrefillWs w;
  size_t logit_elems = 0;
  for (int T = 1; T <= Tc; ++T)
    logit_elems = std::max(logit_elems, (size_t)router_splits(d, T) * T * d->E);
  const int k = d->top_k;
  w.logit_partial = c.take<float>(logit_elems);
  w.topk_idx = c.take<int32_t>((size_t)k * Tc);
  w.topk_w = c.take<float>((size_t)k * Tc);
  w.chunk_hist = c.take<int32_t>((size_t)n_chunks(d, Tc) * d->E);
  w.hist = c.take<int32_t>(d->E);
  w.offsets = c.take<int32_t>(d->E + 1);
  w.perm = c.take<int32_t>((size_t)k * Tc);
  w.inv_perm = c.take<int32_t>((size_t)k * Tc);
  w.block_map = c.take<int32_t>(3 * (size_t)max_blocks(d, Tc));
  w.num_blocks = c.take<int32_t>(1);
  w.items = c.take<int32_t>(3 * (size_t)max_items(d, Tc));
  w.num_items = c.take<int32_t>(1);
  w.h = c.take<uint16_t>((size_t)(k + 1) * Tc * d->I);
  w.partial_r = c.take<uint16_t>((size_t)k * Tc * d->H);
  w.partial_s = c.take<float>((size_t)Tc * d->H);
  *bytes = c.used;
  return w;
}

struct DecodeWs {
  float *logits, *topk_w;
  int32_t* topk_idx;
  uint16_t* h;
};

DecodeWs carve_decode(const moe_dims* d, int T, void* ws, size_t* bytes) {
  Carve c{static_cast<uint8_t*>(ws)};
  DecodeWs w;
  const int k = d->top_k;
  w.logits = c.take<float>((size_t)T * d->E);
  w.topk_idx = c.take<int32_t>((size_t)k * T);
  w.topk_w = c.take<float>((size_t)k * T);
  w.h = c.take<uint16_t>((size_t)(k + 1) * T * d->I);
  *bytes = c.used;
  return w;
}

size_t route_ws(const moe_dims* d, int T, void* ws, int32_t** chunk_hist) {
  Carve c{static_cast<uint8_t*>(ws)};
  *chunk_hist = c.take<int32_t>((size_t)n_chunks(d, T) * d->E);
  return c.used;
}

// The kernels move activations, outputs, workspace pieces and packed weights
// in 16-byte vectors and everything else in 4-byte words; a misaligned
// pointer is rejected before anything is enqueued (null passes: null checks
// are separate).
bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
bool al4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; }

// (token, slot) pair indices are 32-bit in the kernels
constexpr int64_t kMaxPairs = int64_t(1) << 30;
bool too_many_pairs(const moe_dims* d, int64_t T) { return T * d->top_k >= kMaxPairs; }

bool route_out_ok(const moe_route_out* o) {
  return o && o->topk_idx && o->topk_w && o->hist && o->offsets && o->perm && o->inv_perm &&
         o->block_map && o->num_blocks && al4(o->topk_idx) && al4(o->topk_w) && al4(o->hist) &&
         al4(o->offsets) && al4(o->perm) && al4(o->inv_perm) && al4(o->block_map) &&
         al4(o->num_blocks);
}

bool weights_aligned(const moe_layer_weights* w) {
  return al16(w->router_w3) && al16(w->router_w) && al4(w->router_bias) && al16(w->experts_gate_up) &&
         al16(w->experts_down) && al16(w->shared_gate_up) && al16(w->shared_down);
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

// Optional timing hook: records events[i] before the i-th kernel launch and
// one more after the last launch.
struct Recorder {
  hipEvent_t* ev = nullptr;
  int n = 0, used = 0;
  hipError_t mark(hipStream_t s) {
    if (!ev) return hipSuccess;
    if (used >= n) return hipErrorInvalidValue;
    return hipEventRecord(ev[used++], s);
  }
};

constexpr int kPrefillLaunchesPerChunk = 6;
constexpr int kDecodeLaunches = 3;

int prefill_impl(const moe_dims* dims, const moe_layer_weights* w, const uint16_t* x, uint16_t* y,
                 int32_t T, int32_t chunk_T, float* logits_out, const moe_route_out* route_out,
                 void* ws, size_t ws_bytes, void* stream, Recorder rec, bool host_routed = false,
                 uint8_t* unfused_w = nullptr);
int decode_impl(const moe_dims* dims, const moe_layer_weights* w, const uint16_t* x, uint16_t* y,
                int32_t T, float* logits_out, const moe_route_out* route_out, void* ws,
                size_t ws_bytes, void* stream, hipEvent_t* ev);
int decode_args(const moe_dims* dims, const moe_layer_weights* w, const uint16_t* x, uint16_t* y,
                int32_t T, float* logits_out, const moe_route_out* route_out);

}  // namespace

extern "C" {

int64_t moe_max_blocks(const moe_dims* dims, int32_t T) {
  if (!dims_ok(dims)) return MOE_EUNSUPPORTED;
  if (T < 0) return MOE_EINVAL;
  return max_blocks(dims, T);
}

int moe_workspace_bytes(const moe_dims* dims, int32_t T_chunk, int32_t mode, size_t* bytes) {
  if (!bytes || T_chunk < 0) return MOE_EINVAL;
  if (!dims_ok(dims) || too_many_pairs(dims, T_chunk)) return MOE_EUNSUPPORTED;
  const int T = std::max(T_chunk, 1);
  if (mode == 0) {
    carve_prefill(dims, T, nullptr, bytes);
  } else if (mode == 1) {
    if (T > kDecodeMaxT) return MOE_EUNSUPPORTED;
    carve_decode(dims, T, nullptr, bytes);
  } else if (mode == 2) {
    int32_t* ch;
    *bytes = route_ws(dims, T, nullptr, &ch);
  } else {
    return MOE_EINVAL;
  }
  return MOE_OK;
}

int moe_route(const moe_dims* dims, const float* logits, int32_t T, const moe_route_out* out,
              void* ws, size_t ws_bytes, void* stream) {
  if (!dims || T < 0) return MOE_EINVAL;
  if (!dims_ok(dims) || too_many_pairs(dims, T)) return MOE_EUNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!logits || !route_out_ok(out) || !ws || !al4(logits) || !al16(ws)) return MOE_EINVAL;
  int32_t* chunk_hist;
  if (ws_bytes < route_ws(dims, T, nullptr, &chunk_hist)) return MOE_EWORKSPACE;
  route_ws(dims, T, ws, &chunk_hist);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (launch_fill_zero(chunk_hist, n_chunks(dims, T) * dims->E, s) != hipSuccess) return MOE_EHIP;
  TopkArgs ta{};
  ta.partial = logits;
  ta.splits = 1;
  ta.topk_idx = out->topk_idx;
  ta.topk_w = out->topk_w;
  ta.chunk_hist = chunk_hist;
  ta.T = T;
  ta.E = dims->E;
  ta.k = dims->top_k;
  if (launch_topk(ta, s) != hipSuccess) return MOE_EHIP;
  ScatterArgs sa{};
  sa.topk_idx = out->topk_idx;
  sa.chunk_hist = chunk_hist;
  sa.hist = out->hist;
  sa.offsets = out->offsets;
  sa.perm = out->perm;
  sa.inv_perm = out->inv_perm;
  sa.block_map = out->block_map;
  sa.num_blocks = out->num_blocks;
  sa.T = T;
  sa.E = dims->E;
  sa.k = dims->top_k;
  sa.block_m = dims->block_m;
  return hip_status(launch_scan_scatter(sa, s));
}

int moe_prefill_layer(const moe_dims* dims, const moe_layer_weights* w, const uint16_t* x,
                      uint16_t* y, int32_t T, int32_t chunk_T, float* logits_out,
                      const moe_route_out* route_out, void* ws, size_t ws_bytes, void* stream) {
  return prefill_impl(dims, w, x, y, T, chunk_T, logits_out, route_out, ws, ws_bytes, stream,
                      Recorder{});
}

int moe_prefill_layer_host_routed(const moe_dims* dims, const moe_layer_weights* w,
                                  const uint16_t* x, uint16_t* y, int32_t T, int32_t chunk_T,
                                  void* ws, size_t ws_bytes, void* stream) {
  return prefill_impl(dims, w, x, y, T, chunk_T, nullptr, nullptr, ws, ws_bytes, stream,
                      Recorder{}, true);
}

int moe_unfused_weight_bytes(const moe_dims* dims, size_t* bytes) {
  if (!bytes) return MOE_EINVAL;
  if (!dims_ok(dims)) return MOE_EUNSUPPORTED;
  const PackGeom gu = pack_geom(dims->I, dims->H, 1), dn = pack_geom(dims->H, dims->I, 0);
  *bytes = (size_t)(dims->E + 1) *
           ((size_t)gu.n_wt * gu.G + (size_t)dn.n_wt * dn.G) * kBf16GroupBytes;
  return MOE_OK;
}

int moe_prefill_layer_unfused(const moe_dims* dims, const moe_layer_weights* w, const uint16_t* x,
                              uint16_t* y, int32_t T, int32_t chunk_T, void* wbuf, size_t wbuf_bytes,
                              void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  const int rc = moe_unfused_weight_bytes(dims, &need);
  if (rc != MOE_OK) return rc;
  if (!wbuf || !al16(wbuf)) return MOE_EINVAL;
  if (wbuf_bytes < need) return MOE_EBUFFER;
  return prefill_impl(dims, w, x, y, T, chunk_T, nullptr, nullptr, ws, ws_bytes, stream,
                      Recorder{}, false, static_cast<uint8_t*>(wbuf));
}

int moe_prefill_layer_profiled(const moe_dims* dims, const moe_layer_weights* w,
                               const uint16_t* x, uint16_t* y, int32_t T, int32_t chunk_T,
                               float* logits_out, const moe_route_out* route_out, void* ws,
                               size_t ws_bytes, void* stream, void* const* events,
                               int32_t n_events) {
  if (!events || n_events < 0 || !dims || T < 0) return MOE_EINVAL;
  if (T > 0) {
    const int Tc = (chunk_T <= 0 || chunk_T > T) ? T : chunk_T;
    const int chunks = (T + Tc - 1) / Tc;
    if (n_events < kPrefillLaunchesPerChunk * chunks + 1) return MOE_EINVAL;
  }
  Recorder r;
  r.ev = reinterpret_cast<hipEvent_t*>(const_cast<void**>(events));
  r.n = n_events;
  return prefill_impl(dims, w, x, y, T, chunk_T, logits_out, route_out, ws, ws_bytes, stream, r);
}

}  // extern "C"

namespace {

int prefill_impl(const moe_dims* dims, const moe_layer_weights* w, const uint16_t* x, uint16_t* y,
                 int32_t T, int32_t chunk_T, float* logits_out, const moe_route_out* route_out,
                 void* ws, size_t ws_bytes, void* stream, Recorder rec, bool host_routed,
                 uint8_t* unfused_w) {
  if (!dims || T < 0) return MOE_EINVAL;
  if (!dims_ok(dims) || too_many_pairs(dims, T)) return MOE_EUNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!w || !x || !y || !ws || !w->router_w3 || !w->experts_gate_up || !w->experts_down ||
      !w->shared_gate_up || !w->shared_down)
    return MOE_EINVAL;
  if (route_out && !route_out_ok(route_out)) return MOE_EINVAL;
  if (!al16(x) || !al16(y) || !al16(ws) || !al4(logits_out) || !weights_aligned(w)) return MOE_EINVAL;
  const int Tc = (chunk_T <= 0 || chunk_T > T) ? T : chunk_T;
  size_t need;
  carve_prefill(dims, Tc, nullptr, &need);
  if (ws_bytes < need) return MOE_EWORKSPACE;
  const PrefillWs W = carve_prefill(dims, Tc, ws, &need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int H = dims->H, I = dims->I, E = dims->E, k = dims->top_k;
  const PackGeom gu = pack_geom(I, H, 1), dn = pack_geom(H, I, 0);
  const uint8_t* planes = static_cast<const uint8_t*>(w->router_w3) + kHeaderBytes;

  for (int t0 = 0; t0 < T; t0 += Tc) {
    const int Tn = std::min(Tc, T - t0);
    const bool last = t0 + Tc >= T;
    const moe_route_out* ro = (last && route_out) ? route_out : nullptr;
    int32_t* topk_idx = ro ? ro->topk_idx : W.topk_idx;
    float* topk_w = ro ? ro->topk_w : W.topk_w;
    const uint16_t* xc = x + (int64_t)t0 * H;
    const int splits = router_splits(dims, Tn);
    const int nch = n_chunks(dims, Tn);

    if (rec.mark(s) != hipSuccess) return MOE_EHIP;
    if (launch_router(xc, reinterpret_cast<const uint16_t*>(planes), W.logit_partial, Tn, H, E,
                      splits, W.chunk_hist, nch * E, s) != hipSuccess)
      return MOE_EHIP;
    TopkArgs ta{};
    ta.partial = W.logit_partial;
    ta.splits = splits;
    ta.rbias = w->router_bias;
    ta.logits_out = logits_out ? logits_out + (int64_t)t0 * E : nullptr;
    ta.topk_idx = topk_idx;
    ta.topk_w = topk_w;
    ta.chunk_hist = W.chunk_hist;
    ta.T = Tn;
    ta.E = E;
    ta.k = k;
    if (rec.mark(s) != hipSuccess) return MOE_EHIP;
    if (launch_topk(ta, s) != hipSuccess) return MOE_EHIP;

    ScatterArgs sa{};
    sa.topk_idx = topk_idx;
    sa.chunk_hist = W.chunk_hist;
    sa.hist = ro ? ro->hist : W.hist;
    sa.offsets = ro ? ro->offsets : W.offsets;
    sa.perm = ro ? ro->perm : W.perm;
    sa.inv_perm = ro ? ro->inv_perm : W.inv_perm;
    sa.block_map = ro ? ro->block_map : W.block_map;
    sa.num_blocks = ro ? ro->num_blocks : W.num_blocks;
    sa.items = W.items;
    sa.num_items = W.num_items;
    sa.T = Tn;
    sa.E = E;
    sa.k = k;
    sa.block_m = dims->block_m;
    // GEMM work items: one per routing block (exact kernels), or up to
    // kWideRows rows of one expert (wide kernels; not for the unfused path)
    const bool wide = !unfused_w && use_wide(dims, Tn);
    const int item_rows = wide ? kWideRows : dims->block_m;
    sa.item_rows = item_rows;
    sa.longest_first = wide ? 1 : 0;
    if (rec.mark(s) != hipSuccess) return MOE_EHIP;
    if (launch_scan_scatter(sa, s) != hipSuccess) return MOE_EHIP;

    const int shared_slots = (Tn + item_rows - 1) / item_rows;
    // work-list slots the wide grids cover (an upper bound on the device's count)
    int wide_slots = max_items(dims, Tn) + shared_slots;
    // host-routed variant: the host waits for the routing, reads the work
    // item count and launches exact grids (one block per 256-column unit)
    int gu_blocks = 0, dn_blocks = 0;
    if (host_routed) {
      int32_t ni = 0;
      if (hipMemcpyAsync(&ni, W.num_items, sizeof ni, hipMemcpyDeviceToHost, s) != hipSuccess ||
          hipStreamSynchronize(s) != hipSuccess)
        return MOE_EHIP;
      const int slots = ni + shared_slots;
      gu_blocks = std::max(1, slots * ((gu.n_wt + 3) / 4));
      dn_blocks = std::max(1, slots * ((dn.n_wt + 3) / 4));
      wide_slots = slots;
    }

    GemmArgs g{};
    g.items = W.items;
    g.num_items = W.num_items;
    g.item_rows = item_rows;
    g.shared_slots = shared_slots;
    g.T = Tn;
    g.k = k;
    g.perm = sa.perm;

    // unfused comparison path: the touched experts' weights expanded to bf16
    // in memory first, then the same GEMMs on the bf16 weights
    const int64_t gu_bf = (int64_t)gu.n_wt * gu.G * kBf16GroupBytes;
    const int64_t dn_bf = (int64_t)dn.n_wt * dn.G * kBf16GroupBytes;
    uint8_t* gu_w = unfused_w;
    uint8_t* gu_sh = unfused_w ? gu_w + E * gu_bf : nullptr;
    uint8_t* dn_w = unfused_w ? gu_sh + gu_bf : nullptr;
    uint8_t* dn_sh = unfused_w ? dn_w + E * dn_bf : nullptr;
    g.bf16_weights = unfused_w ? 1 : 0;

    // gate/up + SwiGLU (routed and shared items in one launch)
    g.blob = static_cast<const uint8_t*>(w->experts_gate_up) + kHeaderBytes;
    g.shared_blob = static_cast<const uint8_t*>(w->shared_gate_up) + kHeaderBytes;
    g.expert_bytes = gu.expert_bytes;
    if (unfused_w) {
      if (launch_expand_bf16(g.blob, gu.expert_bytes, g.shared_blob, E, sa.hist, I, H, 1, gu_w, gu_sh,
                             s) != hipSuccess)
        return MOE_EHIP;
      g.blob = gu_w;
      g.shared_blob = gu_sh;
      g.expert_bytes = gu_bf;
    }
    g.N = I;
    g.K = H;
    g.paired = 1;
    g.act = xc;
    g.h_out = W.h;
    if (rec.mark(s) != hipSuccess) return MOE_EHIP;
    if ((wide ? launch_gemm_wide(kGateUp, g, wide_slots, s) : launch_gemm(kGateUp, g, s, gu_blocks)) !=
        hipSuccess)
      return MOE_EHIP;

    // down: routed items (one output row per pair) and shared items in one launch
    g.blob = static_cast<const uint8_t*>(w->experts_down) + kHeaderBytes;
    g.shared_blob = static_cast<const uint8_t*>(w->shared_down) + kHeaderBytes;
    g.expert_bytes = dn.expert_bytes;
    if (unfused_w) {
      if (launch_expand_bf16(g.blob, dn.expert_bytes, g.shared_blob, E, sa.hist, H, I, 0, dn_w, dn_sh,
                             s) != hipSuccess)
        return MOE_EHIP;
      g.blob = dn_w;
      g.shared_blob = dn_sh;
      g.expert_bytes = dn_bf;
    }
    g.N = H;
    g.K = I;
    g.paired = 0;
    g.act = W.h;
    g.h_out = nullptr;
    g.partial_r = W.partial_r;
    g.partial_s = W.partial_s;
    if (rec.mark(s) != hipSuccess) return MOE_EHIP;
    if ((wide ? launch_gemm_wide(kDown, g, wide_slots, s) : launch_gemm(kDown, g, s, dn_blocks)) !=
        hipSuccess)
      return MOE_EHIP;

    // y = bf16(shared + sum of the k weighted expert outputs)
    if (rec.mark(s) != hipSuccess) return MOE_EHIP;
    if (launch_combine(W.partial_r, W.partial_s, topk_w, y + (int64_t)t0 * H, Tn, H, k, s) != hipSuccess)
      return MOE_EHIP;
  }
  if (rec.mark(s) != hipSuccess) return MOE_EHIP;
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_decode_layer(const moe_dims* dims, const moe_layer_weights* w, const uint16_t* x,
                     uint16_t* y, int32_t T, float* logits_out, const moe_route_out* route_out,
                     void* ws, size_t ws_bytes, void* stream) {
  return decode_impl(dims, w, x, y, T, logits_out, route_out, ws, ws_bytes, stream, nullptr);
}

int moe_decode_layer_profiled(const moe_dims* dims, const moe_layer_weights* w, const uint16_t* x,
                              uint16_t* y, int32_t T, float* logits_out,
                              const moe_route_out* route_out, void* ws, size_t ws_bytes,
                              void* stream, void* const* events, int32_t n_events) {
  if (!events || n_events < kDecodeLaunches + 1) return MOE_EINVAL;
  return decode_impl(dims, w, x, y, T, logits_out, route_out, ws, ws_bytes, stream,
                     reinterpret_cast<hipEvent_t*>(const_cast<void**>(events)));
}

}  // extern "C"

namespace {

// Checks of the decode arguments other than the workspace (MOE_OK: valid,
// T > 0).
int decode_args(const moe_dims* dims, const moe_layer_weights* w, const uint16_t* x, uint16_t* y,
                int32_t T, float* logits_out, const moe_route_out* route_out) {
  if (!dims || T < 0) return MOE_EINVAL;
  if (!dims_ok(dims) || T > kDecodeMaxT) return MOE_EUNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!w || !x || !y || !w->router_w || !w->experts_gate_up || !w->experts_down ||
      !w->shared_gate_up || !w->shared_down)
    return MOE_EINVAL;
  if (route_out && !route_out_ok(route_out)) return MOE_EINVAL;
  if (!al16(x) || !al16(y) || !al4(logits_out) || !weights_aligned(w)) return MOE_EINVAL;
  return MOE_OK;
}

int decode_impl(const moe_dims* dims, const moe_layer_weights* w, const uint16_t* x, uint16_t* y,
                int32_t T, float* logits_out, const moe_route_out* route_out, void* ws,
                size_t ws_bytes, void* stream, hipEvent_t* ev) {
  const int rc = decode_args(dims, w, x, y, T, logits_out, route_out);
  if (rc != MOE_OK || T == 0) return rc;
  if (!ws || !al16(ws)) return MOE_EINVAL;
  size_t need;
  carve_decode(dims, T, nullptr, &need);
  if (ws_bytes < need) return MOE_EWORKSPACE;
  const DecodeWs W = carve_decode(dims, T, ws, &need);
  const PackGeom gu = pack_geom(dims->I, dims->H, 1), dn = pack_geom(dims->H, dims->I, 0);
  DecodeArgs a{};
  a.x = x;
  a.router_w = w->router_w;
  a.rbias = w->router_bias;
  a.logits = W.logits;
  a.logits_out = logits_out;
  a.topk_idx = route_out ? route_out->topk_idx : W.topk_idx;
  a.topk_w = route_out ? route_out->topk_w : W.topk_w;
  if (route_out) {
    a.hist = route_out->hist;
    a.offsets = route_out->offsets;
    a.perm = route_out->perm;
    a.inv_perm = route_out->inv_perm;
    a.block_map = route_out->block_map;
    a.num_blocks = route_out->num_blocks;
  }
  a.gu_blob = static_cast<const uint8_t*>(w->experts_gate_up) + kHeaderBytes;
  a.gu_shared = static_cast<const uint8_t*>(w->shared_gate_up) + kHeaderBytes;
  a.gu_expert_bytes = gu.expert_bytes;
  a.dn_blob = static_cast<const uint8_t*>(w->experts_down) + kHeaderBytes;
  a.dn_shared = static_cast<const uint8_t*>(w->shared_down) + kHeaderBytes;
  a.dn_expert_bytes = dn.expert_bytes;
  a.h = W.h;
  a.y = y;
  a.T = T;
  a.H = dims->H;
  a.I = dims->I;
  a.E = dims->E;
  a.k = dims->top_k;
  a.block_m = dims->block_m;
  return hip_status(launch_decode(a, static_cast<hipStream_t>(stream), ev));
}

}  // namespace

// Scratch of moe_decode_layer_noalloc: a file-scope device array, one copy
// per GPU. Host code never passes `scratch` itself to a kernel (on the host
// it names a stand-in, not a device address); it uses the per-device address
// from hipGetSymbolAddress below.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on the current device, resolved once per device
// with that device current. Concurrent first calls may both resolve it and
// store the same value. Null if the address cannot be resolved.
void* scratch_address() {
  static std::atomic<void*> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  void* p = cached[dev].load(std::memory_order_acquire);
  if (!p) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
    cached[dev].store(q, std::memory_order_release);
    p = q;
  }
  return p;
}

}  // namespace

extern "C" {

int moe_decode_layer_noalloc(const moe_dims* dims, const moe_layer_weights* w, const uint16_t* x,
                             uint16_t* y, int32_t T, float* logits_out,
                             const moe_route_out* route_out, void* stream) {
  const int rc = decode_args(dims, w, x, y, T, logits_out, route_out);
  if (rc != MOE_OK || T == 0) return rc;
  size_t need = 0;
  carve_decode(dims, T, nullptr, &need);
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ESCRATCH;
  void* ws = scratch_address();
  if (!ws) return MOE_EHIP;
  return decode_impl(dims, w, x, y, T, logits_out, route_out, ws, MOE_NOALLOC_SCRATCH_BYTES, stream,
                     nullptr);
}

const char* moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (null pointer, negative size or bad mode)";
    case MOE_EUNSUPPORTED: return "unsupported dimensions";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_EHIP: return "HIP launch error";
    case MOE_EBUFFER: return "output buffer too small";
    case MOE_EFORMAT: return "int4 code outside 0..15";
    case MOE_ESCRATCH: return "request exceeds the static scratch of the no-allocation entry point";
    default: return "unknown error";
  }
}

int moe_test_dequant(const void* blob, int32_t count, int32_t N, int32_t K, int32_t paired,
                     int32_t expert, float* out, void* stream) {
  if (!blob || !out || expert < 0 || expert >= count || !al16(blob) || !al4(out)) return MOE_EINVAL;
  if (moe_packed_bytes(count, N, K, paired) == 0) return MOE_EUNSUPPORTED;
  const PackGeom g = pack_geom(N, K, paired);
  const uint8_t* base = static_cast<const uint8_t*>(blob) + kHeaderBytes + (int64_t)expert * g.expert_bytes;
  return hip_status(launch_test_dequant(base, N, K, paired, out, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
