// Plain CPU oracle for the int4 mixture-of-experts layer.
//
// TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or call
// this file: it exists so that the tests, the smoke check and the bench's CPU
// baseline can compare the HIP kernels against a slow, obviously correct
// definition. It shares no code, header, table or helper with the HIP library.
//
// Sources (the pages are news reports on Perplexity's Lily engine; they give
// the method in prose only):
//   [P1] diariobitcoin.com, "Perplexity libera Lily, un motor de IA que supera a
//        MLX-LM en Apple Silicon"; sections "Qwen3.6 combina tres cargas de
//        trabajo" and "Las optimizaciones en el prefill".
//   [P2] conexaoia.blog.br, "Perplexity disponibiliza Lily, motor de inferência
//        local para chips da Apple"; the model paragraph and the prefill paragraph.
// Where the pages are silent (activation, softmax rule, tie-break, shared-expert
// combine, group axis) the reading used is stated at the function.
//
// Precision: every floating-point step is done in double. Router logits are
// rounded once to fp32 because the selection rule is defined on fp32 logits.
// Expert outputs are returned in double; nothing is rounded to bf16.
//
// Pins: every function here is checked in tests/test_oracle_pins.py against
// closed forms, invariants, brute force and library routines (numpy / scipy
// on special cases); see the header of that file for the list.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>
#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

// A bf16 value is the top 16 bits of an IEEE fp32; widening is exact.
double bf16_value(uint16_t bits) {
  uint32_t u = static_cast<uint32_t>(bits) << 16;
  float f;
  std::memcpy(&f, &u, sizeof f);
  return static_cast<double>(f);
}

const int64_t kGroup = 64;  // quantisation group length [P1 "Qwen3.6 combina..."]

// One affine 4-bit weight: w = q * scale + bias, with one (scale, bias) pair per
// group of 64 consecutive elements along the input (column) dimension.
// [P1 "Qwen3.6 combina tres cargas de trabajo": 4-bit affine, groups of 64,
// bf16 scale and bias per group.] q is read as an unsigned integer 0..15.
inline double dequant_one(const uint8_t* q, const uint16_t* scale,
                          const uint16_t* bias, int64_t cols, int64_t n,
                          int64_t c) {
  const int64_t groups = cols / kGroup;
  const int64_t g = c / kGroup;
  return static_cast<double>(q[n * cols + c]) * bf16_value(scale[n * groups + g]) +
         bf16_value(bias[n * groups + g]);
}

double silu(double z) { return z / (1.0 + std::exp(-z)); }

// out[r] = sum_n Wd[r][n] * silu(sum_c Wg[n][c] x[c]) * (sum_c Wu[n][c] x[c])
// The pages never name the expert activation; this layer is a SwiGLU MLP
// (gate and up are [I][H], down is [H][I]), each matrix stored int4 affine.
void expert_ffn(const double* x, int64_t H, int64_t I, const uint8_t* qg,
                const uint16_t* sg, const uint16_t* bg, const uint8_t* qu,
                const uint16_t* su, const uint16_t* bu, const uint8_t* qd,
                const uint16_t* sd, const uint16_t* bd, double* out) {
  std::vector<double> h(I);
  for (int64_t n = 0; n < I; ++n) {
    double g = 0.0, u = 0.0;
    for (int64_t c = 0; c < H; ++c) {
      g += dequant_one(qg, sg, bg, H, n, c) * x[c];
      u += dequant_one(qu, su, bu, H, n, c) * x[c];
    }
    h[n] = silu(g) * u;
  }
  for (int64_t r = 0; r < H; ++r) {
    double d = 0.0;
    for (int64_t n = 0; n < I; ++n) d += dequant_one(qd, sd, bd, I, r, n) * h[n];
    out[r] = d;
  }
}

// Order of experts for one token: larger fp32 logit first, equal logits by
// lower expert index. Selection is done on the fp32 logits themselves (the
// softmax is monotone, so this picks the same set as ranking probabilities,
// and it does not depend on how exp rounds).
std::vector<int32_t> rank_experts(const float* l, int64_t E) {
  std::vector<int32_t> order(E);
  for (int64_t e = 0; e < E; ++e) order[e] = static_cast<int32_t>(e);
  std::stable_sort(order.begin(), order.end(), [l](int32_t a, int32_t b) {
    return l[a] > l[b];  // stable: ties keep ascending index
  });
  return order;
}

// Router selection for one token [P1 "Qwen3.6 combina tres cargas de trabajo":
// a router scores 256 experts and picks eight per token]. Weights: the softmax
// over all E logits, restricted to the selected experts and renormalised to sum
// to one. alt_swap=1 selects ranks 0..k-2 and k instead of 0..k-1 (the other
// valid choice when ranks k-1 and k are tied within rounding).
void select_token(const float* l, int64_t E, int64_t k, int alt_swap,
                  int32_t* idx, float* w) {
  std::vector<int32_t> order = rank_experts(l, E);
  for (int64_t j = 0; j < k; ++j) idx[j] = order[j];
  if (alt_swap && k < E) idx[k - 1] = order[k];
  double lmax = -INFINITY;
  for (int64_t e = 0; e < E; ++e) lmax = std::max(lmax, static_cast<double>(l[e]));
  std::vector<double> p(E);
  double z = 0.0;
  for (int64_t e = 0; e < E; ++e) {
    p[e] = std::exp(static_cast<double>(l[e]) - lmax);
    z += p[e];
  }
  for (int64_t e = 0; e < E; ++e) p[e] /= z;  // full softmax over E experts
  double zsel = 0.0;
  for (int64_t j = 0; j < k; ++j) zsel += p[idx[j]];
  for (int64_t j = 0; j < k; ++j) w[j] = static_cast<float>(p[idx[j]] / zsel);
}

// One token's logits, summed in double and rounded once to fp32.
void token_logits(const uint16_t* xrow, const float* wr, const float* rbias,
                  int64_t H, int64_t E, float* l) {
  for (int64_t e = 0; e < E; ++e) {
    double acc = 0.0;
    for (int64_t h = 0; h < H; ++h)
      acc += bf16_value(xrow[h]) * static_cast<double>(wr[e * H + h]);
    if (rbias) acc += static_cast<double>(rbias[e]);
    l[e] = static_cast<float>(acc);
  }
}

void set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
}

}  // namespace

extern "C" {

int oracle_max_threads() {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

// Expanded weights of one int4 matrix: w[n][c] = q[n][c]*scale[n][c/64] + bias[n][c/64].
int oracle_dequant(const uint8_t* q, const uint16_t* scale, const uint16_t* bias,
                   int64_t rows, int64_t cols, double* w) {
  if (!q || !scale || !bias || !w || rows < 0 || cols <= 0 || cols % kGroup) return -1;
  for (int64_t n = 0; n < rows; ++n)
    for (int64_t c = 0; c < cols; ++c) {
      if (q[n * cols + c] > 15) return -2;
      w[n * cols + c] = dequant_one(q, scale, bias, cols, n, c);
    }
  return 0;
}

// Router logits: logits[t][e] = fp32( sum_h x[t][h]*Wr[e][h] + rbias[e] ),
// the sum taken in double. x is bf16, Wr and rbias are fp32; rbias may be null.
int oracle_router_logits(const uint16_t* x, const float* wr, const float* rbias,
                         int64_t T, int64_t H, int64_t E, float* logits,
                         int nthreads) {
  if (!x || !wr || !logits || T < 0 || H <= 0 || E <= 0) return -1;
  set_threads(nthreads);
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) token_logits(x + t * H, wr, rbias, H, E, logits + t * E);
  return 0;
}

// Top-k selection and renormalised softmax weights, per token.
int oracle_topk(const float* logits, int64_t T, int64_t E, int64_t k,
                int alt_swap, int32_t* idx, float* w) {
  if (!logits || !idx || !w || T < 0 || E <= 0 || k <= 0 || k > E) return -1;
  for (int64_t t = 0; t < T; ++t)
    select_token(logits + t * E, E, k, alt_swap, idx + t * k, w + t * k);
  return 0;
}

// Routing metadata from the selected expert ids [P1 "Las optimizaciones en el
// prefill": routing histogram, prefix scan, scatter and block map].
//   hist[e]      number of (token, slot) pairs routed to e; sums to k*T
//   offsets[e]   exclusive prefix sum of hist; offsets[E] = k*T
//   perm[pos]    pair p = t*k + j placed at pos; pairs of one expert are
//                contiguous and in ascending p (a stable counting sort)
//   inv_perm[p]  the position of pair p
//   block_map    for each expert in ascending order, ceil(hist[e]/BM) blocks
//                (expert, first row, rows), rows in 1..BM
// Returns a negative value if an invariant fails (the sum, the bijection).
int oracle_route_meta(const int32_t* idx, int64_t T, int64_t E, int64_t k,
                      int64_t BM, int32_t* hist, int32_t* offsets, int32_t* perm,
                      int32_t* inv_perm, int32_t* block_map, int64_t max_blocks,
                      int32_t* num_blocks) {
  if (!idx || !hist || !offsets || !perm || !inv_perm || !block_map || !num_blocks ||
      T < 0 || E <= 0 || k <= 0 || BM <= 0)
    return -1;
  const int64_t P = T * k;
  for (int64_t e = 0; e < E; ++e) hist[e] = 0;
  for (int64_t p = 0; p < P; ++p) {
    if (idx[p] < 0 || idx[p] >= E) return -2;
    hist[idx[p]] += 1;
  }
  int64_t total = 0;
  for (int64_t e = 0; e < E; ++e) {
    offsets[e] = static_cast<int32_t>(total);
    total += hist[e];
  }
  offsets[E] = static_cast<int32_t>(total);
  if (total != P) return -3;
  std::vector<int64_t> fill(E, 0);
  for (int64_t p = 0; p < P; ++p) {
    const int32_t e = idx[p];
    const int64_t pos = offsets[e] + fill[e]++;
    perm[pos] = static_cast<int32_t>(p);
    inv_perm[p] = static_cast<int32_t>(pos);
  }
  std::vector<char> seen(P, 0);
  for (int64_t pos = 0; pos < P; ++pos) {
    if (perm[pos] < 0 || perm[pos] >= P || seen[perm[pos]]) return -4;
    seen[perm[pos]] = 1;
    if (inv_perm[perm[pos]] != pos) return -5;
  }
  int64_t nb = 0;
  for (int64_t e = 0; e < E; ++e) {
    for (int64_t i = 0; i * BM < hist[e]; ++i) {
      if (nb >= max_blocks) return -6;
      block_map[3 * nb + 0] = static_cast<int32_t>(e);
      block_map[3 * nb + 1] = static_cast<int32_t>(offsets[e] + i * BM);
      block_map[3 * nb + 2] = static_cast<int32_t>(std::min<int64_t>(BM, hist[e] - i * BM));
      ++nb;
    }
  }
  *num_blocks = static_cast<int32_t>(nb);
  return 0;
}

// One SwiGLU expert on one bf16 token row; out has H doubles.
int oracle_expert_ffn(const uint16_t* xrow, int64_t H, int64_t I,
                      const uint8_t* qg, const uint16_t* sg, const uint16_t* bg,
                      const uint8_t* qu, const uint16_t* su, const uint16_t* bu,
                      const uint8_t* qd, const uint16_t* sd, const uint16_t* bd,
                      double* out) {
  if (!xrow || !out || H <= 0 || I <= 0 || H % kGroup || I % kGroup) return -1;
  std::vector<double> x(H);
  for (int64_t c = 0; c < H; ++c) x[c] = bf16_value(xrow[c]);
  expert_ffn(x.data(), H, I, qg, sg, bg, qu, su, bu, qd, sd, bd, out);
  return 0;
}

// The whole layer for a list of tokens (all tokens when `tokens` is null).
// Expert arrays hold E+1 experts; index E is the shared expert, which every
// token uses with weight one [P1 "Qwen3.6 combina tres cargas de trabajo": a
// shared expert processes every token; its output is added unweighted].
//   y[t] = shared(x_t) + sum_j w[t][j] * expert_{idx[t][j]}(x_t)
// Logits, idx and w of the evaluated tokens are written when the pointers are
// non-null. Shapes: gate/up q [E+1][I][H], scale/bias [E+1][I][H/64];
// down q [E+1][H][I], scale/bias [E+1][H][I/64].
int oracle_layer(const uint16_t* x, int64_t T, int64_t H, int64_t I, int64_t E,
                 int64_t k, const float* wr, const float* rbias,
                 const uint8_t* qg, const uint16_t* sg, const uint16_t* bg,
                 const uint8_t* qu, const uint16_t* su, const uint16_t* bu,
                 const uint8_t* qd, const uint16_t* sd, const uint16_t* bd,
                 const int64_t* tokens, int64_t n_tokens, int alt_swap,
                 float* logits_out, int32_t* idx_out, float* w_out, double* y,
                 int nthreads) {
  if (!x || !wr || !qg || !qu || !qd || !y || T < 0 || H <= 0 || I <= 0 ||
      H % kGroup || I % kGroup || E <= 0 || k <= 0 || k > E)
    return -1;
  if (!tokens) n_tokens = T;
  for (int64_t i = 0; i < n_tokens; ++i)
    if (tokens && (tokens[i] < 0 || tokens[i] >= T)) return -2;
  const int64_t gu = I * H, gus = I * (H / kGroup);
  const int64_t dn = H * I, dns = H * (I / kGroup);
  set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < n_tokens; ++i) {
    const int64_t t = tokens ? tokens[i] : i;
    std::vector<float> l(E);
    token_logits(x + t * H, wr, rbias, H, E, l.data());
    std::vector<int32_t> idx(k);
    std::vector<float> w(k);
    select_token(l.data(), E, k, alt_swap, idx.data(), w.data());
    std::vector<double> xr(H), d(H), acc(H, 0.0);
    for (int64_t c = 0; c < H; ++c) xr[c] = bf16_value(x[t * H + c]);
    expert_ffn(xr.data(), H, I, qg + E * gu, sg + E * gus, bg + E * gus,
               qu + E * gu, su + E * gus, bu + E * gus, qd + E * dn,
               sd + E * dns, bd + E * dns, acc.data());
    for (int64_t j = 0; j < k; ++j) {
      const int64_t e = idx[j];
      expert_ffn(xr.data(), H, I, qg + e * gu, sg + e * gus, bg + e * gus,
                 qu + e * gu, su + e * gus, bu + e * gus, qd + e * dn,
                 sd + e * dns, bd + e * dns, d.data());
      for (int64_t r = 0; r < H; ++r) acc[r] += static_cast<double>(w[j]) * d[r];
    }
    for (int64_t r = 0; r < H; ++r) y[i * H + r] = acc[r];
    if (logits_out) std::memcpy(logits_out + i * E, l.data(), E * sizeof(float));
    if (idx_out) std::memcpy(idx_out + i * k, idx.data(), k * sizeof(int32_t));
    if (w_out) std::memcpy(w_out + i * k, w.data(), k * sizeof(float));
  }
  return 0;
}

// Brute-force form of the same layer: every token runs through all E routed
// experts, and each expert's output is multiplied by a mask that holds the
// renormalised weight for the k selected experts and zero for the rest.
int oracle_layer_dense_masked(const uint16_t* x, int64_t T, int64_t H, int64_t I,
                              int64_t E, int64_t k, const float* wr,
                              const float* rbias, const uint8_t* qg,
                              const uint16_t* sg, const uint16_t* bg,
                              const uint8_t* qu, const uint16_t* su,
                              const uint16_t* bu, const uint8_t* qd,
                              const uint16_t* sd, const uint16_t* bd, double* y,
                              int nthreads) {
  if (!x || !wr || !y || T < 0 || H <= 0 || I <= 0 || H % kGroup || I % kGroup ||
      E <= 0 || k <= 0 || k > E)
    return -1;
  const int64_t gu = I * H, gus = I * (H / kGroup);
  const int64_t dn = H * I, dns = H * (I / kGroup);
  set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < T; ++t) {
    std::vector<float> l(E);
    token_logits(x + t * H, wr, rbias, H, E, l.data());
    std::vector<int32_t> idx(k);
    std::vector<float> w(k);
    select_token(l.data(), E, k, 0, idx.data(), w.data());
    std::vector<double> mask(E, 0.0);
    for (int64_t j = 0; j < k; ++j) mask[idx[j]] = static_cast<double>(w[j]);
    std::vector<double> xr(H), d(H), acc(H, 0.0);
    for (int64_t c = 0; c < H; ++c) xr[c] = bf16_value(x[t * H + c]);
    for (int64_t e = 0; e <= E; ++e) {
      expert_ffn(xr.data(), H, I, qg + e * gu, sg + e * gus, bg + e * gus,
                 qu + e * gu, su + e * gus, bu + e * gus, qd + e * dn,
                 sd + e * dns, bd + e * dns, d.data());
      const double m = (e == E) ? 1.0 : mask[e];
      for (int64_t r = 0; r < H; ++r) acc[r] += m * d[r];
    }
    for (int64_t r = 0; r < H; ++r) y[t * H + r] = acc[r];
  }
  return 0;
}

}  // extern "C"
