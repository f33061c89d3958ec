// Drives every entry point of the CPU oracle on small inputs, including the
// argument checks, for a build with AddressSanitizer and UndefinedBehavior-
// Sanitizer (host code only). Exits non-zero on a wrong return code; the
// sanitizers abort on any memory or undefined-behaviour error.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

extern "C" {
int oracle_max_threads();
int oracle_dequant(const uint8_t*, const uint16_t*, const uint16_t*, int64_t, int64_t, double*);
int oracle_router_logits(const uint16_t*, const float*, const float*, int64_t, int64_t, int64_t, float*, int);
int oracle_topk(const float*, int64_t, int64_t, int64_t, int, int32_t*, float*);
int oracle_route_meta(const int32_t*, int64_t, int64_t, int64_t, int64_t, int32_t*, int32_t*, int32_t*,
                      int32_t*, int32_t*, int64_t, int32_t*);
int oracle_expert_ffn(const uint16_t*, int64_t, int64_t, const uint8_t*, const uint16_t*, const uint16_t*,
                      const uint8_t*, const uint16_t*, const uint16_t*, const uint8_t*, const uint16_t*,
                      const uint16_t*, double*);
int oracle_layer(const uint16_t*, int64_t, int64_t, int64_t, int64_t, int64_t, const float*, const float*,
                 const uint8_t*, const uint16_t*, const uint16_t*, const uint8_t*, const uint16_t*,
                 const uint16_t*, const uint8_t*, const uint16_t*, const uint16_t*, const int64_t*, int64_t,
                 int, float*, int32_t*, float*, double*, int);
int oracle_layer_dense_masked(const uint16_t*, int64_t, int64_t, int64_t, int64_t, int64_t, const float*,
                              const float*, const uint8_t*, const uint16_t*, const uint16_t*, const uint8_t*,
                              const uint16_t*, const uint16_t*, const uint8_t*, const uint16_t*,
                              const uint16_t*, double*, int);
}

static int failures = 0;
static void expect(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "FAILED: %s\n", what);
    ++failures;
  }
}

static uint16_t bf16_of(float f) {  // truncation is enough for test data
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

int main() {
  std::mt19937 rng(7);
  std::normal_distribution<float> nd(0.f, 1.f);
  std::uniform_int_distribution<int> qd(0, 15);
  const int64_t T = 5, H = 128, I = 64, E = 16, k = 8, BM = 4;
  std::vector<uint16_t> x(T * H);
  for (auto& v : x) v = bf16_of(nd(rng));
  std::vector<float> wr(E * H), rb(E);
  for (auto& v : wr) v = 0.05f * nd(rng);
  for (auto& v : rb) v = 0.1f * nd(rng);
  // E + 1 experts (the last is the shared one)
  auto qv = [&](int64_t n) { std::vector<uint8_t> q(n); for (auto& v : q) v = (uint8_t)qd(rng); return q; };
  auto sv = [&](int64_t n, float s) { std::vector<uint16_t> a(n); for (auto& v : a) v = bf16_of(s * (1.f + 0.1f * nd(rng))); return a; };
  const int64_t gu = (E + 1) * I * H, gus = (E + 1) * I * (H / 64), dn = (E + 1) * H * I, dns = (E + 1) * H * (I / 64);
  auto qg = qv(gu), qu = qv(gu), qdn = qv(dn);
  auto sg = sv(gus, 0.01f), bg = sv(gus, -0.08f), su = sv(gus, 0.01f), bu = sv(gus, -0.08f);
  auto sd = sv(dns, 0.01f), bd = sv(dns, -0.08f);

  expect(oracle_max_threads() >= 1, "max_threads");
  std::vector<double> w(I * H);
  expect(oracle_dequant(qg.data(), sg.data(), bg.data(), I, H, w.data()) == 0, "dequant");
  expect(oracle_dequant(qg.data(), sg.data(), bg.data(), I, 100, w.data()) == -1, "dequant bad cols");
  std::vector<uint8_t> badq(qg.begin(), qg.begin() + I * H);
  badq[5] = 16;
  expect(oracle_dequant(badq.data(), sg.data(), bg.data(), I, H, w.data()) == -2, "dequant code > 15");

  std::vector<float> logits(T * E);
  expect(oracle_router_logits(x.data(), wr.data(), rb.data(), T, H, E, logits.data(), 2) == 0, "logits");
  expect(oracle_router_logits(x.data(), wr.data(), nullptr, T, H, E, logits.data(), 0) == 0, "logits, no bias");
  expect(oracle_router_logits(nullptr, wr.data(), nullptr, T, H, E, logits.data(), 0) == -1, "logits null");

  std::vector<int32_t> idx(T * k);
  std::vector<float> wsel(T * k);
  std::vector<float> tied(T * E, 0.5f);  // every logit equal
  expect(oracle_topk(tied.data(), T, E, k, 0, idx.data(), wsel.data()) == 0, "topk ties");
  expect(oracle_topk(tied.data(), T, E, k, 1, idx.data(), wsel.data()) == 0, "topk ties, alternate swap");
  expect(oracle_topk(logits.data(), T, E, k, 0, idx.data(), wsel.data()) == 0, "topk");
  expect(oracle_topk(logits.data(), T, E, E + 1, 0, idx.data(), wsel.data()) == -1, "topk k > E");

  const int64_t max_blocks = T * k / BM + E;
  std::vector<int32_t> hist(E), offs(E + 1), perm(T * k), inv(T * k), bmap(3 * max_blocks), nb(1);
  expect(oracle_route_meta(idx.data(), T, E, k, BM, hist.data(), offs.data(), perm.data(), inv.data(),
                           bmap.data(), max_blocks, nb.data()) == 0, "route meta");
  std::vector<int32_t> one_expert(T * k, 3);  // every pair on expert 3: 15 empty experts
  expect(oracle_route_meta(one_expert.data(), T, E, k, BM, hist.data(), offs.data(), perm.data(), inv.data(),
                           bmap.data(), max_blocks, nb.data()) == 0, "route meta, one expert");

  std::vector<double> out(H);
  expect(oracle_expert_ffn(x.data(), H, I, qg.data(), sg.data(), bg.data(), qu.data(), su.data(), bu.data(),
                           qdn.data(), sd.data(), bd.data(), out.data()) == 0, "expert ffn");

  std::vector<double> y(T * H);
  std::vector<int64_t> toks = {4, 0, 2};
  expect(oracle_layer(x.data(), T, H, I, E, k, wr.data(), rb.data(), qg.data(), sg.data(), bg.data(), qu.data(),
                      su.data(), bu.data(), qdn.data(), sd.data(), bd.data(), nullptr, 0, 0, logits.data(),
                      idx.data(), wsel.data(), y.data(), 2) == 0, "layer, all tokens");
  expect(oracle_layer(x.data(), T, H, I, E, k, wr.data(), nullptr, qg.data(), sg.data(), bg.data(), qu.data(),
                      su.data(), bu.data(), qdn.data(), sd.data(), bd.data(), toks.data(), 3, 1, nullptr,
                      nullptr, nullptr, y.data(), 1) == 0, "layer, token list");
  expect(oracle_layer(x.data(), 0, H, I, E, k, wr.data(), nullptr, qg.data(), sg.data(), bg.data(), qu.data(),
                      su.data(), bu.data(), qdn.data(), sd.data(), bd.data(), nullptr, 0, 0, nullptr, nullptr,
                      nullptr, y.data(), 1) == 0, "layer, T = 0");
  expect(oracle_layer_dense_masked(x.data(), T, H, I, E, k, wr.data(), rb.data(), qg.data(), sg.data(),
                                   bg.data(), qu.data(), su.data(), bu.data(), qdn.data(), sd.data(), bd.data(),
                                   y.data(), 2) == 0, "dense masked layer");
  expect(oracle_layer_dense_masked(x.data(), T, 100, I, E, k, wr.data(), rb.data(), qg.data(), sg.data(),
                                   bg.data(), qu.data(), su.data(), bu.data(), qdn.data(), sd.data(), bd.data(),
                                   y.data(), 2) == -1, "dense masked, bad H");
  if (failures) return 1;
  std::printf("oracle sanitizer run: all entry points clean\n");
  return 0;
}
