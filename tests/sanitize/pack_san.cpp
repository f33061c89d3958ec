// Drives the host-side packers of the library (int4 affine weights, the
// router matrix) on small inputs, including every argument check, for a
// build with AddressSanitizer and UndefinedBehaviorSanitizer (host code
// only). Exits non-zero on a wrong return code; the sanitizers abort on any
// memory or undefined-behaviour error.
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "moe_int4.h"

static int failures = 0;
static void expect(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "FAILED: %s\n", what);
    ++failures;
  }
}

int main() {
  std::mt19937 rng(11);
  std::uniform_int_distribution<int> qd(0, 15);
  std::uniform_int_distribution<int> sd(0x3c00, 0x3d00);
  for (int paired = 0; paired < 2; ++paired) {
    for (int count : {1, 3}) {
      const int N = paired ? 32 : 64, K = 192;
      std::vector<uint8_t> q0(count * N * K), q1(count * N * K);
      std::vector<uint16_t> s0(count * N * K / 64), b0(s0.size()), s1(s0.size()), b1(s0.size());
      for (auto& v : q0) v = (uint8_t)qd(rng);
      for (auto& v : q1) v = (uint8_t)qd(rng);
      for (auto& v : s0) v = (uint16_t)sd(rng);
      for (auto& v : b0) v = (uint16_t)sd(rng);
      for (auto& v : s1) v = (uint16_t)sd(rng);
      for (auto& v : b1) v = (uint16_t)sd(rng);
      const size_t need = moe_packed_bytes(count, N, K, paired);
      expect(need > 0, "packed bytes");
      std::vector<uint8_t> out(need);
      const uint8_t* q1p = paired ? q1.data() : nullptr;
      expect(pack_int4_g64(q0.data(), s0.data(), b0.data(), q1p, s1.data(), b1.data(), count, N, K, out.data(),
                           need) == MOE_OK, "pack");
      expect(pack_int4_g64(q0.data(), s0.data(), b0.data(), q1p, s1.data(), b1.data(), count, N, K, out.data(),
                           need - 1) == MOE_EBUFFER, "pack, buffer one byte short");
      expect(pack_int4_g64(nullptr, s0.data(), b0.data(), q1p, s1.data(), b1.data(), count, N, K, out.data(),
                           need) == MOE_EINVAL, "pack, null codes");
      expect(pack_int4_g64(q0.data(), s0.data(), b0.data(), q1p, s1.data(), b1.data(), count, N, K - 1,
                           out.data(), need) == MOE_EUNSUPPORTED, "pack, K not a multiple of 64");
      q0[count * N * K - 1] = 16;
      expect(pack_int4_g64(q0.data(), s0.data(), b0.data(), q1p, s1.data(), b1.data(), count, N, K, out.data(),
                           need) == MOE_EFORMAT, "pack, code 16");
    }
  }
  expect(moe_packed_bytes(0, 64, 64, 0) == 0 && moe_packed_bytes(1, -64, 64, 0) == 0 &&
             moe_packed_bytes(1, 48, 64, 0) == 0 && moe_packed_bytes(1, 48, 64, 1) == 0,
         "packed bytes of unsupported dims");

  const int E = 64, H = 128;
  std::vector<float> wr(E * H);
  std::normal_distribution<float> nd(0.f, 0.02f);
  for (auto& v : wr) v = nd(rng);
  wr[3] = -0.0f;
  wr[4] = 1e-40f;  // subnormal
  const size_t rneed = moe_router_packed_bytes(E, H);
  expect(rneed > 0, "router packed bytes");
  std::vector<uint8_t> rout(rneed);
  expect(pack_router_bf16x3(wr.data(), E, H, rout.data(), rneed) == MOE_OK, "router pack");
  expect(pack_router_bf16x3(wr.data(), E, H, rout.data(), rneed - 1) == MOE_EBUFFER, "router pack, short");
  expect(pack_router_bf16x3(nullptr, E, H, rout.data(), rneed) == MOE_EINVAL, "router pack, null");
  expect(pack_router_bf16x3(wr.data(), 32, H, rout.data(), rneed) == MOE_EUNSUPPORTED, "router pack, E = 32");
  expect(moe_router_packed_bytes(0, H) == 0 && moe_router_packed_bytes(E, 100) == 0, "router bytes, bad dims");
  if (failures) return 1;
  std::printf("packer sanitizer run: all entry points clean\n");
  return 0;
}
