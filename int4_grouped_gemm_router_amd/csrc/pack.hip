// Host-side packers: logical int4 affine weights and the fp32 router matrix
// into the layouts the gfx950 kernels read (see layout.h).
#include <cstring>

#include "../../include/moe_int4.h"
#include "layout.h"

using namespace moe;

namespace {

struct Header {
  uint32_t magic, version;
  int32_t count, N, K, paired;
  int64_t expert_bytes;
};

bool pack_dims_ok(int32_t count, int32_t N, int32_t K, int32_t paired) {
  if (count <= 0 || N <= 0 || K <= 0 || K % kGroup) return false;
  return paired ? (N % 32 == 0) : (N % 64 == 0);
}

}  // namespace

extern "C" size_t moe_packed_bytes(int32_t count, int32_t N, int32_t K, int32_t paired) {
  if (!pack_dims_ok(count, N, K, paired)) return 0;
  PackGeom g = pack_geom(N, K, paired);
  return (size_t)kHeaderBytes + (size_t)count * (size_t)g.expert_bytes;
}

extern "C" int pack_int4_g64(const uint8_t* q0, const uint16_t* s0, const uint16_t* b0,
                             const uint8_t* q1, const uint16_t* s1, const uint16_t* b1,
                             int32_t count, int32_t N, int32_t K, void* out, size_t out_bytes) {
  const int paired = (q1 != nullptr);
  if (!q0 || !s0 || !b0 || !out || (paired && (!s1 || !b1))) return MOE_EINVAL;
  if (!pack_dims_ok(count, N, K, paired)) return MOE_EUNSUPPORTED;
  const size_t need = moe_packed_bytes(count, N, K, paired);
  if (out_bytes < need) return MOE_EBUFFER;
  const PackGeom g = pack_geom(N, K, paired);
  uint8_t* base = static_cast<uint8_t*>(out);
  std::memset(base, 0, need);
  Header h{kMagic, (uint32_t)kVersion, count, N, K, paired, g.expert_bytes};
  std::memcpy(base, &h, sizeof h);
  const int64_t mat = (int64_t)N * K, mats = (int64_t)N * g.G;
  for (int e = 0; e < count; ++e) {
    uint8_t* eb = base + kHeaderBytes + (int64_t)e * g.expert_bytes;
    uint32_t* nib = reinterpret_cast<uint32_t*>(eb + g.nib_off);
    uint16_t* sb = reinterpret_cast<uint16_t*>(eb + g.sb_off);
    for (int wt = 0; wt < g.n_wt; ++wt) {
      for (int j = 0; j < kWaveCols; ++j) {
        // logical source of column j of this wave tile
        const uint8_t* q;
        const uint16_t *s, *b;
        int row;
        if (paired) {
          const bool up = (j >> 4) & 1;
          row = 32 * wt + 16 * (j >> 5) + (j & 15);
          q = (up ? q1 : q0) + e * mat;
          s = (up ? s1 : s0) + e * mats;
          b = (up ? b1 : b0) + e * mats;
        } else {
          row = 64 * wt + j;
          q = q0 + e * mat;
          s = s0 + e * mats;
          b = b0 + e * mats;
        }
        const int ct = j >> 4, c16 = j & 15;
        for (int gi = 0; gi < g.G; ++gi) {
          uint16_t* sbw = sb + (((int64_t)wt * g.G + gi) * 16 + c16) * 8;
          sbw[ct] = s[(int64_t)row * g.G + gi];
          sbw[4 + ct] = b[(int64_t)row * g.G + gi];
          for (int ks = 0; ks < 2; ++ks)
            for (int kb = 0; kb < 4; ++kb) {
              const int lane = kb * 16 + c16;
              uint32_t word = 0;
              for (int o = 0; o < 8; ++o) {
                const int k = gi * kGroup + 32 * ks + 8 * kb + o;
                const uint8_t code = q[(int64_t)row * K + k];
                if (code > 15) return MOE_EFORMAT;
                word |= (uint32_t)code << (4 * nibble_pos(o));
              }
              nib[nib_word(wt, gi, lane, 2 * ct + ks, g.G)] = word;
            }
        }
      }
    }
  }
  return MOE_OK;
}

extern "C" size_t moe_router_packed_bytes(int32_t E, int32_t H) {
  if (E <= 0 || H <= 0 || E % 64 || H % kGroup) return 0;
  return (size_t)kHeaderBytes + (size_t)3 * E * H * 2;
}

extern "C" int pack_router_bf16x3(const float* wr, int32_t E, int32_t H, void* out,
                                  size_t out_bytes) {
  if (!wr || !out) return MOE_EINVAL;
  if (E <= 0 || H <= 0 || E % 64 || H % kGroup) return MOE_EUNSUPPORTED;
  const size_t need = moe_router_packed_bytes(E, H);
  if (out_bytes < need) return MOE_EBUFFER;
  uint8_t* base = static_cast<uint8_t*>(out);
  std::memset(base, 0, need);
  Header h{kRouterMagic, (uint32_t)kVersion, E, H, 0, 0, 0};
  std::memcpy(base, &h, sizeof h);
  uint16_t* planes = reinterpret_cast<uint16_t*>(base + kHeaderBytes);
  const int n_et = E / 64, G = H / kGroup;
  for (int e = 0; e < E; ++e)
    for (int k = 0; k < H; ++k) {
      // Exact three-way split by truncation: each part keeps the next 8
      // significant bits, so hi + mid + lo == w (fp32 has 24).
      uint32_t u;
      std::memcpy(&u, &wr[(int64_t)e * H + k], 4);
      const uint32_t hi = u & 0xFFFF0000u;
      float fhi, r1, fmid, r2;
      std::memcpy(&fhi, &hi, 4);
      r1 = wr[(int64_t)e * H + k] - fhi;
      uint32_t u1;
      std::memcpy(&u1, &r1, 4);
      const uint32_t mid = u1 & 0xFFFF0000u;
      std::memcpy(&fmid, &mid, 4);
      r2 = r1 - fmid;
      uint32_t u2;
      std::memcpy(&u2, &r2, 4);
      const uint16_t parts[3] = {(uint16_t)(hi >> 16), (uint16_t)(mid >> 16), (uint16_t)(u2 >> 16)};
      const int et = e / 64, ct = (e % 64) / 16, c16 = e % 16;
      const int gi = k / kGroup, ks = (k % kGroup) / 32, kb = (k % 32) / 8, o = k % 8;
      const int lane = kb * 16 + c16;
      for (int p = 0; p < 3; ++p)
        planes[router_index(p, et, gi, ct, ks, lane, n_et, G) + o] = parts[p];
    }
  return MOE_OK;
}
