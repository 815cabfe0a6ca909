// Host check of the pipelined prefill's LDS addressing (prefill_layout.h), run
// by tests/test_host_build.py. It fills images of one K slot, one V slot and
// one V^T slot from the loads and writes the kernel issues, every lane of every
// wavefront, and checks that each MFMA operand read finds exactly the key row
// and dims its lane must supply (lane l of v_mfma_f32_32x32x16_bf16 supplies
// A[l % 32][8 (l / 32) .. + 8]), that every access stays inside its slot and
// the 150 KiB array, and that the reads the kernel relies on touch every LDS
// bank once per group of lanes (64 banks of 4 bytes: 16 lanes for the 16-byte
// reads; the 8-byte transposing reads over 32 lanes, more than the LDS needs,
// since it serves them 16 lanes at a time). The transposing read is
// modelled as the kernel comments state it: within a 16-lane group, lanes
// 4a .. 4a + 3 address row a (4 dims each) and lane i receives element i of
// every row.
#include <cstdio>
#include <cstdlib>
#include <set>
#include <utility>
#include <vector>

#include "prefill_layout.h"

using namespace yoco::pipe;

static int failures = 0;
#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      if (failures++ < 20) std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #c); \
    }                                                                   \
  } while (0)

struct Elem {   // what an LDS byte pair holds: (row, dim) of a tile, or (dim, key) in V^T
  int a = -1, b = -1;
};

// One tile slot filled by the direct loads; load_chunk is k_load_chunk or v_load_chunk.
template <typename F>
static std::vector<Elem> fill_slot(F load_chunk) {
  std::vector<Elem> img(kSlotB / 2);
  std::vector<int> hits(kSlotB / 16, 0);
  std::set<std::pair<int, int>> fetched;
  for (int w = 0; w < kWaves; ++w)
    for (int i = 0; i < kLoads; ++i)
      for (int l = 0; l < 64; ++l) {
        const int row = load_row(w, i, l), pos = l & 15, chunk = load_chunk(row, pos);
        const int dst = load_lds_offset(w, i) + 16 * l;   // byte within the slot
        CHECK(row >= 0 && row < kSK && chunk >= 0 && chunk < 16);
        CHECK(dst >= 0 && dst + 16 <= kSlotB && dst == row * kRowB + 16 * pos);
        if (dst < 0 || dst + 16 > kSlotB) continue;
        ++hits[dst / 16];
        fetched.insert({row, chunk});
        for (int e = 0; e < 8; ++e) img[dst / 2 + e] = {row, 8 * chunk + e};
      }
  for (int h : hits) CHECK(h == 1);
  CHECK((int)fetched.size() == kSK * 16);
  return img;
}

static bool distinct_banks(const std::vector<uint32_t>& addr, int bytes) {
  std::set<int> banks;
  for (uint32_t a : addr)
    for (int b = 0; b < bytes / 4; ++b)
      if (!banks.insert((int)((a / 4 + b) % 64)).second) return false;
  return true;
}

int main() {
  static_assert(kLdsBytes <= 160 * 1024, "a workgroup holds at most 160 KiB of LDS");

  // ---- K slot: score operands ----
  const std::vector<Elem> kimg = fill_slot(k_load_chunk);
  for (int hb = 0; hb < kSK / 32; ++hb)
    for (int c = 0; c < kD / 16; ++c) {
      std::vector<uint32_t> grp;
      for (int l = 0; l < 64; ++l) {
        const uint32_t a = k_operand(l, c) + (uint32_t)(hb * 32 * kRowB);
        CHECK(a % 16 == 0 && a + 16 <= (uint32_t)kSlotB);
        if (a + 16 > (uint32_t)kSlotB) continue;
        const int key = 32 * hb + perm_key(l & 31), d0 = 16 * c + 8 * (l >> 5);
        for (int e = 0; e < 8; ++e) CHECK(kimg[a / 2 + e].a == key && kimg[a / 2 + e].b == d0 + e);
        grp.push_back(a);
        if (grp.size() == 16) {
          CHECK(distinct_banks(grp, 16));
          grp.clear();
        }
      }
    }
  // perm_key swaps index bits 2 and 3: a bijection of 0..31 whose bit 2 moves to bit 3,
  // so the causal mask may add 8 q to the permuted row of accumulator element r
  {
    std::set<int> img;
    for (int i = 0; i < 32; ++i) img.insert(perm_key(i));
    CHECK(img.size() == 32 && *img.rbegin() == 31);
    for (int r = 0; r < 16; ++r)
      for (int q = 0; q < 2; ++q)
        CHECK(perm_key(8 * (r >> 2) + 4 * q + (r & 3)) == perm_key(8 * (r >> 2) + (r & 3)) + 8 * q);
  }

  // ---- V slot: transposing reads into V^T ----
  const std::vector<Elem> vimg = fill_slot(v_load_chunk);
  std::vector<Elem> vt(kVTSlotB / 2);
  std::vector<int> vt_hits(kVTSlotB / 2, 0);
  for (int w = 0; w < kWaves; ++w)
    for (int db = 0; db < kD / 32; ++db) {
      uint32_t tr[64];
      for (int l = 0; l < 64; ++l) {
        tr[l] = tr_read(w, l, db);
        CHECK(tr[l] % 8 == 0 && tr[l] >= (uint32_t)kVBase && tr[l] + 8 <= (uint32_t)(kVBase + kSlotB));
      }
      for (int half = 0; half < 2; ++half) CHECK(distinct_banks(std::vector<uint32_t>(tr + 32 * half, tr + 32 * half + 32), 8));
      for (int l = 0; l < 64; ++l) {
        const int g = l >> 4, i = l & 15;
        const uint32_t wa = vt_write(w, l, db);
        CHECK(wa == vt_write(w, l, 0) + (uint32_t)(db * 32 * kVTRow));   // the kernel adds the block offset
        CHECK(wa % 8 == 0 && wa >= (uint32_t)kVTBase && wa + 8 <= (uint32_t)(kVTBase + kVTSlotB));
        for (int k = 0; k < 4; ++k) {
          const uint32_t src = tr[16 * g + 4 * k + (i >> 2)] - kVBase + 2 * (i & 3);
          if (src + 2 > (uint32_t)kSlotB) continue;
          const Elem got = vimg[src / 2];
          CHECK(got.a == tr_first_key(w, l) + k && got.b == tr_dim(l, db));
          const uint32_t dst = wa - kVTBase + 2 * k;
          if (dst + 2 > (uint32_t)kVTSlotB) continue;
          CHECK(dst == (uint32_t)(got.b * kVTRow + 2 * got.a));   // V^T[dim][key]
          vt[dst / 2] = {got.b, got.a};
          ++vt_hits[dst / 2];
        }
      }
    }
  for (int d = 0; d < kD; ++d)
    for (int t = 0; t < kVTRow / 2; ++t) CHECK(vt_hits[d * kVTRow / 2 + t] == (t < kSK ? 1 : 0));   // the pad stays unwritten

  // ---- V^T slot: PV operands ----
  for (int hb = 0; hb < kSK / 32; ++hb)
    for (int hs = 0; hs < 2; ++hs)
      for (int db = 0; db < kD / 32; ++db) {
        std::vector<uint32_t> grp;
        for (int l = 0; l < 64; ++l) {
          const uint32_t a = pv_operand(l, hb, hs, db);
          CHECK(a == pv_operand(l, 0, 0, 0) + (uint32_t)(db * 32 * kVTRow + (32 * hb + 16 * hs) * 2));
          CHECK(a % 16 == 0 && a >= (uint32_t)kVTBase && a + 16 <= (uint32_t)(kVTBase + kVTSlotB));
          if (a < (uint32_t)kVTBase || a + 16 > (uint32_t)(kVTBase + kVTSlotB)) continue;
          const int dim = 32 * db + (l & 31), k0 = 32 * hb + 16 * hs + 8 * (l >> 5);
          for (int e = 0; e < 8; ++e) CHECK(vt[(a - kVTBase) / 2 + e].a == dim && vt[(a - kVTBase) / 2 + e].b == k0 + e);
          grp.push_back(a);
          if (grp.size() == 16) {
            CHECK(distinct_banks(grp, 16));
            grp.clear();
          }
        }
      }

  // slots of every kind stay inside the array, in the order K, V, V^T
  CHECK(kVBase == kNS * kSlotB && kVTBase == 2 * kNS * kSlotB && kVTBase + kNS * kVTSlotB == kLdsBytes);

  if (failures) {
    std::printf("%d failures\n", failures);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
