// Host check of the matrix-core decode's per-wavefront LDS addressing
// (decode_layout.h), run by tests/test_host_build.py, for D = 128 and 64. It
// fills a K and a V buffer image from the block loads' writes, every lane of a
// wavefront, and checks that each score operand read finds the cache row and
// dims its MFMA lane supplies (lane (lg, lr) of v_mfma_f32_16x16x32_bf16:
// A[lr][8 lg .. + 8]), that the transposing reads give lane (lg, r) dim
// 16 n + r of rows 8 lg .. 8 lg + 7, that every access stays inside its
// buffer, and that the 16-byte reads and writes and the 8-byte transposing
// reads touch distinct banks within each group of 16 lanes (64 banks of 4
// bytes; the LDS serves these accesses 16 lanes at a time: the counters of an
// earlier prefill kernel read no bank conflict at all with this V row stride
// and transposing reads, although lanes 16 apart share banks here). One
// exception is known and allowed: at D = 64 a 16-lane V write covers two
// padded rows 192 bytes apart, which share 16 banks (a 2-way conflict on the
// writes; the four transposing reads per write stay conflict-free). The
// transposing read is modelled as in the kernels' comments: within a 16-lane
// group, lanes 4a .. 4a + 3 address row a and lane i receives element i % 4 of
// the 8 bytes lane 4a + i / 4 addressed.
#include <cstdio>
#include <set>
#include <utility>
#include <vector>

#include "decode_layout.h"

using namespace yoco::dlay;

static int failures = 0;
#define CHECK(c)                                                                      \
  do {                                                                                \
    if (!(c)) {                                                                       \
      if (failures++ < 20) std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #c); \
    }                                                                                 \
  } while (0)

struct Elem {
  int row = -1, dim = -1;
};

static bool distinct_banks(const std::vector<int>& elem_offsets, int bytes) {
  std::set<int> banks;
  for (int e : elem_offsets)
    for (int b = 0; b < bytes / 4; ++b)
      if (!banks.insert((2 * e / 4 + b) % 64).second) return false;
  return true;
}

template <int D>
static void check() {
  using S = Shape<D>;
  // ---- the block loads fill both buffers once ----
  std::vector<Elem> kimg(S::kKElems), vimg(S::kVElems);
  std::vector<int> khits(S::kKElems, 0), vhits(S::kVElems, 0);
  for (int i = 0; i < S::NLI; ++i) {
    std::vector<int> kw, vw;
    for (int l = 0; l < 64; ++l) {
      const int row = load_row<D>(i, l), chunk = load_chunk<D>(l);
      CHECK(row >= 0 && row < kBlock && chunk >= 0 && chunk < D / 8);
      const int ko = k_write<D>(i, l), vo = v_write<D>(i, l);
      CHECK(ko % 8 == 0 && ko >= 0 && ko + 8 <= S::kKElems);
      CHECK(vo % 8 == 0 && vo >= 0 && vo + 8 <= S::kVElems);
      if (ko < 0 || ko + 8 > S::kKElems || vo < 0 || vo + 8 > S::kVElems) continue;
      for (int e = 0; e < 8; ++e) {
        kimg[ko + e] = {row, 8 * chunk + e};
        vimg[vo + e] = {row, 8 * chunk + e};
        ++khits[ko + e];
        ++vhits[vo + e];
      }
      kw.push_back(ko);
      vw.push_back(vo);
    }
    for (int g = 0; g < 4; ++g) {
      CHECK(distinct_banks(std::vector<int>(kw.begin() + 16 * g, kw.begin() + 16 * g + 16), 16));
      if (D == 128) CHECK(distinct_banks(std::vector<int>(vw.begin() + 16 * g, vw.begin() + 16 * g + 16), 16));
    }
  }
  for (int h : khits) CHECK(h == 1);
  for (int r = 0; r < kBlock; ++r)
    for (int c = 0; c < S::VPAD; ++c) CHECK(vhits[r * S::VPAD + c] == (c < D ? 1 : 0));   // the pad stays unwritten

  // ---- score operands ----
  for (int bb = 0; bb < 2; ++bb)
    for (int j = 0; j < S::NQK; ++j) {
      std::vector<int> rd;
      for (int l = 0; l < 64; ++l) {
        const int lg = l >> 4, lr = l & 15;
        CHECK(k_row<D>(l, bb) == 8 * (lr / 4) + 4 * bb + lr % 4);
        const int a = k_read<D>(l, bb, j);
        CHECK(a % 8 == 0 && a >= 0 && a + 8 <= S::kKElems);
        if (a < 0 || a + 8 > S::kKElems) continue;
        for (int e = 0; e < 8; ++e) CHECK(kimg[a + e].row == k_row<D>(l, bb) && kimg[a + e].dim == 32 * j + 8 * lg + e);
        rd.push_back(a);
      }
      for (int g = 0; g < 4; ++g) CHECK(distinct_banks(std::vector<int>(rd.begin() + 16 * g, rd.begin() + 16 * g + 16), 16));
    }

  // ---- transposing reads of the V buffer ----
  for (int n = 0; n < S::NDB; ++n)
    for (int h = 0; h < 2; ++h) {
      std::vector<int> addr(64);
      for (int l = 0; l < 64; ++l) {
        addr[l] = v_tr_read<D>(l, n, h);
        CHECK(addr[l] % 4 == 0 && addr[l] >= 0 && addr[l] + 4 <= S::kVElems);
      }
      for (int g = 0; g < 4; ++g)
        CHECK(distinct_banks(std::vector<int>(addr.begin() + 16 * g, addr.begin() + 16 * g + 16), 8));
      for (int l = 0; l < 64; ++l) {
        const int g = l >> 4, i = l & 15;
        for (int e = 0; e < 4; ++e) {
          const int src = addr[16 * g + 4 * e + (i >> 2)] + (i & 3);
          if (src < 0 || src >= S::kVElems) continue;
          CHECK(vimg[src].row == 8 * g + 4 * h + e && vimg[src].dim == 16 * n + i);
        }
      }
    }
}

int main() {
  check<128>();
  check<64>();
  // eight wavefronts' K and V buffers fit the 160 KiB a workgroup may hold
  static_assert(8 * 2 * (Shape<128>::kKElems + Shape<128>::kVElems) <= 160 * 1024, "LDS");
  if (failures) {
    std::printf("%d failures\n", failures);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
