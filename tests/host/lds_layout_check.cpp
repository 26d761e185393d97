// Host-side check of the LDS tile layout used by every kernel (csrc/fa_device.h):
// the chunk swizzle swz<D> is a permutation of each row's 16-byte chunks, and
// the two read shapes the kernels issue touch distinct banks within one LDS
// pass, under a 32-bank (128 B per pass) and a 64-bank (256 B per pass) model:
//   * 128-bit reads: consecutive lanes read the same chunk of consecutive
//     rows (MFMA A-operand fragments of K, Q, dO);
//   * ds_read_b64_tr_b16: in each 16-lane group lane j reads 8 bytes at row
//     R + j/4, column c0 + 4 (j % 4) of a 32-column block; the two 16-lane
//     groups of a half-wave cover columns c0 and c0 + 16 of the same rows.
// Prints one line per case and exits non-zero on any conflict.
#include <cstdio>
#include <set>
#include <vector>

#include "fa_device.h"

namespace {

int conflicts(const std::vector<int>& byte_addrs, int width, int nbanks) {
  std::set<int> seen;
  int n = 0, dup = 0;
  for (int a : byte_addrs)
    for (int k = 0; k < width; k += 4) {
      ++n;
      if (!seen.insert(((a + k) / 4) % nbanks).second) ++dup;
    }
  return dup;
}

template <int D>
int check() {
  constexpr int kChunks = D / 8;
  int bad = 0;
  for (int r = 0; r < 64; ++r) {  // permutation of the chunks of each row
    std::set<int> cs;
    for (int c = 0; c < kChunks; ++c) cs.insert(fa::tile_off<D>(r, c * 8) - r * D);
    if ((int)cs.size() != kChunks) {
      std::printf("D=%d row %d: swizzle is not a permutation\n", D, r);
      ++bad;
    }
  }
  for (int model = 0; model < 2; ++model) {
    const int nbanks = model ? 64 : 32;
    const int lanes_b128 = nbanks * 4 / 16, lanes_b64 = nbanks * 4 / 8;
    int k_conf = 0, v_conf = 0;
    for (int c = 0; c < kChunks; ++c)
      for (int r0 = 0; r0 < 64; r0 += lanes_b128) {
        std::vector<int> a;
        for (int i = 0; i < lanes_b128; ++i) a.push_back(2 * fa::tile_off<D>(r0 + i, c * 8));
        k_conf += conflicts(a, 16, nbanks);
      }
    for (int R = 0; R < 64; R += 4)
      for (int c0 = 0; c0 < D; c0 += 32) {
        std::vector<int> lanes;
        for (int g = 0; g < 2; ++g)
          for (int j = 0; j < 16; ++j)
            lanes.push_back(2 * fa::tile_off<D>(R + j / 4, c0 + 16 * g + 4 * (j % 4)));
        for (int p0 = 0; p0 < 32; p0 += lanes_b64)
          v_conf += conflicts(std::vector<int>(lanes.begin() + p0, lanes.begin() + p0 + lanes_b64),
                              8, nbanks);
      }
    std::printf("D=%d banks=%d: b128 conflicts %d, tr_b16 conflicts %d\n", D, nbanks, k_conf,
                v_conf);
    bad += k_conf + v_conf;
  }
  return bad;
}

// The 8-bit tiles of the FP8 forward (fa_device.h, "8-bit tiles"): both
// swizzles permute each row's chunks, the K-tile row order k8_row covers every
// key once per key block, and the 128-bit reads of a wave are conflict-free.
template <int D>
int check_fp8() {
  int bad = 0;
  constexpr int kChunksK = D / 16;
  for (int r = 0; r < 64; ++r) {
    std::set<int> ck, cv;
    for (int c = 0; c < kChunksK; ++c) ck.insert(fa::k8_off<D>(r, 16 * c) - r * D);
    for (int c = 0; c < 4; ++c) cv.insert(fa::v8_off(r, 16 * c) - r * 64);
    if ((int)ck.size() != kChunksK || (int)cv.size() != 4) {
      std::printf("fp8 D=%d row %d: swizzle is not a permutation\n", D, r);
      ++bad;
    }
  }
  for (int kb = 0; kb < 2; ++kb) {
    std::set<int> rows;
    for (int m = 0; m < 32; ++m) rows.insert(fa::k8_row(kb, m));
    for (int h = 0; h < 2; ++h)
      for (int i = 0; i < 16; ++i) {  // result row 8(i/4) + 4h + i%4 holds key 32h + 16kb + i
        const int m = 8 * (i / 4) + 4 * h + (i % 4);
        if (fa::k8_row(kb, m) != 32 * h + 16 * kb + i) {
          std::printf("fp8 k8_row(%d, %d) != %d\n", kb, m, 32 * h + 16 * kb + i);
          ++bad;
        }
      }
    if ((int)rows.size() != 32) ++bad;
  }
  for (int model = 0; model < 2; ++model) {
    const int nbanks = model ? 64 : 32;
    const int group = nbanks * 4 / 16;  // lanes served per pass by 128-bit reads
    int k_conf = 0, v_conf = 0;
    for (int kb = 0; kb < 2; ++kb)
      for (int st = 0; st < D / 64; ++st)
        for (int u = 0; u < 2; ++u)
          for (int l0 = 0; l0 < 64; l0 += group) {
            std::vector<int> a;
            for (int l = l0; l < l0 + group; ++l) {
              const int m = l % 32, h = l / 32;
              const int chunk = (D == 128 ? 4 * st : 0) + 2 * h + u;
              a.push_back(fa::k8_off<D>(fa::k8_row(kb, m), 16 * chunk));
            }
            k_conf += conflicts(a, 16, nbanks);
          }
    for (int db = 0; db < D / 32; ++db)
      for (int u = 0; u < 2; ++u)
        for (int l0 = 0; l0 < 64; l0 += group) {
          std::vector<int> a;
          for (int l = l0; l < l0 + group; ++l)
            a.push_back(fa::v8_off(32 * db + l % 32, 16 * (2 * (l / 32) + u)));
          v_conf += conflicts(a, 16, nbanks);
        }
    std::printf("fp8 D=%d banks=%d: K b128 conflicts %d, V^T b128 conflicts %d\n", D, nbanks,
                k_conf, v_conf);
    bad += k_conf + v_conf;
  }
  return bad;
}

}  // namespace

int main() {
  const int bad = check<128>() + check<64>() + check_fp8<128>() + check_fp8<64>();
  std::printf(bad ? "FAIL\n" : "OK\n");
  return bad ? 1 : 0;
}
