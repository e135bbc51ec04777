// 47-bit rank of the Leech-lattice ball m <= 12 (host): the tables the device
// unfolding kernel reads, and lvq_rank.
//
// Source: arXiv 2609.02652 serves one 48-bit word per 24-weight block, a 47-bit
// index into the 301-class ball plus one gain bit, unfolded at load time (the
// quality-protocol, published-results and validity-envelope paragraphs).  The
// pages give no enumeration order; this library's is: even type before odd,
// codewords by 12-bit message, then the vector in lexicographic order.

#include <algorithm>
#include <cstring>
#include <memory>
#include <mutex>
#include <vector>

#include "../../include/lvq.h"
#include "index.h"

namespace lvq {
namespace {

int cost_of(int t, int v) { return t ? (v * v - 1) / 8 : v * v / 4; }
int residue_of(int t, int ci) { return t ? 1 + 2 * ci : 2 * ci; }
int zpar_of(int t, int ci, int v) { return ((v - residue_of(t, ci)) >> 2) & 1; }
int vmin_of(int r) {
  int v = r;
  while (v - 4 >= -13) v -= 4;
  return v;
}

std::unique_ptr<IndexTables> build() {
  auto T = std::make_unique<IndexTables>();
  std::memset(T->f, 0, sizeof(T->f));
  for (int t = 0; t < 2; ++t) {
    for (int q = 0; q < kIdxQ; ++q) T->f[idx_f(t, 0, 0, q, 0)] = 1;  // p = 1: 0 ways
    for (int n = 1; n <= 24; ++n) {
      for (int nb = 0; nb <= n; ++nb) {
        const int na = n - nb;
        // remove one coordinate: an A one if any, else a B one
        const int ci = na > 0 ? 0 : 1;
        const int na1 = na - (1 - ci), nb1 = nb - ci;
        const int r = residue_of(t, ci);
        for (int q = 0; q < kIdxQ; ++q)
          for (int p = 0; p < 2; ++p) {
            uint64_t s = 0;
            for (int v = vmin_of(r); v <= 13; v += 4) {
              const int c = cost_of(t, v);
              if (c <= q) s += T->f[idx_f(t, na1, nb1, q - c, p ^ zpar_of(t, ci, v))];
            }
            T->f[idx_f(t, na, nb, q, p)] = s;
          }
      }
    }
  }
  // Golay codewords by message: rows x^i g(x) extended by parity
  const uint32_t g = (1u << 0) | (1u << 2) | (1u << 4) | (1u << 5) | (1u << 6) | (1u << 10) |
                     (1u << 11);
  uint32_t rows[12];
  for (int i = 0; i < 12; ++i) {
    const uint32_t v = g << i;
    rows[i] = v | ((uint32_t)(__builtin_popcount(v) & 1) << 23);
  }
  for (uint32_t msg = 0; msg < 4096; ++msg) {
    uint32_t w = 0;
    for (int i = 0; i < 12; ++i)
      if (msg >> i & 1) w ^= rows[i];
    T->cw[msg] = w;
  }
  T->offs[0] = 0;
  for (int b = 0; b < kIdxBlocks; ++b) {
    const int t = b >> 12;
    const int nb = __builtin_popcount(T->cw[b & 4095]);
    T->offs[b + 1] = T->offs[b] + T->f[idx_f(t, 24 - nb, nb, t ? 21 : 48, t)];
  }
  return T;
}

}  // namespace

const IndexTables& index_tables() {
  static std::once_flag once;
  static std::unique_ptr<IndexTables> T;
  std::call_once(once, [] { T = build(); });
  return *T;
}

}  // namespace lvq

extern "C" int lvq_rank(const int8_t* coords, size_t nblocks, uint64_t* index_out) {
  if (nblocks && (!coords || !index_out)) return LVQ_E_NULL;
  const lvq::IndexTables& T = lvq::index_tables();
  // message of each codeword: (codeword << 12 | message), sorted, searched
  static std::once_flag once;
  static std::vector<uint64_t> by_cw;
  std::call_once(once, [&] {
    by_cw.resize(4096);
    for (uint64_t m = 0; m < 4096; ++m) by_cw[m] = (uint64_t)T.cw[m] << 12 | m;
    std::sort(by_cw.begin(), by_cw.end());
  });
  auto msg_of = [&](uint32_t cw) -> int {
    auto it = std::lower_bound(by_cw.begin(), by_cw.end(), (uint64_t)cw << 12);
    return it != by_cw.end() && (*it >> 12) == cw ? (int)(*it & 4095) : -1;
  };
  for (size_t k = 0; k < nblocks; ++k) {
    const int8_t* x = coords + k * 24;
    const int t = x[0] & 1;
    uint32_t c = 0;
    int sum = 0, norm = 0;
    bool same = true;
    for (int j = 0; j < 24; ++j) {
      same &= (x[j] & 1) == t;
      c |= (uint32_t)(((x[j] - t) >> 1) & 1) << j;
      sum += x[j];
      norm += x[j] * x[j];
    }
    const int msg = msg_of(c);
    if (!same || msg < 0 || (sum & 7) != (t ? 4 : 0)) return LVQ_E_NOT_LEECH;
    if (norm > 192) return LVQ_E_NORM;
    uint64_t idx = T.offs[(t << 12) | msg];
    int nb = __builtin_popcount(c), na = 24 - nb, q = t ? 21 : 48, p = t;
    for (int j = 0; j < 24; ++j) {
      const int ci = c >> j & 1;
      if (ci) --nb; else --na;
      const int r = ci ? (t ? 3 : 2) : (t ? 1 : 0);
      int v = r;
      while (v - 4 >= -13) v -= 4;
      for (; v < x[j]; v += 4) {
        const int cst = t ? (v * v - 1) / 8 : v * v / 4;
        if (cst <= q) idx += T.f[lvq::idx_f(t, na, nb, q - cst, p ^ (((v - r) >> 2) & 1))];
      }
      q -= t ? (x[j] * x[j] - 1) / 8 : x[j] * x[j] / 4;
      p ^= ((x[j] - r) >> 2) & 1;
    }
    index_out[k] = idx;
  }
  return LVQ_OK;
}
