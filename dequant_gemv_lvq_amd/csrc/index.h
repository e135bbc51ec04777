// Index tables of the 47-bit rank of the Leech ball m <= 12 (host-built,
// shared by the host ranker and the device unfolding kernel).
//
// A ball point is x = r + 4 z with r = 2c (even type t = 0) or 1 + 2c (odd
// type t = 1), c an extended Golay codeword, sum(z) even (t = 0) or odd
// (t = 1).  Indices run over (t, codeword message, x in lexicographic order).
// The norm limit sum x^2 <= 192 becomes a budget per type: x^2 = 4U (even,
// sum U <= 48) or x^2 = 1 + 8T (odd, sum T <= 21).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace lvq {

constexpr int kIdxQ = 49;            // budget states 0..48
constexpr int kIdxBlocks = 2 * 4096;  // (type, codeword) blocks
constexpr uint64_t kIdxMask = (1ull << 47) - 1;

// completions(t, nA, nB, q, p): ways to fill nA coordinates with c = 0 and nB
// with c = 1 with total cost <= q and z parities summing to p
constexpr size_t idx_f(int t, int na, int nb, int q, int p) {
  return ((((size_t)t * 25 + na) * 25 + nb) * kIdxQ + q) * 2 + p;
}
constexpr size_t kIdxFSize = (size_t)2 * 25 * 25 * kIdxQ * 2;

struct IndexTables {
  uint64_t f[kIdxFSize];
  uint64_t offs[kIdxBlocks + 1];  // first index of each block; offs[8192] = ball size
  uint32_t cw[4096];              // codeword of each 12-bit message
};

// Built once (thread-safe), never freed.
const IndexTables& index_tables();

}  // namespace lvq
