// Section offsets of the packed Leech blob (see include/lvq.h, lvq_layout_bytes).
#pragma once

#include <stddef.h>

#include "../../include/lvq.h"

namespace lvq {

struct Sections {
  size_t table, codes, cls, scale, tail, total;
};

inline size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

inline Sections blob_sections(size_t rows, size_t cols) {
  const size_t nb = cols / 24, tau = cols % 24;
  Sections s;
  s.table = 0;
  s.codes = s.table + align256((size_t)LVQ_NUM_CLASSES * 8);
  s.cls = s.codes + align256(rows * nb * 12);
  s.scale = s.cls + align256(rows * nb * 2);
  s.tail = s.scale + align256(rows * 2);
  s.total = s.tail + align256(rows * tau * 2);
  return s;
}

// The LP2 blob: the same table, 12-byte code records with the class id inside,
// no class section (cls == codes, 0 bytes), scales and tails as above.
inline Sections lp2_sections(size_t rows, size_t cols) {
  const size_t nb = cols / 24, tau = cols % 24;
  Sections s;
  s.table = 0;
  s.codes = s.table + align256((size_t)LVQ_NUM_CLASSES * 8);
  s.cls = s.codes;
  s.scale = s.codes + align256(rows * nb * 12);
  s.tail = s.scale + align256(rows * 2);
  s.total = s.tail + align256(rows * tau * 2);
  return s;
}

// Direct layout (no class table): 16-byte records, then scales and tails.
inline Sections direct_sections(size_t rows, size_t cols) {
  const size_t nb = cols / 24, tau = cols % 24;
  Sections s;
  s.table = 0;  // none
  s.codes = 0;
  s.cls = 0;
  s.scale = align256(rows * nb * 16);
  s.tail = s.scale + align256(rows * 2);
  s.total = s.tail + align256(rows * tau * 2);
  return s;
}

// Direct code word w (0..3) of a block carries coordinate pairs P = 3w + v
// (v = 0, 1, 2), coordinates 2P and 2P + 1.  With |x| = 2h + p (p the
// block's parity), view v is the word rotated right by 5v: bits 1-3 h of the
// first coordinate, bit 15 its sign, bits 17-19 and 31 the second's.  p is
// bit 0 of word 0; the other bits are zero.
inline int direct_bit(int j, int field) {  // field 0..2: h bits, 3: sign
  const int pair = j >> 1, half = j & 1, v = pair % 3;
  const int b = (field < 3 ? 1 + field : 15) + 16 * half;
  return (b + 5 * v) & 31;
}

// One-hot blob: the LP3 sections with 16-byte code records (four words).
// Word i (0..3) is the indicator mask of rank i + 1 (rank 0: no bit set):
// coordinate 2P at bit P, coordinate 2P + 1 at bit 16 + P (P = 0..11).  Its
// spare bits 12-14 and 28-30 carry the signs of pairs 3i .. 3i + 2 (bit
// 12 + P - 3i for coordinate 2P, 28 + P - 3i for 2P + 1; 1 = negative).
inline Sections onehot_sections(size_t rows, size_t cols) {
  const size_t nb = cols / 24, tau = cols % 24;
  Sections s;
  s.table = 0;
  s.codes = s.table + align256((size_t)LVQ_NUM_CLASSES * 8);
  s.cls = s.codes + align256(rows * nb * 16);
  s.scale = s.cls + align256(rows * nb * 2);
  s.tail = s.scale + align256(rows * 2);
  s.total = s.tail + align256(rows * tau * 2);
  return s;
}
inline int onehot_mask_bit(int j) { return (j >> 1) + 16 * (j & 1); }
inline int onehot_sign_word(int j) { return (j >> 1) / 3; }
inline int onehot_sign_bit(int j) { return 12 + (j >> 1) % 3 + 16 * (j & 1); }

// LP2X: the LP2 blob followed by an exception side channel for the blocks LP2
// cannot hold (their main record is zero): row offsets u32 [rows + 1] and
// 16-byte entries {block index | class id << 16, the three LP3 code words}.
struct Lp2xSections {
  size_t exc_off, exc, total;
};
inline Lp2xSections lp2x_sections(size_t rows, size_t cols, size_t n_exc) {
  Lp2xSections x;
  x.exc_off = lp2_sections(rows, cols).total;
  x.exc = x.exc_off + align256((rows + 1) * 4);
  x.total = x.exc + align256(n_exc * 16);
  return x;
}

// LP2 code word w of a block holds coordinates 8w..8w+7: coordinate 8w+2v+h
// (view v = 0..3, half h = 0, 1) has its rank at bits 2v+16h .. 2v+16h+1 and
// its non-negative flag at bit 8+2v+16h.  Word 0's odd bits 9..15 and 25..31
// hold the class id: id bit 2i at bit 9+2i, id bit 2i+1 at bit 25+2i (i < 4).
constexpr int kLp2MaxClass = 256;
inline uint32_t lp2_class_bits(uint32_t id) {
  uint32_t w = 0;
  for (int i = 0; i < 4; ++i) {
    w |= ((id >> (2 * i)) & 1u) << (9 + 2 * i);
    w |= ((id >> (2 * i + 1)) & 1u) << (25 + 2 * i);
  }
  return w;
}

}  // namespace lvq
