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

}  // namespace lvq
