// Offline expander: integer Leech-lattice blocks -> packed blobs.
//
// Host-only C++ (no HIP call).  Implements lvq_class_table, lvq_strerror,
// lvq_last_error_index and the expanders and blob sizes of include/lvq.h: the
// served LP3 layout (lvq_expand, with the shape-gain bit: lvq_expand_gain),
// LP2 and LP2X (two rank planes, with the exception side channel), the
// table-free direct layout and the one-hot rank-mask layout.  Every expander
// validates each block (membership and the shell-12 limit) and reports the
// first offending one.
//
// Source: arXiv 2609.02652, section 1 (contributions C1 and C2): lattice
// codes are unfolded at load time into divergence-free layouts whose decode
// is shifts, masks and a table lookup; the class table is read once per block
// (related-work paragraph on lookup-table kernels).  The lattice rules and the
// Golay code are the classical construction (the paper cites Conway and
// Sloane); the canonical class order and the bit layout are this library's.

#include <algorithm>
#include <array>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/lvq.h"
#include "layout.h"

namespace {

constexpr int kMaxShell = 12;
constexpr int kMaxMag = 13;  // sqrt(16 * 12) rounded down

thread_local int g_err_row = -1;
thread_local int g_err_block = -1;

// ----------------------------------------------------------------------------
// Golay code: cyclic [23,12] code of g(x) = 1 + x^2 + x^4 + x^5 + x^6 + x^10 +
// x^11, extended with an overall parity bit in position 23.
// ----------------------------------------------------------------------------
struct Golay {
  std::vector<uint64_t> member;  // 2^24 bits
  int weight_count[25] = {0};
  Golay() : member((1u << 24) / 64, 0) {
    const uint32_t g = (1u << 0) | (1u << 2) | (1u << 4) | (1u << 5) | (1u << 6) |
                       (1u << 10) | (1u << 11);
    uint32_t rows[12];
    for (int i = 0; i < 12; ++i) {
      uint32_t v = g << i;
      rows[i] = v | ((uint32_t)(__builtin_popcount(v) & 1) << 23);
    }
    for (uint32_t msg = 0; msg < 4096; ++msg) {
      uint32_t w = 0;
      for (int i = 0; i < 12; ++i)
        if (msg >> i & 1) w ^= rows[i];
      member[w >> 6] |= 1ull << (w & 63);
      weight_count[__builtin_popcount(w)]++;
    }
  }
  bool contains(uint32_t mask) const { return member[mask >> 6] >> (mask & 63) & 1; }
};

const Golay& golay() {
  static const Golay g;
  return g;
}

// ----------------------------------------------------------------------------
// Classes: multisets of |x| realized by a lattice point of shell m <= 12.
// ----------------------------------------------------------------------------
struct ClassInfo {
  int m = 0;
  int parity = 0;
  std::array<uint8_t, 24> key{};      // magnitudes sorted descending
  std::array<uint8_t, 5> mags{};      // ascending distinct magnitudes
  int nmags = 0;
  uint8_t slot_of_mag[kMaxMag + 1]{};  // magnitude -> table slot (rank + 1)
  uint64_t count_key = 0;             // sum_v count[v] * 25^(v-1), v = 1..13
};

uint64_t count_key_of(const int counts[kMaxMag + 1]) {
  uint64_t k = 0, p = 1;
  for (int v = 1; v <= kMaxMag; ++v) {
    k += (uint64_t)counts[v] * p;
    p *= 25;
  }
  return k;
}

// Does some lattice point have |x| multiset `counts` (all values of one parity)?
bool realizable(const int counts[kMaxMag + 1], int parity) {
  const Golay& G = golay();
  if (parity == 0) {
    int w = 0, sum = 0;
    for (int v = 0; v <= kMaxMag; v += 2) {
      if (v % 4 == 2) w += counts[v];
      sum += v * counts[v];
    }
    if (G.weight_count[w] == 0) return false;
    return w > 0 || sum % 8 == 0;  // with w > 0 a sign flip fixes the sum
  }
  // odd type: choose how many of each value sit on a codeword's support (there
  // x = 3 mod 4) and check that the resulting sum can be 4 mod 8
  int vals[7], cnt[7], nv = 0;
  for (int v = 1; v <= kMaxMag; v += 2)
    if (counts[v]) { vals[nv] = v; cnt[nv] = counts[v]; ++nv; }
  int take[7] = {0};
  for (;;) {
    int w = 0, s = 0;
    for (int i = 0; i < nv; ++i) {
      w += take[i];
      int on = (vals[i] % 4 == 3) ? vals[i] : -vals[i];
      int off = (vals[i] % 4 == 1) ? vals[i] : -vals[i];
      s += take[i] * on + (cnt[i] - take[i]) * off;
    }
    if (G.weight_count[w] && ((s % 8) + 8) % 8 == 4) return true;
    int i = 0;
    while (i < nv && take[i] == cnt[i]) take[i++] = 0;
    if (i == nv) return false;
    take[i]++;
  }
}

struct ClassTable {
  std::vector<ClassInfo> cls;
  std::vector<uint64_t> entries;  // the public 8-byte table
  // open-addressing lookup from count_key to class id
  std::vector<uint64_t> hkeys;
  std::vector<int> hvals;

  void enumerate(int m, int parity, int v, int slots, int norm_left, int counts[]) {
    if (v < 0) {
      if (slots == 0 && norm_left == 0 && realizable(counts, parity)) {
        ClassInfo c;
        c.m = m;
        c.parity = parity;
        int pos = 0;
        for (int u = kMaxMag; u >= 0; --u)
          for (int i = 0; i < counts[u]; ++i) c.key[pos++] = (uint8_t)u;
        for (int u = 0; u <= kMaxMag; ++u)
          if (counts[u]) {
            c.slot_of_mag[u] = (uint8_t)(c.nmags + 1);
            c.mags[c.nmags++] = (uint8_t)u;
          }
        c.count_key = count_key_of(counts);
        cls.push_back(c);
      }
      return;
    }
    if (v % 2 != parity) {
      enumerate(m, parity, v - 1, slots, norm_left, counts);
      return;
    }
    int maxc = slots;
    if (v > 0) maxc = std::min(maxc, norm_left / (v * v));
    for (int c = maxc; c >= 0; --c) {
      if (v == 0 && c != slots) continue;
      counts[v] = c;
      enumerate(m, parity, v - 1, slots - c, norm_left - c * v * v, counts);
      counts[v] = 0;
    }
  }

  ClassTable() {
    ClassInfo origin;
    origin.nmags = 1;
    origin.mags[0] = 0;
    origin.slot_of_mag[0] = 1;
    cls.push_back(origin);
    int counts[kMaxMag + 1];
    for (int m = 1; m <= kMaxShell; ++m)
      for (int parity = 0; parity < 2; ++parity) {
        std::fill(counts, counts + kMaxMag + 1, 0);
        enumerate(m, parity, kMaxMag, 24, 16 * m, counts);
      }
    std::sort(cls.begin() + 1, cls.end(), [](const ClassInfo& a, const ClassInfo& b) {
      if (a.m != b.m) return a.m < b.m;
      return a.key < b.key;
    });
    entries.assign(cls.size(), 0);
    for (size_t i = 0; i < cls.size(); ++i) {
      uint8_t b[8] = {0};
      for (int k = 0; k < cls[i].nmags; ++k) b[k] = cls[i].mags[k];
      b[7] = (uint8_t)(cls[i].m | (cls[i].parity << 7));
      uint64_t e;
      std::memcpy(&e, b, 8);
      entries[i] = e;
    }
    hkeys.assign(1024, ~0ull);
    hvals.assign(1024, -1);
    for (size_t i = 0; i < cls.size(); ++i) {
      size_t h = (cls[i].count_key * 0x9E3779B97F4A7C15ull) >> 54;
      while (hkeys[h] != ~0ull) h = (h + 1) & 1023;
      hkeys[h] = cls[i].count_key;
      hvals[h] = (int)i;
    }
  }

  int lookup(uint64_t key) const {
    size_t h = (key * 0x9E3779B97F4A7C15ull) >> 54;
    while (hkeys[h] != ~0ull) {
      if (hkeys[h] == key) return hvals[h];
      h = (h + 1) & 1023;
    }
    return -1;
  }
};

const ClassTable& table() {
  static const ClassTable t;
  return t;
}

}  // namespace

namespace {
enum Format { kLp3, kLp2, kLp2x };
int expand_impl(const int8_t* coords, const uint8_t* gain_bits, const uint16_t* scale,
                const uint16_t* tail, int rows, int cols, void* blob_out, Format fmt = kLp3,
                size_t n_exc = 0);
int classify(const int8_t* x, int* id_out);
bool lp2_eligible(int id);
}  // namespace

extern "C" {

const char* lvq_strerror(int code) {
  switch (code) {
    case LVQ_OK: return "ok";
    case LVQ_E_NULL: return "a required pointer is NULL";
    case LVQ_E_SHAPE: return "unsupported shape (negative, not a required multiple, or too large)";
    case LVQ_E_ALIGN: return "a device pointer is not 16-byte aligned";
    case LVQ_E_NOT_LEECH: return "a block is not a Leech lattice point";
    case LVQ_E_NORM: return "a lattice block lies beyond shell 12";
    case LVQ_E_BATCH: return "batch must be between 1 and 4";
    case LVQ_E_HIP: return "a HIP call or kernel launch failed";
    case LVQ_E_LAYOUT: return "a block's class cannot be stored in the requested layout";
    default: return "unknown status";
  }
}

int lvq_last_error_index(int* row, int* block) {
  if (!row || !block) return LVQ_E_NULL;
  *row = g_err_row;
  *block = g_err_block;
  return LVQ_OK;
}

int lvq_class_table(uint64_t out[LVQ_NUM_CLASSES]) {
  if (!out) return LVQ_E_NULL;
  const ClassTable& t = table();
  if (t.entries.size() != LVQ_NUM_CLASSES) return LVQ_E_SHAPE;  // cannot happen
  std::memcpy(out, t.entries.data(), LVQ_NUM_CLASSES * 8);
  return LVQ_OK;
}

size_t lvq_layout_bytes(int rows, int cols) {
  if (rows < 0 || cols < 0) return 0;
  return lvq::blob_sections((size_t)rows, (size_t)cols).total;
}

int lvq_expand(const int8_t* coords, const uint16_t* scale, const uint16_t* tail, int rows,
               int cols, void* blob_out) {
  return expand_impl(coords, nullptr, scale, tail, rows, cols, blob_out);
}

size_t lvq_layout_bytes_lp2(int rows, int cols) {
  if (rows < 0 || cols < 0) return 0;
  return lvq::lp2_sections((size_t)rows, (size_t)cols).total;
}

int lvq_expand_lp2(const int8_t* coords, const uint16_t* scale, const uint16_t* tail, int rows,
                   int cols, void* blob_out) {
  return expand_impl(coords, nullptr, scale, tail, rows, cols, blob_out, kLp2);
}

int lvq_lp2x_exceptions(const int8_t* coords, int rows, int cols, size_t* n_exceptions) {
  g_err_row = g_err_block = -1;
  if (rows < 0 || cols < 0) return LVQ_E_SHAPE;
  if (!n_exceptions || (rows && cols >= 24 && !coords)) return LVQ_E_NULL;
  const size_t nb = (size_t)cols / 24;
  size_t n = 0;
  for (size_t b = 0; b < (size_t)rows * nb; ++b) {
    int id = 0;
    const int err = classify(coords + b * 24, &id);
    if (err) {
      g_err_row = (int)(b / nb);
      g_err_block = (int)(b % nb);
      return err;
    }
    n += lp2_eligible(id) ? 0 : 1;
  }
  *n_exceptions = n;
  return LVQ_OK;
}

size_t lvq_layout_bytes_lp2x(int rows, int cols, size_t n_exceptions) {
  if (rows < 0 || cols < 0) return 0;
  return lvq::lp2x_sections((size_t)rows, (size_t)cols, n_exceptions).total;
}

size_t lvq_layout_bytes_direct(int rows, int cols) {
  if (rows < 0 || cols < 0) return 0;
  return lvq::direct_sections((size_t)rows, (size_t)cols).total;
}

int lvq_expand_direct(const int8_t* coords, const uint16_t* scale, const uint16_t* tail, int rows,
                      int cols, void* blob_out) {
  g_err_row = g_err_block = -1;
  if (rows < 0 || cols < 0) return LVQ_E_SHAPE;
  const size_t R = (size_t)rows, nb = (size_t)cols / 24, tau = (size_t)cols % 24;
  if (!blob_out || (R && !scale) || (R && nb && !coords) || (R && tau && !tail))
    return LVQ_E_NULL;
  const lvq::Sections s = lvq::direct_sections(R, (size_t)cols);
  uint8_t* out = (uint8_t*)blob_out;
  std::memset(out, 0, s.total);
  uint32_t* codes = (uint32_t*)out;
  for (size_t b = 0; b < R * nb; ++b) {
    const int8_t* x = coords + b * 24;
    int id = 0;
    const int err = classify(x, &id);  // membership and the norm limit
    if (err) {
      g_err_row = (int)(b / nb);
      g_err_block = (int)(b % nb);
      return err;
    }
    const int p = x[0] & 1;
    uint32_t w[4] = {(uint32_t)p, 0, 0, 0};
    for (int j = 0; j < 24; ++j) {
      const int a = x[j] < 0 ? -x[j] : x[j];
      const int h = (a - p) >> 1;  // 0..6
      const int wj = (j >> 1) / 3;
      for (int f = 0; f < 3; ++f)
        if (h >> f & 1) w[wj] |= 1u << lvq::direct_bit(j, f);
      if (x[j] < 0) w[wj] |= 1u << lvq::direct_bit(j, 3);
    }
    std::memcpy(codes + b * 4, w, 16);
  }
  if (R) std::memcpy(out + s.scale, scale, R * 2);
  if (R && tau) std::memcpy(out + s.tail, tail, R * tau * 2);
  return LVQ_OK;
}

size_t lvq_layout_bytes_onehot(int rows, int cols) {
  if (rows < 0 || cols < 0) return 0;
  return lvq::onehot_sections((size_t)rows, (size_t)cols).total;
}

int lvq_expand_onehot(const int8_t* coords, const uint16_t* scale, const uint16_t* tail, int rows,
                      int cols, void* blob_out) {
  g_err_row = g_err_block = -1;
  if (rows < 0 || cols < 0) return LVQ_E_SHAPE;
  const size_t R = (size_t)rows, nb = (size_t)cols / 24, tau = (size_t)cols % 24;
  if (!blob_out || (R && !scale) || (R && nb && !coords) || (R && tau && !tail))
    return LVQ_E_NULL;
  const lvq::Sections s = lvq::onehot_sections(R, (size_t)cols);
  uint8_t* out = (uint8_t*)blob_out;
  std::memset(out, 0, s.total);
  const ClassTable& T = table();
  std::memcpy(out + s.table, T.entries.data(), LVQ_NUM_CLASSES * 8);
  uint32_t* codes = (uint32_t*)(out + s.codes);
  uint16_t* cls = (uint16_t*)(out + s.cls);
  for (size_t b = 0; b < R * nb; ++b) {
    const int8_t* x = coords + b * 24;
    int id = 0;
    const int err = classify(x, &id);  // membership and the norm limit
    if (err) {
      g_err_row = (int)(b / nb);
      g_err_block = (int)(b % nb);
      return err;
    }
    const ClassInfo& c = T.cls[id];
    uint32_t w[4] = {0, 0, 0, 0};
    for (int j = 0; j < 24; ++j) {
      const int a = x[j] < 0 ? -x[j] : x[j];
      const int rank = c.slot_of_mag[a] - 1;  // 0..4
      if (rank > 0) w[rank - 1] |= 1u << lvq::onehot_mask_bit(j);
      if (x[j] < 0) w[lvq::onehot_sign_word(j)] |= 1u << lvq::onehot_sign_bit(j);
    }
    std::memcpy(codes + b * 4, w, 16);
    cls[b] = (uint16_t)id;
  }
  if (R) std::memcpy(out + s.scale, scale, R * 2);
  if (R && tau) std::memcpy(out + s.tail, tail, R * tau * 2);
  return LVQ_OK;
}

int lvq_expand_lp2x(const int8_t* coords, const uint16_t* scale, const uint16_t* tail, int rows,
                    int cols, size_t n_exceptions, void* blob_out) {
  return expand_impl(coords, nullptr, scale, tail, rows, cols, blob_out, kLp2x, n_exceptions);
}

int lvq_expand_gain(const int8_t* coords, const uint8_t* gain_bits, const uint16_t* scale,
                    const uint16_t* tail, int rows, int cols, void* blob_out) {
  if (rows > 0 && cols >= 24 && !gain_bits) return LVQ_E_NULL;
  return expand_impl(coords, gain_bits, scale, tail, rows, cols, blob_out);
}

}  // extern "C"

namespace {

// Membership, norm and class of one block: LVQ_OK and the class id, or the
// error code.
int classify(const int8_t* x, int* id_out) {
  const ClassTable& T = table();
  const Golay& G = golay();
  const int par = x[0] & 1;
  bool same = true;
  uint32_t mask = 0;
  int sum = 0, norm = 0;
  for (int j = 0; j < 24; ++j) {
    const int v = x[j];
    same &= (v & 1) == par;
    const int r4 = v & 3;  // two's complement: v mod 4
    if (r4 == (par ? 3 : 2)) mask |= 1u << j;
    sum += v;
    norm += v * v;
  }
  if (!(same && G.contains(mask) && (sum & 7) == (par ? 4 : 0))) return LVQ_E_NOT_LEECH;
  if (norm > 16 * kMaxShell) return LVQ_E_NORM;
  int counts[kMaxMag + 1] = {0};
  for (int j = 0; j < 24; ++j) counts[x[j] < 0 ? -x[j] : x[j]]++;
  const int id = T.lookup(count_key_of(counts));
  if (id < 0) return LVQ_E_NOT_LEECH;  // a lattice point of shell <= 12 always has a class
  *id_out = id;
  return LVQ_OK;
}

bool lp2_eligible(int id) { return id < lvq::kLp2MaxClass && table().cls[id].nmags <= 4; }

void pack_lp3(const int8_t* x, const ClassInfo& c, uint32_t w[3]) {
  w[0] = w[1] = w[2] = 0;
  for (int j = 0; j < 24; ++j) {
    const int v = x[j];
    const int jj = j & 7;
    const int n = (jj >> 1) + 4 * (jj & 1);  // slot of coordinate j
    const uint32_t slot = c.slot_of_mag[v < 0 ? -v : v];
    w[j >> 3] |= slot << (4 * n);
    if (v >= 0) w[j >> 3] |= 1u << ((4 * n + 11) & 31);
  }
}

void pack_lp2(const int8_t* x, const ClassInfo& c, int id, uint32_t w[3]) {
  w[0] = w[1] = w[2] = 0;
  for (int j = 0; j < 24; ++j) {
    const int v = x[j];
    const int jj = j & 7, vv = jj >> 1, h = jj & 1;
    const uint32_t rk = (uint32_t)c.slot_of_mag[v < 0 ? -v : v] - 1;  // 0..3
    w[j >> 3] |= rk << (2 * vv + 16 * h);
    if (v >= 0) w[j >> 3] |= 1u << (8 + 2 * vv + 16 * h);
  }
  w[0] |= lvq::lp2_class_bits((uint32_t)id);
}

int expand_impl(const int8_t* coords, const uint8_t* gain_bits, const uint16_t* scale,
                const uint16_t* tail, int rows, int cols, void* blob_out, Format fmt,
                size_t n_exc) {
  g_err_row = g_err_block = -1;
  if (rows < 0 || cols < 0) return LVQ_E_SHAPE;
  const size_t R = (size_t)rows, nb = (size_t)cols / 24, tau = (size_t)cols % 24;
  if (!blob_out || (R && !scale) || (R && nb && !coords) || (R && tau && !tail))
    return LVQ_E_NULL;
  const ClassTable& T = table();
  const lvq::Sections s = fmt == kLp3 ? lvq::blob_sections(R, (size_t)cols)
                                      : lvq::lp2_sections(R, (size_t)cols);
  const lvq::Lp2xSections sx = lvq::lp2x_sections(R, (size_t)cols, n_exc);
  uint8_t* out = (uint8_t*)blob_out;
  std::memset(out, 0, fmt == kLp2x ? sx.total : s.total);
  std::memcpy(out + s.table, T.entries.data(), LVQ_NUM_CLASSES * 8);
  uint32_t* codes = (uint32_t*)(out + s.codes);
  uint16_t* cls = (uint16_t*)(out + s.cls);
  uint32_t* exc_off = (uint32_t*)(out + sx.exc_off);
  uint32_t* exc = (uint32_t*)(out + sx.exc);
  size_t e = 0;
  for (size_t r = 0; r < R; ++r) {
    if (fmt == kLp2x) exc_off[r] = (uint32_t)e;
    for (size_t k = 0; k < nb; ++k) {
      const int8_t* x = coords + (r * nb + k) * 24;
      int id = 0;
      const int err = classify(x, &id);
      if (err) {
        g_err_row = (int)r;
        g_err_block = (int)k;
        return err;
      }
      const ClassInfo& c = T.cls[id];
      uint32_t w[3];
      if (fmt != kLp3) {
        if (lp2_eligible(id)) {
          pack_lp2(x, c, id, w);
          std::memcpy(codes + (r * nb + k) * 3, w, 12);
        } else if (fmt == kLp2x) {
          // the side channel: block index, class, and the LP3 record; the
          // main record stays zero (the origin)
          if (e >= n_exc) return LVQ_E_SHAPE;
          pack_lp3(x, c, w);
          exc[4 * e] = (uint32_t)k | ((uint32_t)id << 16);
          std::memcpy(exc + 4 * e + 1, w, 12);
          ++e;
        } else {
          g_err_row = (int)r;
          g_err_block = (int)k;
          return LVQ_E_LAYOUT;
        }
        continue;
      }
      pack_lp3(x, c, w);
      std::memcpy(codes + (r * nb + k) * 3, w, 12);
      uint16_t g = 0;
      if (gain_bits) {
        if (gain_bits[r * nb + k] > 1) {
          g_err_row = (int)r;
          g_err_block = (int)k;
          return LVQ_E_SHAPE;
        }
        g = (uint16_t)(gain_bits[r * nb + k] << 15);
      }
      cls[r * nb + k] = (uint16_t)(id | g);
    }
  }
  if (fmt == kLp2x) {
    if (e != n_exc) return LVQ_E_SHAPE;
    exc_off[R] = (uint32_t)e;
  }
  if (R) std::memcpy(out + s.scale, scale, R * 2);
  if (R && tau) std::memcpy(out + s.tail, tail, R * tau * 2);
  return LVQ_OK;
}

}  // namespace
