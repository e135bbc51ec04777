// Fused Leech-lattice dequantize-plus-matvec for gfx950: lvq_gemv and its
// variants over one kernel template (modes): the fused multi-matrix launch
// and the no-weights control (lvq_gemv_fused, lvq_gemv_noweights), the
// shape-gain GEMV (lvq_gemv_gain), the compact and alternative layouts
// (lvq_gemv_lp2, lvq_gemv_lp2x with its side channel in each row's
// epilogue, lvq_gemv_direct, lvq_gemv_onehot), the rotation in the prologue
// (lvq_gemv_rotated), and the lvq_decode test hook.
//
// Source: arXiv 2609.02652, section 1, contribution C1 (the fused multi-shell
// decoder): the matvec decodes an offline-expanded layout with bit operations
// and one table read per block, with no branch that depends on the block's
// class, and leaves the combinatorial index out of the kernel altogether.  The
// Tetra summary (arXiv 2609.35465, section 5.1) gives the epilogue order: the
// row scale first, then the unquantized tail.
//
// gfx950 design.  One wave64 owns one row at a time (rows are grid-strided
// over all waves).  Lane l takes blocks l, l + 64, ... of the row, so every
// load instruction of a wave reads one contiguous run of the row's code
// records (12 bytes per lane, 16 in the direct and one-hot layouts) and class
// ids (2 bytes per lane).  The loads are raw buffer loads: the per-lane
// offset is fixed, the item's position is in the scalar buffer resource, and
// a load past the row's end reads 0 (which decodes to +0), so no vector
// instruction goes to addressing or masking.  x is copied into LDS once per
// workgroup by buffer loads that write LDS directly (no registers, no vector
// instructions); the pair feeding view v of code word w of block k is the
// natural fp16 pair at column 24k + 8w + 2v.  The class table is staged in
// LDS as 8-byte byte-LUTs.  Per coordinate pair the decode is
//     rotate (v_alignbit), mask (v_and), byte LUT (v_perm)
// giving two signed magnitudes as exact fp16 subnormals (value * 2^-24), and
// one v_dot2_f32_f16 multiplies them with the x pair into an fp32
// accumulator; the 2^24 is folded into the row scale.  No MFMA: the batch-1
// matvec is a stream over HBM whose decode keeps the VALU about half busy
// (54 VALU per block-lane at the metric shape).  The wave reduction is a
// fixed DPP tree and every sum order is fixed by the columns, so the result
// does not depend on timing or on the launch geometry.

#include "common.h"
#include "rotate_dev.h"
#include "layout.h"

namespace lvq {

constexpr int kMaxWgThreads = 1024;
// blocks per lane per work item: the code words of the current and the next
// item must stay in registers (no spills) next to B accumulator pairs
constexpr int max_bpl(int B) { return B <= 2 ? 4 : 2; }

// Workgroup size for `rows` rows: 1024 threads (x staged once per 16 waves)
// when there are rows for 16 waves on every CU, smaller otherwise so the rows
// spread over all CUs.
inline int wg_threads(int rows, int cus) {
  int threads = kMaxWgThreads;
  while (threads > 256 && rows < cus * (threads / kWave)) threads /= 2;
  return threads;
}

// Blocks per lane for rows of nb blocks.  First the fewest idle lane slots in
// a row's last chunk; among those the one giving each wave closest to four
// items (enough loads in flight behind the decode; ties to the larger), or
// with two or fewer waves per SIMD the largest (fewest items, least per-item
// work).  Measured on MI355X over the shapes of a Qwen3-8B layer and the
// same bytes as 2048 x 24576 .. 32768 x 1536: with six or more waves per SIMD
// the largest blocks per lane (one item per wave) were up to 1.3 us slower
// (8192 x 6144: 8.8 against 7.6 us).  The fused multi-matrix launch, whose
// items each pick their matrix, keeps the largest there too (its q/k/v set,
// 6144 rows at 4096 columns: the stack's 144 launches 1321 us, 1376 with
// more, smaller items).
inline int choose_bpl(int nb, int maxb, int rows, int cus, bool fused) {
  const int wpb = wg_threads(rows, cus) / kWave;
  long long waves = ((long long)rows + wpb - 1) / wpb;
  if (waves > 2LL * cus) waves = 2LL * cus;  // up to two workgroups per CU
  waves *= wpb;
  const long long rows_per_wave = ((long long)rows + waves - 1) / waves;
  // with two or fewer waves per SIMD an item's loads cannot hide behind
  // another wave's decode anyway: fewer, larger items win
  const bool largest = waves <= 2LL * 4 * cus || (fused && waves >= 6LL * 4 * cus);
  long long best_idle = -1;
  for (int b = 1; b <= maxb; ++b) {
    const long long per = (long long)kWave * b;
    const long long idle = (nb + per - 1) / per * per - nb;
    if (best_idle < 0 || idle < best_idle) best_idle = idle;
  }
  int best = 1;
  long long best_score = -1;
  for (int b = 1; b <= maxb; ++b) {
    const long long per = (long long)kWave * b;
    if ((nb + per - 1) / per * per - nb != best_idle) continue;
    const long long items = rows_per_wave * ((nb + per - 1) / per);
    const long long score = largest ? b : -(items > 4 ? items - 4 : 4 - items) * 8 + b;
    if (best_score == -1 || score > best_score) { best = b; best_score = score; }
  }
  return best;
}

struct LeechView {
  const uint64_t* table;
  const uint32_t* codes;
  const uint16_t* cls;
  const uint16_t* scale;
  const uint16_t* tail;
};

__host__ __device__ inline LeechView lp2_view(const void* blob, size_t rows, size_t cols) {
  const Sections s = lp2_sections(rows, cols);
  const uint8_t* b = (const uint8_t*)blob;
  LeechView v;
  v.table = (const uint64_t*)(b + s.table);
  v.codes = (const uint32_t*)(b + s.codes);
  v.cls = nullptr;
  v.scale = (const uint16_t*)(b + s.scale);
  v.tail = (const uint16_t*)(b + s.tail);
  return v;
}

__host__ __device__ inline LeechView direct_view(const void* blob, size_t rows, size_t cols) {
  const Sections s = direct_sections(rows, cols);
  const uint8_t* b = (const uint8_t*)blob;
  LeechView v;
  v.table = nullptr;
  v.codes = (const uint32_t*)b;
  v.cls = nullptr;
  v.scale = (const uint16_t*)(b + s.scale);
  v.tail = (const uint16_t*)(b + s.tail);
  return v;
}

__host__ __device__ inline LeechView onehot_view(const void* blob, size_t rows, size_t cols) {
  const Sections s = onehot_sections(rows, cols);
  const uint8_t* b = (const uint8_t*)blob;
  LeechView v;
  v.table = (const uint64_t*)(b + s.table);
  v.codes = (const uint32_t*)(b + s.codes);
  v.cls = (const uint16_t*)(b + s.cls);
  v.scale = (const uint16_t*)(b + s.scale);
  v.tail = (const uint16_t*)(b + s.tail);
  return v;
}

__host__ __device__ inline LeechView leech_view(const void* blob, size_t rows, size_t cols) {
  const Sections s = blob_sections(rows, cols);
  const uint8_t* b = (const uint8_t*)blob;
  LeechView v;
  v.table = (const uint64_t*)(b + s.table);
  v.codes = (const uint32_t*)(b + s.codes);
  v.cls = (const uint16_t*)(b + s.cls);
  v.scale = (const uint16_t*)(b + s.scale);
  v.tail = (const uint16_t*)(b + s.tail);
  return v;
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Raw buffer resources (gfx9 family: untyped, 32-bit data format).  A load
// at a byte offset at or past `bytes` returns 0 without touching memory,
// which is how the loads of a chunk that runs past its row's end stay in
// bounds: every code word and class id past the end reads as 0, and the
// all-zero code word in class 0 decodes to +0 (byte 0 of class 0's LUT is
// 0x00, see stage_lut).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
// cache policy of the streamed loads: non-temporal (read once; they should
// not evict x, the class table or the row scales)
constexpr int kStream = 2;

// The matrices one launch works on: one (lvq_gemv, lvq_gemv_noweights) or up
// to kMaxFused sharing x and the column count (lvq_gemv_fused), their rows
// concatenated: global row g belongs to matrix m when start[m] <= g <
// start[m + 1].  Kernel modes: single matrix, fused set, and the no-weights
// control (the single-matrix launch with every weight load aimed at an empty
// buffer range: the same instructions, it reads x and writes y, and no
// weight byte).
constexpr int kMaxFused = 4;
// kGain: one matrix whose class ids carry a shape-gain bit in bit 15; the
// block's weights are multiplied by gain[bit]
// kLp2: one matrix in the LP2 layout (two rank planes, class in the record)
// kRot: one matrix whose input is first rotated, (H kron Q)(S x), in LDS
// kDirect: one matrix in the table-free direct layout (|x| = 2h + parity)
// kOneHot: one matrix in the one-hot layout (rank-indicator masks)
// kLp2x: kLp2 plus the LP2X exception side channel, added in each row's
// epilogue
constexpr int kSingle = 0, kFused = 1, kNoWeights = 2, kGain = 3, kLp2 = 4, kRot = 5,
              kDirect = 6, kOneHot = 7, kLp2x = 8;
// Rows of three 64-block chunks (128 < nb <= 192 blocks) with
// rows to fill the chip: one block per lane and a ring of three register
// sets, so that a row is in flight whole (measured on MI355X: 4096 x 4096
// batch 1 5.08 -> 4.72 us, 12288 x 4096 8.79 -> 8.37 us; more items in flight
// on longer rows was slower at every depth tried, and on rows of two chunks
// too: 16384 x 3072 7.97 us with a ring of two, 8.52 with three).
// Single-matrix launches only: the fused multi-matrix launch (per-item matrix
// selection) and the rotating one (its prologue) measured slower with it.
inline bool short_rows(int mode, int nb, int rows) {
  return mode != kFused && mode != kRot && nb > 2 * 64 && nb <= 3 * 64 && rows >= 2048;
}

constexpr bool is_lp2(int M) { return M == kLp2 || M == kLp2x; }
// 32-bit code words per block
constexpr int words_of(int M) { return M == kDirect || M == kOneHot ? 4 : 3; }

struct MatSet {
  LeechView v[kMaxFused];
  float* y[kMaxFused];
  int start[kMaxFused + 1];
  float gain[2];
  // kLp2x: the side channel's row offsets and entries
  const uint32_t* exc_off;
  const uint4* exc;
  // kRot: the rotation of x (see lvq_rotate)
  const uint32_t* rot_signs;
  const float* rot_q;
  int rot_m, rot_logk;
  float rot_scale;
};

template <int M>
__device__ __forceinline__ int mat_of(const MatSet& ms, int g) {
  int m = 0;
  if (M == kFused) {
#pragma unroll
    for (int i = 1; i < kMaxFused; ++i) m += g >= ms.start[i] ? 1 : 0;
  }
  return m;
}

// field f of matrix m, for a wave-uniform m, by scalar selects (a runtime
// index into the kernel-argument arrays, or a select of whole structs, would
// copy the arguments to scratch memory)
template <int M, typename F>
__device__ __forceinline__ auto pick(const MatSet& ms, int m, F f) {
  auto r = f(ms, 0);
  if (M == kFused) {
#pragma unroll
    for (int i = 1; i < kMaxFused; ++i) r = m == i ? f(ms, i) : r;
  }
  return r;
}

// start[m] for a wave-uniform m, by selects (indexing the kernel-argument
// array with a runtime index would copy it to scratch memory)
// (every mode: with one matrix m is 0 and start_of(ms, 1) is its row count)
template <int M>
__device__ __forceinline__ int start_of(const MatSet& ms, int m) {
  int r = ms.start[0];
#pragma unroll
  for (int i = 1; i <= kMaxFused; ++i) r = m == i ? ms.start[i] : r;
  return r;
}

// Work item = (row, chunk): a chunk is up to 64 * BPL consecutive blocks of a
// row, lane l taking blocks chunk0 + l, chunk0 + l + 64, ...  Wave w owns rows
// w, w + W, w + 2W, ... (W waves in the grid) and walks their chunks in order;
// its j-th item is row w + (j / nchunks) * W, chunk j % nchunks.  It issues the
// loads of the next items before it decodes the current one, so every wave
// keeps two items of code words in flight.  Rows, chunks and item counters
// are wave-uniform (scalar registers): each item's addresses are scalar buffer
// resources plus a fixed per-lane offset, so no vector instruction is spent on
// addressing.
// The 16-bit fields stay 16-bit: widened where they are used, not where they
// are loaded, so that no wait for them is placed ahead of the decode that
// needs them (a widening at the load is a use of the loaded register).
template <int BPL, int M>
struct ItemRegs {
  uint32_t w[BPL][words_of(M)];
  uint16_t c[BPL];
  uint16_t tail;   // this lane's tail value (0 for lanes >= tau)
  uint16_t scale;  // the row's fp16 scale
  uint32_t e0, e1;  // kLp2x: the row's side-channel entries [e0, e1) (uniform)
};

// LP2: bytes 0..3 the first four ascending magnitudes (rank selectors 0..3),
// byte 4 = 0x80 (negative), byte 5 = 0x00 (non-negative)
__device__ __forceinline__ uint2 stage_lut_lp2(uint64_t entry) {
  return make_uint2((uint32_t)entry, 0x80u);
}

// LP2 view v of a code word: selector bytes [rank A, 4 + nonneg A, rank B,
// 4 + nonneg B] in one AND-OR, then one byte permute
__device__ __forceinline__ uint32_t lp2_pair(uint32_t word, int v, uint32_t lut_lo,
                                             uint32_t lut_hi) {
  const uint32_t w = v ? word >> (2 * v) : word;
  return __builtin_amdgcn_perm(lut_hi, lut_lo, (w & 0x01030103u) | 0x04000400u);
}

// An item's loads come in two groups: its metadata (class ids, this lane's
// tail value, the row scale: everything the table lookups and the epilogue
// need) and its code words.  In the no-weights mode every load is issued
// against an empty range: out of range, it returns 0 and sends no request to
// memory, so the instructions, waits and registers are those of the real
// kernel and no weight byte is read (0 decodes as class 0, scale 0: y = +0).
template <int M>
__device__ __forceinline__ uint32_t weight_bytes(uint32_t n, bool valid) {
  return M == kNoWeights || !valid ? 0u : n;
}

// A lane's byte offsets into an item's class ids / tail values (2 bytes per
// lane) and code records, opaque to the optimiser once per item.  Without
// that the offsets of the item's loads (lane * size + u * 64 * size + 4 k) are
// loop invariants, hoisted into one register each: a register per load, and
// loads the backend can no longer merge (three dword loads per block instead
// of one dwordx3).  Passed through an empty asm statement per item (in place:
// the registers are loop-carried, so no copy), the constants fold into the
// loads' immediate offsets and every load of the item shares one register.
struct LaneOff {
  int meta, codes;
};
__device__ __forceinline__ int opaque(int& v) {
  asm volatile("" : "+v"(v));
  return v;
}

template <int BPL, int M>
__device__ __forceinline__ void load_meta(const MatSet& ms, int nb, int tau, int gr, int chunk,
                                          bool valid, LaneOff& lo, ItemRegs<BPL, M>& g) {
  const int lo2 = opaque(lo.meta);
  const int m = mat_of<M>(ms, gr);
  const int r = gr - start_of<M>(ms, m);
  const uint16_t* cls = pick<M>(ms, m, [](const MatSet& s, int i) { return s.v[i].cls; });
  const uint16_t* tail = pick<M>(ms, m, [](const MatSet& s, int i) { return s.v[i].tail; });
  const uint16_t* scale = pick<M>(ms, m, [](const MatSet& s, int i) { return s.v[i].scale; });
  const int k0 = chunk * (kWave * BPL);
  if (!is_lp2(M) && M != kDirect) {  // LP2 keeps the class in the record; direct has none
    const auto rc =
        buffer_rsrc(cls + (size_t)r * nb + k0, weight_bytes<M>((uint32_t)(nb - k0) * 2, valid));
#pragma unroll
    for (int u = 0; u < BPL; ++u)
      g.c[u] = __builtin_amdgcn_raw_buffer_load_b16(rc, lo2 + u * (kWave * 2), 0, kStream);
  }
  const auto rt = buffer_rsrc(tail + (size_t)r * tau, weight_bytes<M>((uint32_t)tau * 2, valid));
  g.tail = __builtin_amdgcn_raw_buffer_load_b16(rt, lo2, 0, 0);
  // the row scale, read by every lane (one transaction); a vector load, so
  // that waiting for it never holds up the LDS reads
  const auto rs = buffer_rsrc(scale + r, weight_bytes<M>(2, valid));
  g.scale = __builtin_amdgcn_raw_buffer_load_b16(rs, 0, 0, 0);
  if constexpr (M == kLp2x) {
    const auto re = buffer_rsrc(ms.exc_off + r, valid ? 8u : 0u);
    g.e0 = __builtin_amdgcn_raw_buffer_load_b32(re, 0, 0, 0);
    g.e1 = __builtin_amdgcn_raw_buffer_load_b32(re, 4, 0, 0);
  }
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(3))) uint32_t lds_u32;
typedef const __attribute__((address_space(3))) u32x4_t lds_u32x4;

template <int BPL, int M>
__device__ __forceinline__ void load_codes(const MatSet& ms, int nb, int gr, int chunk,
                                           bool valid, LaneOff& loff, ItemRegs<BPL, M>& g) {
  const int lo = opaque(loff.codes);
  const int m = mat_of<M>(ms, gr);
  const int r = gr - start_of<M>(ms, m);
  const uint32_t* codes = pick<M>(ms, m, [](const MatSet& s, int i) { return s.v[i].codes; });
  const int k0 = chunk * (kWave * BPL);
  if constexpr (M == kDirect || M == kOneHot) {
    // one 16-byte record per block
    const auto rw = buffer_rsrc(codes + ((size_t)r * nb + k0) * 4,
                                weight_bytes<M>((uint32_t)(nb - k0) * 16, valid));
#pragma unroll
    for (int u = 0; u < BPL; ++u) {
      const auto v = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, lo + u * (kWave * 16), 0, kStream));
      g.w[u][0] = v.x;
      g.w[u][1] = v.y;
      g.w[u][2] = v.z;
      g.w[u][3] = v.w;
    }
    return;
  } else {
  const auto rw = buffer_rsrc(codes + ((size_t)r * nb + k0) * 3,
                              weight_bytes<M>((uint32_t)(nb - k0) * 12, valid));
#pragma unroll
  for (int u = 0; u < BPL; ++u) {
    const int o = lo + u * (kWave * 12);
    g.w[u][0] = __builtin_amdgcn_raw_buffer_load_b32(rw, o, 0, kStream);
    g.w[u][1] = __builtin_amdgcn_raw_buffer_load_b32(rw, o + 4, 0, kStream);
    g.w[u][2] = __builtin_amdgcn_raw_buffer_load_b32(rw, o + 8, 0, kStream);
  }
  }
}

// Both groups, metadata first, so a table lookup never waits for code words.
template <int BPL, int M>
__device__ __forceinline__ void load_item(const MatSet& ms, int nb, int tau, int gr, int chunk,
                                          bool valid, LaneOff& lo, ItemRegs<BPL, M>& g) {
  load_meta<BPL, M>(ms, nb, tau, gr, chunk, valid, lo, g);
  load_codes<BPL, M>(ms, nb, gr, chunk, valid, lo, g);
}

// LDS layout (dynamic): lut uint2[302] | x.  At batch 1, and in the rotating
// mode, x is fp16 [B][kpad], kpad >= 24 * npad and >= cols, a multiple of 512,
// with npad = nchunks * 64 * BPL blocks; columns past cols are zero (the
// rotating mode adds its f32 buffer, Q and sign words after x).  The 32-bit
// pair feeding view v of code word w of block k is element 12k + 4w + v of a
// batch row (natural column order; in the direct and one-hot layouts pair
// P = 3w + v, element 12k + P).
// Above batch 1 (other modes) x is chunk-major: the 64 BPL 24 columns of
// chunk c of batch row bb at (c B + bb) 64 BPL 24 halves, then the tail
// columns 24 nb .. 24 nb + 23 of every batch row, 32 halves each.  The batch
// stride is then a constant of the kernel, so every x read of an item takes
// an immediate offset from one per-item base (with the run-time stride
// kpad each read of batch rows 1.. paid an address add).
template <int B, int M>
constexpr bool x_chunk_major() { return B >= 2 && M != kRot; }
template <int BPL>
constexpr int x_chunk_dwords() { return kWave * BPL * 12; }  // one chunk of one batch row

template <int B, int BPL, int M>
__device__ __forceinline__ void decode_item(const MatSet& ms, int nb, int tau, int nchunks,
                                            int kpad, int gr, int chunk, int lane,
                                            const ItemRegs<BPL, M>& g, const uint2* lut,
                                            const uint32_t* xs, lds_u32* xlane,
                                            float (&acc)[B][3]) {
  asm volatile("" ::: "memory");  // keep this item's LDS reads inside this item
  // Word wi of every block goes to accumulator wi: consecutive words always
  // use different registers, and each lane adds its blocks in column order
  // into the same registers whatever the blocks-per-lane of the launch, so a
  // row's result does not depend on the launch geometry (or on which other
  // matrices share the launch).
  constexpr bool kXC = x_chunk_major<B, M>();
  constexpr int kXS = x_chunk_dwords<BPL>();
  const int npair = kXC ? kXS : kpad / 2;  // batch-row stride of x, 32-bit words
  // The 16 bytes of x at 32-bit word o of the lane's x (word 0 = the pair
  // feeding view 0 of code word 0 of this item's first block, batch row 0),
  // through a 32-bit LDS pointer.  Batch 1 starts from this lane's base, set
  // once per kernel (one add per item); above batch 1 that extra live register
  // pushes the 64-VGPR variants into spills, so the address is formed per item.
  lds_u32* xl = B == 1 ? xlane + chunk * (kWave * BPL * 12)
                : kXC  ? (lds_u32*)xs + chunk * (B * kXS) + lane * 12
                       : (lds_u32*)xs + (chunk * (kWave * BPL) + lane) * 12;
  auto xq = [&](int o) -> u32x4_t { return *(lds_u32x4*)(xl + o); };
#pragma unroll
  for (int u = 0; u < BPL; ++u) {
    if constexpr (M == kDirect) {
      // view v of word w: the word rotated right by 5v, AND the h and sign
      // fields, OR the block parity into bit 0 of both halves: the fp16
      // subnormal pair (2h + p) 2^-24 with its signs, no table
      const uint32_t pp = (g.w[u][0] & 1u) * 0x00010001u;
#pragma unroll
      for (int bb = 0; bb < B; ++bb) {
        const int o = bb * npair + u * (kWave * 12);
        const u32x4_t q0 = xq(o), q1 = xq(o + 4), q2 = xq(o + 8);
        const uint32_t xp[12] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w,
                                 q2.x, q2.y, q2.z, q2.w};
#pragma unroll
        for (int wi = 0; wi < 4; ++wi) {
#pragma unroll
          for (int vi = 0; vi < 3; ++vi) {
            const uint32_t w = g.w[u][wi];
            const uint32_t r = vi ? __builtin_amdgcn_alignbit(w, w, 5 * vi) : w;
            const uint32_t d = (r & 0x800E800Eu) | pp;
            acc[bb][vi] = dot2(d, xp[3 * wi + vi], acc[bb][vi]);
          }
        }
      }
      continue;
    }
    if constexpr (M == kOneHot) {
      // pair P: magnitudes = m0 + sum over ranks i of [indicator] * (m_i - m0),
      // both halves at once (indicator bits at P and 16 + P); then the two
      // signs from the spare bits of word P / 3
      const uint2 l = lut[g.c[u]];
      uint32_t dm[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) dm[i] = (l.y >> (8 * i)) & 0xFFu;
#pragma unroll
      for (int bb = 0; bb < B; ++bb) {
        const int o = bb * npair + u * (kWave * 12);
        const u32x4_t q0 = xq(o), q1 = xq(o + 4), q2 = xq(o + 8);
        const uint32_t xp[12] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w,
                                 q2.x, q2.y, q2.z, q2.w};
#pragma unroll
        for (int P = 0; P < 12; ++P) {
          uint32_t m = l.x;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            m += ((g.w[u][i] >> P) & 0x00010001u) * dm[i];  // v_mad_u32_u24
          const uint32_t d = ((g.w[u][P / 3] << (3 - P % 3)) & 0x80008000u) | m;
          acc[bb][P % 3] = dot2(d, xp[P], acc[bb][P % 3]);
        }
      }
      continue;
    }
    // ids < 302 by construction (lvq_expand); bit 15 is the gain bit (kGain);
    // LP2: the id sits in the odd bits 9..15 and 25..31 of word 0
    const uint32_t w0 = g.w[u][0];
    const uint32_t cid = is_lp2(M) ? (((w0 >> 9) & 0x55u) | ((w0 >> 24) & 0xAAu))
                       : M == kGain ? (g.c[u] & 0x7FFFu) : g.c[u];
    const uint2 l = lut[cid];
    const float gam = M == kGain ? ((g.c[u] >> 15) ? ms.gain[1] : ms.gain[0]) : 1.f;
#pragma unroll
    for (int wi = 0; wi < 3; ++wi) {
      uint32_t d[4];
#pragma unroll
      for (int vi = 0; vi < 4; ++vi)
        d[vi] = is_lp2(M) ? lp2_pair(g.w[u][wi], vi, l.x, l.y)
                          : leech_pair(g.w[u][wi], vi, l.x, l.y);
#pragma unroll
      for (int bb = 0; bb < B; ++bb) {
        const u32x4_t xv = xq(bb * npair + u * (kWave * 12) + 4 * wi);
        if (M == kGain) {
          // the word's partial sum, times its block's gain
          float pw = dot2(d[0], xv.x, 0.f);
          pw = dot2(d[1], xv.y, pw);
          pw = dot2(d[2], xv.z, pw);
          pw = dot2(d[3], xv.w, pw);
          acc[bb][wi] = __builtin_fmaf(pw, gam, acc[bb][wi]);
        } else {
          float& a = acc[bb][wi];
          a = dot2(d[0], xv.x, a);
          a = dot2(d[1], xv.y, a);
          a = dot2(d[2], xv.z, a);
          a = dot2(d[3], xv.w, a);
        }
      }
    }
  }
  if (chunk == nchunks - 1) {
    if constexpr (M == kLp2x) {
      // the row's side-channel blocks (LP2 holds zeros there): lanes take the
      // entries in turn, decode the LP3 code words with the class's LP3 LUT
      // and add into their accumulators like any other block
      const uint32_t e0 = __builtin_amdgcn_readfirstlane(g.e0);
      const uint32_t e1 = __builtin_amdgcn_readfirstlane(g.e1);
      if (e0 != e1) {
        for (uint32_t e = e0 + lane; e < e1; e += kWave) {
          const uint4 ent = ms.exc[e];
          const int k = (int)(ent.x & 0xFFFFu);
          // batch row 0's pairs of block k
          const int xk = kXC ? (k / (kWave * BPL)) * (B * kXS) + (k % (kWave * BPL)) * 12 : 12 * k;
          const uint2 l = leech_lut(ms.v[0].table[ent.x >> 16]);  // never class 0
          const uint32_t w[3] = {ent.y, ent.z, ent.w};
#pragma unroll
          for (int wi = 0; wi < 3; ++wi) {
#pragma unroll
            for (int vi = 0; vi < 4; ++vi) {
              const uint32_t d = leech_pair(w[wi], vi, l.x, l.y);
#pragma unroll
              for (int bb = 0; bb < B; ++bb)
                acc[bb][wi] = dot2(d, xs[bb * npair + xk + 4 * wi + vi], acc[bb][wi]);
            }
          }
        }
      }
    }
    // epilogue: scale (with the 2^24 of the subnormal encoding), then the tail
    const float s = half_bits_to_float((uint16_t)g.scale) * 16777216.0f;
    const uint16_t* xh = (const uint16_t*)xs;
#pragma unroll
    for (int bb = 0; bb < B; ++bb) {
      float part = (acc[bb][0] + acc[bb][1] + acc[bb][2]) * s;
      if (lane < tau)
        part += half_bits_to_float((uint16_t)g.tail) *
                half_bits_to_float(kXC ? xh[nchunks * B * 2 * kXS + bb * 32 + lane]
                                       : xh[bb * kpad + 24 * nb + lane]);
      const float tot = wave_sum_lane63(part);
      if (lane == kWave - 1) {
        const int m = mat_of<M>(ms, gr);
        const int s0 = start_of<M>(ms, m);
        const int rows_m = start_of<M>(ms, m + 1) - s0;
        pick<M>(ms, m, [](const MatSet& s, int i) { return s.y[i]; })[(size_t)bb * rows_m + (gr - s0)] = tot;
      }
      acc[bb][0] = acc[bb][1] = acc[bb][2] = 0.f;
    }
  }
  asm volatile("" ::: "memory");
}

// The class table staged as per-class byte LUTs (leech_lut); class 0 gets
// 0x00 in byte 0 so that an all-zero code word reads as +0 (valid class-0
// code words never select byte 0).
// One-hot LUT: m0 in both 16-bit halves, and the steps m_i - m0 of ranks
// 1..4 as bytes (0 past the class's distinct magnitudes).
__device__ __forceinline__ uint2 stage_lut_onehot(uint64_t entry) {
  const uint32_t m0 = (uint32_t)entry & 0xFFu;
  uint32_t steps = 0;
#pragma unroll
  for (int i = 1; i <= 4; ++i) {
    const uint32_t mi = (uint32_t)(entry >> (8 * i)) & 0xFFu;
    steps |= (mi ? mi - m0 : 0u) << (8 * (i - 1));
  }
  return make_uint2(m0 * 0x00010001u, steps);
}

__device__ __forceinline__ uint2 stage_lut(int c, uint64_t entry) {
  uint2 l = leech_lut(entry);
  if (c == 0) l.x &= ~0xFFu;
  return l;
}

// Waves per SIMD the register allocation must leave room for: 8 (at most 64
// VGPRs, two 1024-thread workgroups per CU) for the variants that fit there
// without spilling, and whatever the allocation gives for the larger ones.
// (The shape-gain mode keeps a partial sum per word and goes without, as do
// the rotating mode, whose prologue holds 16-value butterfly sets, LP2
// above batch 1, whose class extraction needs the registers, and the one-hot
// mode, which keeps a block's four masks and its steps live across 12 pairs.)
constexpr int leech_min_waves(int B, int BPL, int M, int D) {
  return M != kGain && M != kRot && M != kOneHot && M != kLp2x && !(M == kLp2 && B > 1) &&
                 B + (D * BPL + 1) / 2 <= 4
             ? 8
             : 1;
}

// Stages s .. s + R - 1 of every sequence of the f32 buffer fb (the m
// sequences of K values one after another): coordinates 2^s apart.  The first
// pass (s = 0, m = 1) reads the staged fp16 x with its signs instead; the last
// scales, rounds and writes fp16 back to x at c m + b.
template <int R>
__device__ __forceinline__ void rot_lds_pass(uint16_t* xh, float* fb, const uint32_t* signs,
                                             int k, int m, int s, bool first, bool last,
                                             float scale, int tid, int nthr) {
  constexpr int kR = 1 << R;
  const int low = (1 << s) - 1;
  const int nsets = k >> R;
  for (int sg = tid; sg < m * nsets; sg += nthr) {
    const int b = m == 1 ? 0 : sg / nsets;
    const int set = sg - b * nsets;
    const int c0 = ((set & ~low) << R) | (set & low);
    float v[kR];
    if (first && kR == 16) {  // m == 1, s == 0: 16 consecutive fp16 of x, two 16-byte reads
      const uint32_t s16 = signs ? signs[c0 >> 5] >> (c0 & 31) : 0u;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint4 u = rot_apply_signs(*(const uint4*)(xh + c0 + 8 * h), s16 >> (8 * h));
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[8 * h + 2 * i] = rot_half((uint16_t)w[i]);
          v[8 * h + 2 * i + 1] = rot_half((uint16_t)(w[i] >> 16));
        }
      }
    } else if (first) {  // fewer than 16: element by element
#pragma unroll
      for (int t = 0; t < kR; ++t) v[t] = rot_half(xh[c0 + t] ^ rot_sign_bit(signs, c0 + t));
    } else {
#pragma unroll
      for (int t = 0; t < kR; ++t) v[t] = fb[b * k + c0 + (t << s)];
    }
    rot_set_stages<R>(v);
    if (last) {
#pragma unroll
      for (int t = 0; t < kR; ++t) xh[(c0 + (t << s)) * m + b] = rot_out(v[t], scale);
    } else {
#pragma unroll
      for (int t = 0; t < kR; ++t) fb[b * k + c0 + (t << s)] = v[t];
    }
  }
}

// Stages s .. s + R - 1 (s >= 4) of the MM sequences of K values in fb,
// coordinates 2^s apart: consecutive threads take consecutive sets, so
// consecutive addresses.  The last pass scales, rounds and writes fp16 x at
// c MM + b.
template <int R, int MM>
__device__ __forceinline__ void rot_fb_pass(uint16_t* xh, float* fb, int logk, int s, bool last,
                                            float scale, int tid, int nthr) {
  constexpr int kR = 1 << R;
  const int lsets = logk - R;  // log2 of the sets per sequence
  const int low = (1 << s) - 1;
  for (int sg = tid; sg < (MM << lsets); sg += nthr) {
    const int b = MM == 1 ? 0 : sg >> lsets;
    const int set = sg & ((1 << lsets) - 1);
    const int c0 = ((set & ~low) << R) | (set & low);
    float* f = fb + (b << logk) + c0;
    float v[kR];
#pragma unroll
    for (int t = 0; t < kR; ++t) v[t] = f[t << s];
    rot_set_stages<R>(v);
    if (last) {
#pragma unroll
      for (int t = 0; t < kR; ++t) xh[(c0 + (t << s)) * MM + b] = rot_out(v[t], scale);
    } else {
#pragma unroll
      for (int t = 0; t < kR; ++t) f[t << s] = v[t];
    }
  }
}

// The rotation of one batch row for K >= 16 and m = MM <= 8.  1: the signs go
// into the staged x in place (16-byte units).  2: task L = b K/16 + c16 takes
// values 16 c16 .. 16 c16 + 15 of sequence b: for m = 1 two 16-byte reads of
// x, for m > 1 the Q mix of the 16 groups (32 m contiguous bytes of x, eight
// groups at a time) in registers, in lvq_rotate's fma order; stages 0-3 in
// registers; the 16 values to the f32 buffer (for m = 1 and K = 16, the
// result straight back to x).  3: radix passes for stages 4 and up, threads
// on consecutive sets (consecutive addresses); the last pass scales, rounds
// and writes x at c m + b (m > 1, K = 16: a copy pass does that).  Every
// stage is the same butterflies on the same operands as everywhere else, so
// the result is lvq_rotate's bit for bit.
template <int MM>
__device__ __forceinline__ void rotate_x_regs(uint16_t* xh, float* fb, const float* qs, const uint32_t* signs,
                              const MatSet& ms, int cols, int tid, int nthr) {
  const int logk = ms.rot_logk;
  float scale = ms.rot_scale;
  if (MM == 1 && qs) scale *= qs[0];
  if (signs) {
    for (int j8 = tid; j8 < (cols >> 3); j8 += nthr) {
      uint4* p = (uint4*)(xh + 8 * j8);
      *p = rot_apply_signs(*p, signs[j8 >> 2] >> ((j8 & 3) * 8));
    }
    __syncthreads();
  }
  // the 16-byte unit of x holding coordinates 8 j8 .. 8 j8 + 7
  auto unit = [&](int j8) { return *(const uint4*)(xh + 8 * j8); };
  const int lck = logk - 4;  // log2 of the 16-value chunks per sequence
  const bool direct = MM == 1 && logk == 4;
  for (int l = tid; l < (MM << lck); l += nthr) {
    const int b = MM == 1 ? 0 : l >> lck;
    const int c16 = l & ((1 << lck) - 1);
    float v[16];
    if (MM == 1) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint4 u = unit(2 * c16 + h);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[8 * h + 2 * i] = rot_half((uint16_t)w[i]);
          v[8 * h + 2 * i + 1] = rot_half((uint16_t)(w[i] >> 16));
        }
      }
    } else {
      float qrow[MM];
#pragma unroll
      for (int d = 0; d < MM; ++d) qrow[d] = qs ? qs[b * MM + d] : (d == b ? 1.f : 0.f);
      // groups g0 .. g0 + 7 (16 MM contiguous bytes) mixed into o[8]
      auto mix8 = [&](int g0, float* o) {
        uint32_t w[4 * MM];
#pragma unroll
        for (int i = 0; i < MM; ++i) {
          const uint4 u = unit(g0 * MM / 8 + i);
          w[4 * i] = u.x;
          w[4 * i + 1] = u.y;
          w[4 * i + 2] = u.z;
          w[4 * i + 3] = u.w;
        }
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          float a = 0.f;
#pragma unroll
          for (int d = 0; d < MM; ++d) {
            const int e = g * MM + d;
            a = __builtin_fmaf(qrow[d], rot_half((uint16_t)(w[e >> 1] >> (16 * (e & 1)))), a);
          }
          o[g] = a;
        }
      };
      mix8(16 * c16, v);
      asm volatile("" ::: "memory");  // one half's words live at a time
      mix8(16 * c16 + 8, v + 8);
    }
    rot_set_stages<4>(v);
    if (direct) {
      uint32_t o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        o[i] = rot_out(v[2 * i], scale) | ((uint32_t)rot_out(v[2 * i + 1], scale) << 16);
      *(uint4*)(xh + 16 * c16) = make_uint4(o[0], o[1], o[2], o[3]);
      *(uint4*)(xh + 16 * c16 + 8) = make_uint4(o[4], o[5], o[6], o[7]);
    } else {
      float4* f = (float4*)(fb + (b << logk) + 16 * c16);
#pragma unroll
      for (int i = 0; i < 4; ++i) f[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
    }
  }
  __syncthreads();
  if (direct) return;
  if (logk == 4) {  // m > 1, K = 16: the values are final; scale, round, interleave
    for (int c = tid; c < (MM << 4); c += nthr) xh[(c & 15) * MM + (c >> 4)] = rot_out(fb[c], scale);
    __syncthreads();
    return;
  }
  for (int st = 4; st < logk; st += 4) {
    const int r = logk - st < 4 ? logk - st : 4;
    const bool last = st + r == logk;
    if (r == 4) rot_fb_pass<4, MM>(xh, fb, logk, st, last, scale, tid, nthr);
    else if (r == 3) rot_fb_pass<3, MM>(xh, fb, logk, st, last, scale, tid, nthr);
    else if (r == 2) rot_fb_pass<2, MM>(xh, fb, logk, st, last, scale, tid, nthr);
    else rot_fb_pass<1, MM>(xh, fb, logk, st, last, scale, tid, nthr);
    __syncthreads();
  }
}

// One batch row of the staged x (fp16, in LDS, zero past cols) rotated in
// place.  The butterflies are lvq_rotate's, stage by stage in the same order on
// the same operands (only where the values live differs), and so is the Q mix,
// so the result is that kernel's output bit for bit.  K >= 16 and m <= 8 (every
// Qwen3 width but 25600) take rotate_x_regs; otherwise a thread takes whole
// groups of m coordinates for the Q mix, then radix-16 passes over the K-point
// sequences in LDS, one barrier each.  Every thread of the workgroup takes
// part; ends with a barrier.
__device__ __forceinline__ void rotate_x_lds(uint16_t* xh, float* fb, const float* qs, const uint32_t* signs,
                             const MatSet& ms, int cols, int tid, int nthr) {
  // qs and signs are the LDS copies (or null); no global load here, so
  // nothing waits on the weight loads in flight
  const int m = ms.rot_m, logk = ms.rot_logk;
  if (logk >= 4) {  // uniform
    switch (m) {
      case 1: return rotate_x_regs<1>(xh, fb, qs, signs, ms, cols, tid, nthr);
      case 2: return rotate_x_regs<2>(xh, fb, qs, signs, ms, cols, tid, nthr);
      case 3: return rotate_x_regs<3>(xh, fb, qs, signs, ms, cols, tid, nthr);
      case 4: return rotate_x_regs<4>(xh, fb, qs, signs, ms, cols, tid, nthr);
      case 5: return rotate_x_regs<5>(xh, fb, qs, signs, ms, cols, tid, nthr);
      case 6: return rotate_x_regs<6>(xh, fb, qs, signs, ms, cols, tid, nthr);
      case 7: return rotate_x_regs<7>(xh, fb, qs, signs, ms, cols, tid, nthr);
      case 8: return rotate_x_regs<8>(xh, fb, qs, signs, ms, cols, tid, nthr);
      default: break;
    }
  }
  // K < 16 or m > 8: passes over LDS
  const int k = cols / m;
  float scale = ms.rot_scale;
  if (m == 1 && qs) scale *= qs[0];
  if (m > 1) {
    for (int c = tid; c < k; c += nthr) {
      float xv[8];
      const bool small = m <= 8;  // uniform
      if (small) {
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          const int j = c * m + d;
          xv[d] = d < m ? rot_half(xh[j] ^ rot_sign_bit(signs, j)) : 0.f;
        }
      }
      for (int b = 0; b < m; ++b) {
        float a = 0.f;
        if (small) {
#pragma unroll
          for (int d = 0; d < 8; ++d)
            if (d < m) a = __builtin_fmaf(qs ? qs[b * m + d] : (d == b ? 1.f : 0.f), xv[d], a);
        } else {
          for (int d = 0; d < m; ++d) {
            const int j = c * m + d;
            a = __builtin_fmaf(qs ? qs[b * m + d] : (d == b ? 1.f : 0.f),
                               rot_half(xh[j] ^ rot_sign_bit(signs, j)), a);
          }
        }
        fb[b * k + c] = a;
      }
    }
    __syncthreads();
  }
  for (int s = 0; s < logk; s += 4) {
    const int r = logk - s < 4 ? logk - s : 4;
    const bool first = s == 0 && m == 1, last = s + r == logk;
    if (r == 4) rot_lds_pass<4>(xh, fb, signs, k, m, s, first, last, scale, tid, nthr);
    else if (r == 3) rot_lds_pass<3>(xh, fb, signs, k, m, s, first, last, scale, tid, nthr);
    else if (r == 2) rot_lds_pass<2>(xh, fb, signs, k, m, s, first, last, scale, tid, nthr);
    else rot_lds_pass<1>(xh, fb, signs, k, m, s, first, last, scale, tid, nthr);
    __syncthreads();
  }
  if (logk == 0) {  // K = 1: y = scale Q x, nothing but the mix
    for (int c = tid; c < cols; c += nthr) {
      const float v = m == 1 ? rot_half(xh[c] ^ rot_sign_bit(signs, c)) : fb[c];
      xh[c] = rot_out(v, scale);
    }
    __syncthreads();
  }
}

template <int B, int BPL, int M, int D>
__global__ void __launch_bounds__(kMaxWgThreads)
__attribute__((amdgpu_waves_per_eu(leech_min_waves(B, BPL, M, D))))
leech_gemv_kernel(MatSet ms, int rows, int nb, int tau, int cols, int nchunks, int kpad,
                  const uint16_t* __restrict__ x) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint2* lut = (uint2*)smem;
  uint32_t* xs = (uint32_t*)(smem + LVQ_NUM_CLASSES * 8);

  const int tid = threadIdx.x, nthr = blockDim.x;
  const int lane = tid & (kWave - 1);
  const int wpb = nthr / kWave;
  const int wave = __builtin_amdgcn_readfirstlane(blockIdx.x * wpb + (tid >> 6));
  const int nwaves = gridDim.x * wpb;
  // this wave's items: rows wave, wave + nwaves, ..., each with nchunks chunks
  const int myrows = wave < rows ? (rows - 1 - wave) / nwaves + 1 : 0;
  const int items = myrows * nchunks;
  const int per = kpad >> 3;  // 16-byte chunks per batch row of the staged x
  const int nq = B * per;
  const bool vec = ((cols & 7) == 0) && ((((uintptr_t)x) & 15) == 0);

  // 1. x into LDS.  With whole 16-byte units per batch row: buffer loads
  //    that write LDS directly, 1 KiB per wave instruction, columns past
  //    cols reading as 0 (kpad is a multiple of 512 columns, so a 1 KiB unit
  //    never straddles two batch rows).  Otherwise element by element.
  //    Up to 32 KiB the copies are issued by the first four waves only:
  //    waves start in order, so their copies enter the CU's memory queue
  //    ahead of most weight loads and the barrier below is not held up by a
  //    late wave's copies queued behind other waves' weight loads (measured:
  //    7.70 -> 7.45 us at 4096 x 12288, batch 1).  Larger copies go to every
  //    wave (issuing 24+ copies per wave costs more than it saves).
  //    Chunk-major x (above batch 1): 1 KiB unit q of the region goes to
  //    byte q * 1024, from column c 64 BPL 24 + 512 k of its batch row (3 BPL
  //    units per chunk and batch row); then the tail columns, one per thread.
  constexpr bool kXC = x_chunk_major<B, M>();
  if (kXC) {
    constexpr int kU = 3 * BPL, kXW = 2 * x_chunk_dwords<BPL>();  // units, halves per chunk row
    uint16_t* xh = (uint16_t*)xs;
    const int nu = nchunks * B * kU;
    if (vec) {
      const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
      const int nx = nu > 32 || wpb < 4 ? wpb : 4;
      for (int q = wv < nx ? wv : nu; q < nu; q += nx) {
        const int cb = q / kU, k = q - cb * kU, c = cb / B, bb = cb - c * B;
        const auto rx = buffer_rsrc(x + (size_t)bb * cols, (uint32_t)cols * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rx, (__attribute__((address_space(3))) void*)((uint8_t*)xs + (size_t)q * 1024), 16,
            lane * 16, c * (kXW * 2) + k * 1024, 0, 0);
      }
    } else {
      for (int i = tid; i < nchunks * B * kXW; i += nthr) {
        const int cb = i / kXW, e = i - cb * kXW, c = cb / B, bb = cb - c * B;
        const int col = c * kXW + e;
        xh[i] = col < cols ? x[(size_t)bb * cols + col] : (uint16_t)0;
      }
    }
    for (int i = tid; i < B * 32; i += nthr) {
      const int bb = i >> 5, t = i & 31;
      xh[nchunks * B * kXW + i] = t < tau ? x[(size_t)bb * cols + 24 * nb + t] : (uint16_t)0;
    }
  } else if (vec) {
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nx = nq > 32 * kWave || wpb < 4 ? wpb : 4;
    for (int q = wv < nx ? wv : nq; q * kWave < nq; q += nx) {
      const int u0 = q * kWave;  // first 16-byte unit of this KiB
      const int bb = B == 1 ? 0 : u0 / per;
      const int c0 = 8 * (u0 - bb * per);
      const auto rx = buffer_rsrc(x + (size_t)bb * cols, (uint32_t)cols * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (__attribute__((address_space(3))) void*)((uint8_t*)xs + (size_t)u0 * 16), 16,
          lane * 16, c0 * 2, 0, 0);
    }
  } else {
    uint16_t* xh = (uint16_t*)xs;
    for (int i = tid; i < B * kpad; i += nthr) {
      const int bb = i / kpad, c = i - bb * kpad;
      xh[i] = c < cols ? x[(size_t)bb * cols + c] : (uint16_t)0;
    }
  }
  // kRot: LDS after x holds the f32 rotation buffer [cols], then Q [m][m] and
  // the sign words, each rounded up to 256 bytes (one 4-byte-per-lane copy);
  // Q and the signs come in by buffer-to-LDS loads issued before the weight
  // loads, so the barrier below waits for them and the rotation makes no
  // global load
  float* fb = (float*)((uint8_t*)xs + (size_t)B * kpad * 2);
  float* qs = nullptr;
  uint32_t* sw = nullptr;
  if (M == kRot) {
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint8_t* p = (uint8_t*)fb + (((size_t)cols * 4 + 15) & ~(size_t)15);
    if (ms.rot_q) {
      qs = (float*)p;
      const uint32_t qb = (uint32_t)(ms.rot_m * ms.rot_m * 4);
      const auto rq = buffer_rsrc(ms.rot_q, qb);
      for (uint32_t q = wv; q * 256 < qb; q += wpb)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rq, (__attribute__((address_space(3))) void*)(p + q * 256), 4, lane * 4, q * 256, 0, 0);
      p += (qb + 255) & ~255u;
    }
    if (ms.rot_signs) {
      sw = (uint32_t*)p;
      const uint32_t sb = (uint32_t)((cols + 31) / 32 * 4);
      const auto rs = buffer_rsrc(ms.rot_signs, sb);
      for (uint32_t q = wv; q * 256 < sb; q += wpb)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)(p + q * 256), 4, lane * 4, q * 256, 0, 0);
    }
  }
  const uint64_t* table = ms.v[0].table;  // the same universal table in every blob
  const uint64_t te = M == kDirect ? 0 : table[min(tid, LVQ_NUM_CLASSES - 1)];
  asm volatile("" ::: "memory");
  // 2. the first D items, one in each register set of the ring.  Item j of
  //    this wave is row wave + (j / nchunks) nwaves, chunk j % nchunks.  A set
  //    whose item lies past the wave's last is loaded from an empty range (no
  //    memory request, every value 0), so the load sequence has no branch and
  //    every later wait counts exactly.
  ItemRegs<BPL, M> ring[D];
  int rr[D], rc[D];
  LaneOff lo = {lane * 2, lane * 4 * words_of(M)};
  lds_u32* const xlane = (lds_u32*)xs + lane * 12;
  {
    int r = wave, c = 0;
#pragma unroll
    for (int s = 0; s < D; ++s) {
      rr[s] = r;
      rc[s] = c;
      load_item<BPL, M>(ms, nb, tau, r, c, s < items, lo, ring[s]);
      if (++c == nchunks) { c = 0; r += nwaves; }
    }
  }
  asm volatile("" ::: "memory");
  // 3. the class table into LDS; the barrier also waits for x
  for (int c = tid; M != kDirect && c < LVQ_NUM_CLASSES; c += nthr) {
    const uint64_t e = c == tid ? te : table[c];
    lut[c] = is_lp2(M) ? stage_lut_lp2(e) : M == kOneHot ? stage_lut_onehot(e) : stage_lut(c, e);
  }
  __syncthreads();
  if (M == kRot) {
    // the first items' weight loads stay in flight meanwhile
    for (int bb = 0; bb < B; ++bb)
      rotate_x_lds((uint16_t*)xs + (size_t)bb * kpad, fb, qs, sw, ms, cols, tid, nthr);
  }

  float acc[B][3];
#pragma unroll
  for (int bb = 0; bb < B; ++bb) acc[bb][0] = acc[bb][1] = acc[bb][2] = 0.f;
  if (items == 0) return;
  auto decode = [&](int s) {
    decode_item<B, BPL, M>(ms, nb, tau, nchunks, kpad, rr[s], rc[s], lane, ring[s], lut, xs, xlane,
                           acc);
  };
  // steady state: set s holds item j + s; decode it, then load item j + s + D
  // into the same registers, so D - 1 items stay in flight behind each decode
  auto advance = [&](int& r, int& c) {
    c += D;
    while (c >= nchunks) { c -= nchunks; r += nwaves; }
  };
  int j = 0;
  for (; j + D < items; j += D) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      decode(s);
      advance(rr[s], rc[s]);
      load_item<BPL, M>(ms, nb, tau, rr[s], rc[s], j + s + D < items, lo, ring[s]);
    }
  }
  // the last one to D items, in sets 0 .. items - j - 1
#pragma unroll
  for (int s = 0; s < D; ++s)
    if (j + s < items) decode(s);
}

// Rows shorter than one block: y = sum of the unquantized tail only.
template <int B>
__global__ void __launch_bounds__(256)
leech_tail_only_kernel(LeechView v, int rows, int tau, const uint16_t* __restrict__ x,
                       float* __restrict__ y) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
#pragma unroll
  for (int bb = 0; bb < B; ++bb) {
    float a = 0.f;
    for (int t = 0; t < tau; ++t)
      a += half_bits_to_float(v.tail[(size_t)r * tau + t]) * half_bits_to_float(x[(size_t)bb * tau + t]);
    y[(size_t)bb * rows + r] = a;
  }
}

// One thread per block: blob -> int8 coordinates, through the same pair decode.
__global__ void __launch_bounds__(256)
leech_decode_kernel(LeechView v, size_t nblocks, int8_t* __restrict__ out) {
  const size_t g = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= nblocks) return;
  const uint2 l = leech_lut(v.table[min((uint32_t)v.cls[g], (uint32_t)(LVQ_NUM_CLASSES - 1))]);
  int8_t vals[24];
#pragma unroll
  for (int wi = 0; wi < 3; ++wi) {
    const uint32_t word = v.codes[3 * g + wi];
#pragma unroll
    for (int vi = 0; vi < 4; ++vi) {
      const uint32_t p = leech_pair(word, vi, l.x, l.y);
      const int lo = (int)(p & 0x3FFu), hi = (int)((p >> 16) & 0x3FFu);
      vals[8 * wi + 2 * vi] = (int8_t)((p & 0x8000u) ? -lo : lo);
      vals[8 * wi + 2 * vi + 1] = (int8_t)((p & 0x80000000u) ? -hi : hi);
    }
  }
  uint32_t* o = (uint32_t*)(out + 24 * g);
#pragma unroll
  for (int i = 0; i < 6; ++i)
    o[i] = (uint32_t)(uint8_t)vals[4 * i] | (uint32_t)(uint8_t)vals[4 * i + 1] << 8 |
           (uint32_t)(uint8_t)vals[4 * i + 2] << 16 | (uint32_t)(uint8_t)vals[4 * i + 3] << 24;
}

__global__ void zero_kernel(float* y, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = 0.f;
}

// Device attributes, cached per device id (ints written whole, with the same
// value by any thread that races on them).
int device_cus() {
  static int cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = __atomic_load_n(&cached[dev], __ATOMIC_RELAXED);
  if (!n) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    __atomic_store_n(&cached[dev], n, __ATOMIC_RELAXED);
  }
  return n;
}

size_t device_lds_bytes() {
  static int cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 65536;
  int n = __atomic_load_n(&cached[dev], __ATOMIC_RELAXED);
  if (!n) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
        n <= 0)
      n = 65536;
    __atomic_store_n(&cached[dev], n, __ATOMIC_RELAXED);
  }
  return (size_t)n;
}

int zero_output(float* y, size_t n, hipStream_t st) {
  if (!n) return LVQ_OK;
  clear_hip_error();
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, y, n);
  return launch_status();
}


// When set (lvq_gemv_launch_info), the Leech launch path records the launch
// it would make here instead of making it.
struct LaunchInfo {
  int threads, workgroups, blocks_per_lane, ring, lds_bytes;
};
thread_local LaunchInfo* t_dry_run = nullptr;

template <int B, int BPL, int M, int D>
int launch_leech_mode(const MatSet& ms, int rows, int cols, const uint16_t* x, hipStream_t st) {
  const int nb = cols / 24, tau = cols % 24;
  const int nchunks = (nb + kWave * BPL - 1) / (kWave * BPL);
  const size_t npad = (size_t)nchunks * kWave * BPL;
  size_t kpad = npad * 24 > (size_t)cols ? npad * 24 : (size_t)cols;
  kpad = (kpad + 511) & ~(size_t)511;
  size_t lds = (size_t)LVQ_NUM_CLASSES * 8 +
               (x_chunk_major<B, M>() ? (size_t)B * (npad * 24 + 32) * 2 : (size_t)B * kpad * 2);
  if (M == kRot) {
    lds += ((size_t)cols * 4 + 15) & ~(size_t)15;
    if (ms.rot_q) lds += ((size_t)ms.rot_m * ms.rot_m * 4 + 255) & ~(size_t)255;
    if (ms.rot_signs) lds += ((size_t)(cols + 31) / 32 * 4 + 255) & ~(size_t)255;
  }
  if (lds > device_lds_bytes()) return LVQ_E_SHAPE;
  const int cus = device_cus();
  const int threads = wg_threads(rows, cus);
  const int wpb = threads / kWave;
  // as many workgroups as fit on the chip at once (one or two per CU, by
  // registers and LDS), rows grid-strided over their waves
  static OccupancyCache occupancy;  // this instantiation's own
  const int occ = wgs_per_cu(occupancy, leech_gemv_kernel<B, BPL, M, D>, threads, lds);
  long long wgs = ((long long)rows + wpb - 1) / wpb;
  if (wgs > (long long)occ * cus) wgs = (long long)occ * cus;
  if (wgs < 1) wgs = 1;
  if (t_dry_run) {
    *t_dry_run = {threads, (int)wgs, BPL, D, (int)lds};
    return LVQ_OK;
  }
  clear_hip_error();
  hipLaunchKernelGGL((leech_gemv_kernel<B, BPL, M, D>), dim3((unsigned)wgs), dim3(threads), lds,
                     st, ms, rows, nb, tau, cols, nchunks, (int)kpad, x);
  return launch_status();
}

template <int B, int BPL, int M>
int launch_leech_ring(const MatSet& ms, int rows, int cols, const uint16_t* x, hipStream_t st) {
  if constexpr (BPL == 1 && M != kFused && M != kRot) {
    if (short_rows(M, cols / 24, rows)) return launch_leech_mode<B, BPL, M, 3>(ms, rows, cols, x, st);
  }
  return launch_leech_mode<B, BPL, M, 2>(ms, rows, cols, x, st);
}

// the shape-gain mode's extra partial sums, and the rotating mode's prologue,
// do not fit 4 blocks per lane at batch 2 (launch_leech never asks for it)
constexpr bool gain_bpl_ok(int B, int BPL) { return !(B >= 2 && BPL >= 4); }

template <int B, int BPL>
int launch_leech_bpl(const MatSet& ms, int mode, int rows, int cols, const uint16_t* x,
                     hipStream_t st) {
  if (mode == kFused) return launch_leech_ring<B, BPL, kFused>(ms, rows, cols, x, st);
  if (mode == kNoWeights) return launch_leech_ring<B, BPL, kNoWeights>(ms, rows, cols, x, st);
  if constexpr (gain_bpl_ok(B, BPL)) {
    if (mode == kGain) return launch_leech_ring<B, BPL, kGain>(ms, rows, cols, x, st);
  }
  if (mode == kLp2) return launch_leech_ring<B, BPL, kLp2>(ms, rows, cols, x, st);
  if (mode == kLp2x) return launch_leech_ring<B, BPL, kLp2x>(ms, rows, cols, x, st);
  if (mode == kDirect) return launch_leech_ring<B, BPL, kDirect>(ms, rows, cols, x, st);
  if (mode == kOneHot) return launch_leech_ring<B, BPL, kOneHot>(ms, rows, cols, x, st);
  if constexpr (gain_bpl_ok(B, BPL)) {
    if (mode == kRot) return launch_leech_ring<B, BPL, kRot>(ms, rows, cols, x, st);
  }
  return launch_leech_ring<B, BPL, kSingle>(ms, rows, cols, x, st);
}

// rows = total rows of the set; rows shorter than one block go to the
// tail-only kernel, one launch per matrix
template <int B>
int launch_leech(const MatSet& ms, int n, int mode, int rows, int cols, const uint16_t* x,
                 hipStream_t st) {
  const int nb = cols / 24;
  if (nb == 0) {
    for (int m = 0; m < n; ++m) {
      const int rm = ms.start[m + 1] - ms.start[m];
      if (!rm) continue;
      if (mode == kNoWeights) {  // the only weights are the tail: none are read
        const int e = zero_output(ms.y[m], (size_t)B * rm, st);
        if (e) return e;
        continue;
      }
      clear_hip_error();
      hipLaunchKernelGGL(leech_tail_only_kernel<B>, dim3((unsigned)((rm + 255) / 256)), dim3(256),
                         0, st, ms.v[m], rm, cols, x, ms.y[m]);
      const int e = launch_status();
      if (e) return e;
    }
    return LVQ_OK;
  }
  // short rows (short_rows): one block per lane, the whole row in flight;
  // otherwise the blocks-per-lane rule
  const int bpl = short_rows(mode, nb, rows)
                      ? 1
                      : choose_bpl(nb, (mode == kGain || mode == kRot) && B >= 2 ? 3 : max_bpl(B),
                                   rows, device_cus(), mode == kFused);
  if constexpr (max_bpl(B) >= 4) {
    if (bpl == 4) {
      const int e = launch_leech_bpl<B, 4>(ms, mode, rows, cols, x, st);
      if (!(e == LVQ_E_SHAPE && mode == kRot)) return e;
    }
  }
  if constexpr (max_bpl(B) >= 3) {
    if (bpl == 3) {
      const int e = launch_leech_bpl<B, 3>(ms, mode, rows, cols, x, st);
      if (!(e == LVQ_E_SHAPE && mode == kRot)) return e;
    }
  }
  if (bpl == 2) {
    const int e = launch_leech_bpl<B, 2>(ms, mode, rows, cols, x, st);
    // the rotating mode's LDS can miss by the padding of x; one block per
    // lane pads least (the size check fails before anything is launched)
    if (!(e == LVQ_E_SHAPE && mode == kRot)) return e;
  }
  return launch_leech_bpl<B, 1>(ms, mode, rows, cols, x, st);
}

int launch_set(const MatSet& ms, int n, int mode, int rows, int cols, const uint16_t* x, int batch,
               hipStream_t st) {
  switch (batch) {
    case 1: return launch_leech<1>(ms, n, mode, rows, cols, x, st);
    case 2: return launch_leech<2>(ms, n, mode, rows, cols, x, st);
    case 3: return launch_leech<3>(ms, n, mode, rows, cols, x, st);
    default: return launch_leech<4>(ms, n, mode, rows, cols, x, st);
  }
}

struct RotArgs {
  const uint32_t* signs = nullptr;
  const float* q = nullptr;
  int m = 1, logk = 0;
  float scale = 1.f;
};

int single_gemv(const void* blob, int rows, int cols, const uint16_t* x, float* y, int batch,
                void* stream, int mode, float gain0 = 1.f, float gain1 = 1.f,
                const RotArgs& rot = RotArgs(), const uint32_t* exc_off = nullptr,
                const uint4* exc = nullptr) {
  if (rows < 0 || cols < 0) return LVQ_E_SHAPE;
  int e = check_batch(batch);
  if (e) return e;
  if (!blob || !y || (cols && !x)) return LVQ_E_NULL;
  if (!aligned16(blob) || !aligned16(x) || !aligned16(y)) return LVQ_E_ALIGN;
  if ((long long)batch * cols > 65536) return LVQ_E_SHAPE;
  hipStream_t st = (hipStream_t)stream;
  if (rows == 0) return LVQ_OK;
  if (cols == 0) return zero_output(y, (size_t)batch * rows, st);
  MatSet ms = {};
  ms.v[0] = is_lp2(mode)     ? lp2_view(blob, (size_t)rows, (size_t)cols)
            : mode == kDirect ? direct_view(blob, (size_t)rows, (size_t)cols)
            : mode == kOneHot ? onehot_view(blob, (size_t)rows, (size_t)cols)
                              : leech_view(blob, (size_t)rows, (size_t)cols);
  ms.y[0] = y;
  ms.start[0] = 0;
  for (int i = 1; i <= kMaxFused; ++i) ms.start[i] = rows;
  ms.gain[0] = gain0;
  ms.gain[1] = gain1;
  ms.exc_off = exc_off;
  ms.exc = exc;
  ms.rot_signs = rot.signs;
  ms.rot_q = rot.q;
  ms.rot_m = rot.m;
  ms.rot_logk = rot.logk;
  ms.rot_scale = rot.scale;
  return launch_set(ms, 1, mode, rows, cols, x, batch, st);
}

}  // namespace lvq

using namespace lvq;

extern "C" int lvq_gemv(const void* blob, int rows, int cols, const uint16_t* x, float* y,
                        int batch, void* stream) {
  return single_gemv(blob, rows, cols, x, y, batch, stream, kSingle);
}

extern "C" int lvq_gemv_direct(const void* blob, int rows, int cols, const uint16_t* x, float* y,
                               int batch, void* stream) {
  return single_gemv(blob, rows, cols, x, y, batch, stream, kDirect);
}

extern "C" int lvq_gemv_onehot(const void* blob, int rows, int cols, const uint16_t* x, float* y,
                               int batch, void* stream) {
  return single_gemv(blob, rows, cols, x, y, batch, stream, kOneHot);
}

extern "C" int lvq_gemv_lp2(const void* blob, int rows, int cols, const uint16_t* x, float* y,
                            int batch, void* stream) {
  return single_gemv(blob, rows, cols, x, y, batch, stream, kLp2);
}

extern "C" int lvq_gemv_rotated(const void* blob, int rows, int cols, const uint32_t* sign_words,
                                const float* q, int m, const uint16_t* x, float* y, int batch,
                                void* stream) {
  if (m < 1 || m > 32 || cols < 24 || cols % m) return cols < 0 ? LVQ_E_SHAPE : LVQ_E_SHAPE;
  const int k = cols / m;
  if (k & (k - 1)) return LVQ_E_SHAPE;
  RotArgs rot;
  while ((1 << rot.logk) < k) ++rot.logk;
  if (rot.logk > 15) return LVQ_E_SHAPE;
  if (!aligned16(sign_words) || !aligned16(q)) return LVQ_E_ALIGN;
  rot.signs = sign_words;
  rot.q = q;
  rot.m = m;
  rot.scale = (float)(1.0 / __builtin_sqrt((double)k));
  return single_gemv(blob, rows, cols, x, y, batch, stream, kRot, 1.f, 1.f, rot);
}

extern "C" int lvq_gemv_lp2x(const void* blob, int rows, int cols, size_t n_exceptions,
                             const uint16_t* x, float* y, int batch, void* stream) {
  // without side-channel blocks the blob reads as plain LP2
  if (n_exceptions == 0 || rows <= 0 || cols < 24)
    return single_gemv(blob, rows, cols, x, y, batch, stream, kLp2);
  if (!blob) return LVQ_E_NULL;
  const uint8_t* b = (const uint8_t*)blob;
  const Lp2xSections sx = lp2x_sections((size_t)rows, (size_t)cols, n_exceptions);
  return single_gemv(blob, rows, cols, x, y, batch, stream, kLp2x, 1.f, 1.f, RotArgs(),
                     (const uint32_t*)(b + sx.exc_off), (const uint4*)(b + sx.exc));
}

extern "C" int lvq_gemv_gain(const void* blob, int rows, int cols, float gain0, float gain1,
                             const uint16_t* x, float* y, int batch, void* stream) {
  return single_gemv(blob, rows, cols, x, y, batch, stream, kGain, gain0, gain1);
}

extern "C" int lvq_gemv_noweights(const void* blob, int rows, int cols, const uint16_t* x,
                                  float* y, int batch, void* stream) {
  return single_gemv(blob, rows, cols, x, y, batch, stream, kNoWeights);
}

extern "C" int lvq_gemv_fused(int n, const void* const* blobs, const int* rows, int cols,
                              const uint16_t* x, float* const* y, int batch, void* stream) {
  if (n < 1 || n > kMaxFused) return LVQ_E_SHAPE;
  if (!blobs || !rows || !y) return LVQ_E_NULL;
  if (cols < 0) return LVQ_E_SHAPE;
  int e = check_batch(batch);
  if (e) return e;
  if ((long long)batch * cols > 65536) return LVQ_E_SHAPE;
  if (cols && !x) return LVQ_E_NULL;
  if (!aligned16(x)) return LVQ_E_ALIGN;
  MatSet ms = {};
  long long total = 0;
  for (int m = 0; m < n; ++m) {
    if (rows[m] < 0) return LVQ_E_SHAPE;
    if (!blobs[m] || !y[m]) return LVQ_E_NULL;
    if (!aligned16(blobs[m]) || !aligned16(y[m])) return LVQ_E_ALIGN;
    ms.v[m] = leech_view(blobs[m], (size_t)rows[m], (size_t)cols);
    ms.y[m] = y[m];
    ms.start[m] = (int)total;
    total += rows[m];
  }
  if (total > 0x7FFFFFFF) return LVQ_E_SHAPE;
  for (int m = n; m <= kMaxFused; ++m) ms.start[m] = (int)total;
  for (int m = n; m < kMaxFused; ++m) { ms.v[m] = ms.v[0]; ms.y[m] = ms.y[0]; }
  hipStream_t st = (hipStream_t)stream;
  if (total == 0) return LVQ_OK;
  if (cols == 0) {
    for (int m = 0; m < n; ++m) {
      const int ze = zero_output(y[m], (size_t)batch * rows[m], st);
      if (ze) return ze;
    }
    return LVQ_OK;
  }
  return launch_set(ms, n, kFused, (int)total, cols, x, batch, st);
}

extern "C" int lvq_decode(const void* blob, int rows, int cols, int8_t* coords_out,
                          void* stream) {
  if (rows < 0 || cols < 0) return LVQ_E_SHAPE;
  if (!blob || !coords_out) return LVQ_E_NULL;
  if (!aligned16(blob) || !aligned16(coords_out)) return LVQ_E_ALIGN;
  const size_t nblocks = (size_t)rows * (size_t)(cols / 24);
  if (!nblocks) return LVQ_OK;
  const LeechView v = leech_view(blob, (size_t)rows, (size_t)cols);
  clear_hip_error();
  hipLaunchKernelGGL(leech_decode_kernel, dim3((unsigned)((nblocks + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream, v, nblocks, coords_out);
  return launch_status();
}

// The launch a Leech GEMV entry point would make, without making it (see
// include/lvq.h): the launch path runs with a thread-local record in place of
// the launch, on fake 16-byte-aligned addresses that are never dereferenced.
extern "C" int lvq_gemv_launch_info(int kind, int rows, int cols, int batch, int m,
                                    int* info_out) {
  if (!info_out) return LVQ_E_NULL;
  if (rows < 1 || cols < 24) return LVQ_E_SHAPE;
  static const int modes[] = {kSingle, kRot, kDirect, kOneHot, kLp2, kGain, kNoWeights};
  if (kind < 0 || kind >= (int)(sizeof(modes) / sizeof(modes[0]))) return LVQ_E_SHAPE;
  LaunchInfo info = {0, 0, 0, 0, 0};
  t_dry_run = &info;
  const uintptr_t fake = (uintptr_t)1 << 30;
  const void* blob = (const void*)fake;
  const uint16_t* x = (const uint16_t*)fake;
  float* y = (float*)fake;
  int e;
  if (modes[kind] == kRot) {
    e = lvq_gemv_rotated(blob, rows, cols, (const uint32_t*)fake, m > 1 ? (const float*)fake : nullptr,
                         m, x, y, batch, nullptr);
  } else {
    e = single_gemv(blob, rows, cols, x, y, batch, nullptr, modes[kind]);
  }
  t_dry_run = nullptr;
  if (e) return e;
  info_out[0] = info.threads;
  info_out[1] = info.workgroups;
  info_out[2] = info.blocks_per_lane;
  info_out[3] = info.ring;
  info_out[4] = info.lds_bytes;
  return LVQ_OK;
}
