// BPDQ bit-plane matvec (bpdq_gemv), the 2-bit comparison arm.
//
// Source: model card "Qwen3-8B - 2-bit BPDQ (packed)".  Section Format:
// w[r,c] = c0 * bit_0 + c1 * bit_1 + c2 per (group of 256 columns, row); the
// "Elsewhere" layout keeps 16 columns per 32-bit word (2 bits each, the two
// planes of a column interleaved into one code) with out_features innermost.
// Section Kernels: the multiply-without-dequantising form, per group
// c0 * S0 + c1 * S1 + c2 * sum(x), with S_i the sum of the activations that
// plane i selects, and a deterministic split over K.
//
// gfx950 design.  The layout puts consecutive rows in consecutive words, so a
// lane is a (row, quarter group) pair, a quarter being 4 consecutive code
// words (64 columns): a workgroup covers 16 rows x SLOTS quarters, every load
// instruction of a wave reads four 64-byte runs (16 rows of 4 quarters), and
// a lane walks its quarters SLOTS apart, the next quarter's words requested
// while the current one is summed.  The form is linear, so each lane applies
// its group's coefficients to its own quarter: c0 * S0q + c1 * S1q + c2 * Xq,
// with Xq the sum of x over the quarter.  Bits are never shifted into place:
// a mask keeps bit 2c (plane 0) or 2c+1 (plane 1) of the columns c and c+8
// of a word, and that masked word, read as two fp16 subnormals (2^(2c) or
// 2^(2c+1) times 2^-24), goes straight into v_dot2_f32_f16 against the x
// pair (x_c, x_{c+8}); columns 5..7 use the word shifted right by 10.  Ten
// fp32 accumulators per batch row (2 planes x 5 powers of two) are rescaled
// exactly at the end of each quarter.  x pairs and quarter sums are staged in
// LDS once per workgroup, the x words requested before the code words so the
// copy runs under their latency; the SLOTS partials of a row are summed by
// shuffles inside a wave and then over the waves in LDS, always in the same
// order.  Neighbouring 16-row tiles share 128-byte lines and are mapped to
// workgroups on the same XCD.

#include "common.h"

namespace lvq {

constexpr int kBpdqRows = 16;
constexpr int kBpdqUnit = 4;  // code words per lane unit: a quarter group

// dot2(a, b, 0.f) as v_dot2_f32_f16 with an inline zero accumulator: the same
// sum of two products; the compiler emits a move of 0 and the tied v_dot2c,
// one instruction more for each of the 10 B accumulators of every quarter.
__device__ __forceinline__ float dot2_first(uint32_t a, uint32_t b) {
  float d;
  asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(d) : "v"(a), "v"(b));
  return d;
}

template <int B, int SLOTS>
__global__ void __launch_bounds__(kBpdqRows * SLOTS)
bpdq_gemv_kernel(const uint32_t* __restrict__ codes, const uint16_t* __restrict__ coeffs,
                 int rows, int cols, const uint16_t* __restrict__ x, float* __restrict__ y) {
  constexpr int U = kBpdqUnit;
  constexpr int kThreads = kBpdqRows * SLOTS, kWaves = kThreads / kWave;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int nwords = cols / 16, nunits = nwords / U;
  // x pairs [quarter][batch row][4 words][8 pairs] and quarter sums
  // [quarter][batch row]: the batch stride is a constant, so the reads of a
  // quarter take immediate offsets from one base.  Each quarter is padded by
  // 8 words: a wave's four slots read four consecutive quarters, which
  // unpadded would sit B x 512 bytes apart, on the same banks.
  constexpr int kQS = B * U * 8 + 8;  // 32-bit words per quarter
  uint32_t* xp = (uint32_t*)smem;
  float* xu = (float*)(xp + (size_t)nunits * kQS);
  float* red = xu + (size_t)B * nunits;                    // [waves][16 rows][B]

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int ntiles = (rows + kBpdqRows - 1) / kBpdqRows;
  int tile = blockIdx.x;
  if ((ntiles & 7) == 0) tile = (blockIdx.x & 7) * (ntiles >> 3) + (blockIdx.x >> 3);
  const int ir = lane & (kBpdqRows - 1);
  const int slot = wave * (kWave / kBpdqRows) + (lane >> 4);
  const int r = tile * kBpdqRows + ir;
  const int rr = r < rows ? r : rows - 1;  // loads stay in bounds; the row is dropped at the end

  // 1. this thread's first B x words (16 columns each), requested first: the
  //    copy into LDS is what the barrier waits for.  A word past the end
  //    reads word 0 and stores nothing.
  const int nst = B * nwords;
  uint4 xlo[B], xhi[B];
#pragma unroll
  for (int k = 0; k < B; ++k) {
    const int i = tid + k * kThreads;
    const uint4* xs = (const uint4*)(x + (size_t)(i < nst ? i : 0) * 16);
    xlo[k] = xs[0];  // columns 0..7
    xhi[k] = xs[1];  // columns 8..15
  }

  // 2. this lane's first unit: code words and coefficients.  Raw buffer
  //    loads: the lane's offset is computed once per unit and the word j and
  //    coefficient i steps are scalar offsets, so no vector instruction goes
  //    to 64-bit addressing.  A unit past the row's end gets an offset past
  //    the buffer, which the hardware answers with zeros and no request; the
  //    loads stay branch-free, so every later wait counts exactly them.
  uint32_t u[U];
  uint16_t cf[3];
  const uint32_t code_bytes = (uint32_t)nwords * rows * 4;
  const auto rcodes = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(codes), (short)0,
                                                        (int)code_bytes, 0x00020000);
  const auto rcoef = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(coeffs), (short)0,
                                                       (int)((uint32_t)(cols / 256) * 3 * rows * 2),
                                                       0x00020000);
  auto load_unit = [&](int n) {
    const bool ok = n < nunits;
    const int vo = ok ? (U * n * rows + rr) * 4 : (int)code_bytes;
#pragma unroll
    for (int j = 0; j < U; ++j)
      u[j] = __builtin_amdgcn_raw_buffer_load_b32(rcodes, vo, j * rows * 4, 2);
    const int vc = ok ? ((n * U / 16) * 3 * rows + rr) * 2 : (int)code_bytes;
#pragma unroll
    for (int i = 0; i < 3; ++i) cf[i] = __builtin_amdgcn_raw_buffer_load_b16(rcoef, vc, i * rows * 2, 0);
  };
  load_unit(slot);

  // 3. x pairs (x_c, x_{c+8}) of each code word, and the sum of x over each
  //    quarter, into LDS.  The thread that pairs a word also sums its 16
  //    values (v_dot2 against (1, 1), fixed order); the 4 words of a quarter
  //    sit in the 4 lanes of a quad and are added by two quad swaps, the same
  //    operands on every lane.
  auto stage = [&](int i, uint4 lo, uint4 hi) {
    const uint32_t a[4] = {lo.x, lo.y, lo.z, lo.w}, b[4] = {hi.x, hi.y, hi.z, hi.w};
    uint32_t p[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      p[2 * k] = __builtin_amdgcn_perm(b[k], a[k], 0x05040100u);      // x_{2k}, x_{2k+8}
      p[2 * k + 1] = __builtin_amdgcn_perm(b[k], a[k], 0x07060302u);  // x_{2k+1}, x_{2k+9}
    }
    constexpr uint32_t kOnes = 0x3C003C00u;  // (1.0, 1.0)
    float s = (dot2(a[1], kOnes, dot2(a[0], kOnes, 0.f)) +
               dot2(a[3], kOnes, dot2(a[2], kOnes, 0.f))) +
              (dot2(b[1], kOnes, dot2(b[0], kOnes, 0.f)) +
               dot2(b[3], kOnes, dot2(b[2], kOnes, 0.f)));
    s = dpp_add<0x4E, 0xF>(dpp_add<0xB1, 0xF>(s));  // quad_perm swaps: the quarter's 4 words
    if (i < nst) {
      int bb = 0;  // word i is word w of batch row bb
#pragma unroll
      for (int k = 1; k < B; ++k) bb += i >= k * nwords;
      const int w = i - bb * nwords, q = w >> 2;
      uint4* d = (uint4*)(xp + (size_t)q * kQS + (bb * U + (w & 3)) * 8);
      d[0] = make_uint4(p[0], p[1], p[2], p[3]);
      d[1] = make_uint4(p[4], p[5], p[6], p[7]);
      if ((w & 3) == 0) xu[q * B + bb] = s;
    }
  };
#pragma unroll
  for (int k = 0; k < B; ++k) stage(tid + k * kThreads, xlo[k], xhi[k]);
  for (int i = tid + B * kThreads; i < nst; i += kThreads) {
    const uint4* xs = (const uint4*)(x + (size_t)i * 16);
    stage(i, xs[0], xs[1]);
  }
  __syncthreads();

  // 4. units of this lane's row.  Per code word the 16 masked operands are
  //    formed once and used by every batch row.
  float acc[B];
#pragma unroll
  for (int bb = 0; bb < B; ++bb) acc[bb] = 0.f;
  for (int n = slot; n < nunits; n += SLOTS) {
    const float c0 = (float)__builtin_bit_cast(_Float16, cf[0]);
    const float c1 = (float)__builtin_bit_cast(_Float16, cf[1]);
    const float c2 = (float)__builtin_bit_cast(_Float16, cf[2]);
    uint32_t w[U];
#pragma unroll
    for (int j = 0; j < U; ++j) w[j] = u[j];
    load_unit(n + SLOTS);  // the next unit, or nothing past the row
    const uint32_t* xq = xp + (size_t)n * kQS;  // this quarter's pairs, batch row 0
    float a0[B][5], a1[B][5];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const uint32_t wj = w[j], w10 = wj >> 10;
      uint32_t m0[8], m1[8];
#pragma unroll
      for (int c = 0; c < 5; ++c) {
        m0[c] = wj & (0x00010001u << (2 * c));
        m1[c] = wj & (0x00020002u << (2 * c));
      }
#pragma unroll
      for (int c = 0; c < 3; ++c) {
        m0[c + 5] = w10 & (0x00010001u << (2 * c));
        m1[c + 5] = w10 & (0x00020002u << (2 * c));
      }
#pragma unroll
      for (int bb = 0; bb < B; ++bb) {
        const uint4* xw = (const uint4*)(xq + (bb * U + j) * 8);
        const uint4 xa = xw[0], xb = xw[1];
        const uint32_t xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int e = c < 5 ? c : c - 5;  // columns 5..7 ride at the powers of 0..2
          if (j == 0 && c < 5) {  // the accumulator's first term
            a0[bb][e] = dot2_first(m0[c], xv[c]);
            a1[bb][e] = dot2_first(m1[c], xv[c]);
          } else {
            a0[bb][e] = dot2(m0[c], xv[c], a0[bb][e]);
            a1[bb][e] = dot2(m1[c], xv[c], a1[bb][e]);
          }
        }
      }
    }
#pragma unroll
    for (int bb = 0; bb < B; ++bb) {
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int e = 0; e < 5; ++e) {
        const float sc = (float)(1u << (24 - 2 * e));  // exact powers of two
        s0 += a0[bb][e] * sc;
        s1 += a1[bb][e] * (sc * 0.5f);
      }
      acc[bb] += c0 * s0 + c1 * s1 + c2 * xu[n * B + bb];
    }
  }

  // 5. fixed-order reduction: the 4 unit slots of a wave, then the waves
#pragma unroll
  for (int bb = 0; bb < B; ++bb) {
    float v = acc[bb];
    v += __shfl_xor(v, 16, kWave);
    v += __shfl_xor(v, 32, kWave);
    if (lane < kBpdqRows) red[(wave * kBpdqRows + ir) * B + bb] = v;
  }
  __syncthreads();
  if (tid < kBpdqRows * B) {
    const int row = tid / B, bb = tid - row * B;
    const int rg = tile * kBpdqRows + row;
    float s = 0.f;
    for (int wv = 0; wv < kWaves; ++wv) s += red[(wv * kBpdqRows + row) * B + bb];
    if (rg < rows) y[(size_t)bb * rows + rg] = s;
  }
}

int zero_output(float* y, size_t n, hipStream_t st);

template <int B, int SLOTS>
int launch_bpdq(const uint32_t* codes, const uint16_t* coeffs, int rows, int cols,
                const uint16_t* x, float* y, hipStream_t st) {
  constexpr int kThreads = kBpdqRows * SLOTS;
  const size_t quarters = cols / (16 * kBpdqUnit);
  const size_t lds = quarters * (B * kBpdqUnit * 8 + 8) * 4 + quarters * B * 4 +
                     (size_t)(kThreads / kWave) * kBpdqRows * B * 4;
  if (lds > device_lds_bytes()) return LVQ_E_SHAPE;
  const int ntiles = (rows + kBpdqRows - 1) / kBpdqRows;
  clear_hip_error();
  hipLaunchKernelGGL((bpdq_gemv_kernel<B, SLOTS>), dim3(ntiles), dim3(kThreads), lds, st, codes,
                     coeffs, rows, cols, x, y);
  return launch_status();
}

// Quarters per workgroup row: each lane should take about two quarters (the
// next one's words requested while the current one is summed), so the most
// slots of 64, 32 and 16 that still give two per lane, else 16.  At 4096
// columns 32 slots (512-thread workgroups, two waves per SIMD), at 12288 64
// slots and three quarters per lane.  Measured over the six shapes of a
// Qwen3-8B layer against whole or half groups per lane and other slot counts:
// within 0.14 us of the best at batch 1 and 0.6 us at batch 4.
template <int B>
int launch_bpdq_batch(const uint32_t* codes, const uint16_t* coeffs, int rows, int cols,
                      const uint16_t* x, float* y, hipStream_t st) {
  const int quarters = cols / 64;
  if (quarters >= 2 * 64) return launch_bpdq<B, 64>(codes, coeffs, rows, cols, x, y, st);
  if (quarters >= 2 * 32) return launch_bpdq<B, 32>(codes, coeffs, rows, cols, x, y, st);
  return launch_bpdq<B, 16>(codes, coeffs, rows, cols, x, y, st);
}

}  // namespace lvq

using namespace lvq;

extern "C" int bpdq_gemv(const uint32_t* codes, const uint16_t* coeffs, int rows, int cols,
                         const uint16_t* x, float* y, int batch, void* stream) {
  if (rows < 0 || cols < 0 || cols % 256) return LVQ_E_SHAPE;
  int e = check_batch(batch);
  if (e) return e;
  if (!y || (rows && cols && (!codes || !coeffs || !x))) return LVQ_E_NULL;
  if (!aligned16(codes) || !aligned16(coeffs) || !aligned16(x) || !aligned16(y)) return LVQ_E_ALIGN;
  if ((long long)batch * cols > 65536) return LVQ_E_SHAPE;
  if ((long long)rows * cols / 4 > INT32_MAX) return LVQ_E_SHAPE;  // 32-bit buffer offsets
  hipStream_t st = (hipStream_t)stream;
  if (rows == 0) return LVQ_OK;
  if (cols == 0) return zero_output(y, (size_t)batch * rows, st);
  switch (batch) {
    case 1: return launch_bpdq_batch<1>(codes, coeffs, rows, cols, x, y, st);
    case 2: return launch_bpdq_batch<2>(codes, coeffs, rows, cols, x, y, st);
    case 3: return launch_bpdq_batch<3>(codes, coeffs, rows, cols, x, y, st);
    default: return launch_bpdq_batch<4>(codes, coeffs, rows, cols, x, y, st);
  }
}
