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
// lane is a (row, quarter group) pair: a 1024-thread workgroup covers 16 rows
// x 64 quarter groups of 64 columns (4 code words each); every load
// instruction of a wave reads four 64-byte runs (16 rows of 4 quarter
// groups).  The form is linear, so each lane applies its group's coefficients
// to its own quarter: c0 * S0q + c1 * S1q + c2 * Xq, with Xq the sum of x over
// the quarter.  Bits are never shifted into place: a mask keeps bit 2c (plane
// 0) or 2c+1 (plane 1) of the columns c and c+8 of a word, and that masked
// word, read as two fp16 subnormals (2^(2c) or 2^(2c+1) times 2^-24), goes
// straight into v_dot2_f32_f16 against the x pair (x_c, x_{c+8}); columns
// 5..7 use the word shifted right by 10.  Ten fp32 accumulators (2 planes x 5
// powers of two) are rescaled exactly at the end of each quarter.  x pairs
// and quarter sums are staged in LDS once per workgroup; the 64 partials of a
// row are summed by shuffles inside a wave and then over the 16 waves in LDS,
// always in the same order.  Neighbouring 16-row tiles share 128-byte lines
// and are mapped to workgroups on the same XCD.

#include "common.h"

namespace lvq {

constexpr int kBpdqThreads = 1024;
constexpr int kBpdqRows = 16;
constexpr int kBpdqWaves = kBpdqThreads / kWave;
constexpr int kBpdqSlices = kBpdqWaves * (kWave / kBpdqRows);  // 64 quarter-group slots

template <int B>
__global__ void __launch_bounds__(kBpdqThreads)
bpdq_gemv_kernel(const uint32_t* __restrict__ codes, const uint16_t* __restrict__ coeffs,
                 int rows, int cols, const uint16_t* __restrict__ x, float* __restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int nwords = cols / 16, Q = cols / 64;
  uint32_t* xp = (uint32_t*)smem;                          // [B][nwords][8] pairs
  float* xq = (float*)(xp + (size_t)B * nwords * 8);       // [B][Q] quarter sums
  float* red = xq + (size_t)B * Q;                         // [16 waves][16 rows][B]

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int ntiles = (rows + kBpdqRows - 1) / kBpdqRows;
  int tile = blockIdx.x;
  if ((ntiles & 7) == 0) tile = (blockIdx.x & 7) * (ntiles >> 3) + (blockIdx.x >> 3);
  const int ir = lane & (kBpdqRows - 1);
  const int slice = wave * (kWave / kBpdqRows) + (lane >> 4);
  const int r = tile * kBpdqRows + ir;
  const int rr = r < rows ? r : rows - 1;  // loads stay in bounds; the row is dropped at the end

  // 1. this lane's first quarter: code words and coefficients, requested first
  uint32_t u[4];
  uint16_t cf[3];
  auto load_q = [&](int q) {
#pragma unroll
    for (int j = 0; j < 4; ++j) u[j] = __builtin_nontemporal_load(codes + (size_t)(4 * q + j) * rows + rr);
    const int g = q >> 2;
#pragma unroll
    for (int i = 0; i < 3; ++i) cf[i] = coeffs[((size_t)g * 3 + i) * rows + rr];
  };
  if (slice < Q) load_q(slice);

  // 2. x pairs (x_c, x_{c+8}) per code word, and quarter sums, in LDS
  for (int i = tid; i < B * nwords; i += kBpdqThreads) {
    const uint4* s = (const uint4*)(x + (size_t)i * 16);  // batch rows are contiguous
    const uint4 lo = s[0], hi = s[1];                      // columns 0..7 and 8..15
    const uint32_t a[4] = {lo.x, lo.y, lo.z, lo.w}, b[4] = {hi.x, hi.y, hi.z, hi.w};
    uint32_t p[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      p[2 * k] = __builtin_amdgcn_perm(b[k], a[k], 0x05040100u);      // x_{2k}, x_{2k+8}
      p[2 * k + 1] = __builtin_amdgcn_perm(b[k], a[k], 0x07060302u);  // x_{2k+1}, x_{2k+9}
    }
    uint4* d = (uint4*)(xp + (size_t)i * 8);
    d[0] = make_uint4(p[0], p[1], p[2], p[3]);
    d[1] = make_uint4(p[4], p[5], p[6], p[7]);
  }
  {
    // 16 threads per quarter (4 columns each), summed in a fixed tree
    const int nq = B * Q;
    for (int base = 0; base < nq * 16; base += kBpdqThreads) {
      const int i = base + tid, q = i >> 4, part = i & 15;
      float s = 0.f;
      if (q < nq) {
        const uint2 v = *(const uint2*)(x + (size_t)q * 64 + 4 * part);
        s = (float)__builtin_bit_cast(_Float16, (uint16_t)v.x) +
            (float)__builtin_bit_cast(_Float16, (uint16_t)(v.x >> 16));
        s += (float)__builtin_bit_cast(_Float16, (uint16_t)v.y) +
             (float)__builtin_bit_cast(_Float16, (uint16_t)(v.y >> 16));
      }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) s += __shfl_xor(s, off, kWave);
      if (q < nq && part == 0) xq[q] = s;
    }
  }
  __syncthreads();

  // 3. quarters of this lane's row
  float acc[B];
#pragma unroll
  for (int bb = 0; bb < B; ++bb) acc[bb] = 0.f;
  for (int q = slice; q < Q; q += kBpdqSlices) {
    const float c0 = (float)__builtin_bit_cast(_Float16, cf[0]);
    const float c1 = (float)__builtin_bit_cast(_Float16, cf[1]);
    const float c2 = (float)__builtin_bit_cast(_Float16, cf[2]);
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = u[j];
    if (q + kBpdqSlices < Q) load_q(q + kBpdqSlices);  // the next quarter, if any
    // one batch row at a time: ten accumulators live, not ten per row
#pragma unroll
    for (int bb = 0; bb < B; ++bb) {
      float a0[5], a1[5];
#pragma unroll
      for (int e = 0; e < 5; ++e) a0[e] = a1[e] = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t wj = w[j], w10 = wj >> 10;
        const uint4* xw = (const uint4*)(xp + ((size_t)bb * nwords + 4 * q + j) * 8);
        const uint4 xa = xw[0], xb = xw[1];
        const uint32_t xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
        for (int c = 0; c < 5; ++c) {
          a0[c] = dot2(wj & (0x00010001u << (2 * c)), xv[c], a0[c]);
          a1[c] = dot2(wj & (0x00020002u << (2 * c)), xv[c], a1[c]);
        }
#pragma unroll
        for (int c = 0; c < 3; ++c) {
          a0[c] = dot2(w10 & (0x00010001u << (2 * c)), xv[c + 5], a0[c]);
          a1[c] = dot2(w10 & (0x00020002u << (2 * c)), xv[c + 5], a1[c]);
        }
      }
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int e = 0; e < 5; ++e) {
        const float sc = (float)(1u << (24 - 2 * e));  // exact powers of two
        s0 += a0[e] * sc;
        s1 += a1[e] * (sc * 0.5f);
      }
      acc[bb] += c0 * s0 + c1 * s1 + c2 * xq[bb * Q + q];
    }
  }

  // 4. fixed-order reduction: the 4 quarter slots of a wave, then 16 waves
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
    for (int wv = 0; wv < kBpdqWaves; ++wv) s += red[(wv * kBpdqRows + row) * B + bb];
    if (rg < rows) y[(size_t)bb * rows + rg] = s;
  }
}

int zero_output(float* y, size_t n, hipStream_t st);

template <int B>
int launch_bpdq(const uint32_t* codes, const uint16_t* coeffs, int rows, int cols,
                const uint16_t* x, float* y, hipStream_t st) {
  const size_t lds = (size_t)B * cols * 2 + (size_t)B * (cols / 64) * 4 +
                     (size_t)kBpdqWaves * kBpdqRows * B * 4;
  if (lds > device_lds_bytes()) return LVQ_E_SHAPE;
  const int ntiles = (rows + kBpdqRows - 1) / kBpdqRows;
  clear_hip_error();
  hipLaunchKernelGGL(bpdq_gemv_kernel<B>, dim3(ntiles), dim3(kBpdqThreads), lds, st, codes, coeffs,
                     rows, cols, x, y);
  return launch_status();
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
  hipStream_t st = (hipStream_t)stream;
  if (rows == 0) return LVQ_OK;
  if (cols == 0) return zero_output(y, (size_t)batch * rows, st);
  switch (batch) {
    case 1: return launch_bpdq<1>(codes, coeffs, rows, cols, x, y, st);
    case 2: return launch_bpdq<2>(codes, coeffs, rows, cols, x, y, st);
    case 3: return launch_bpdq<3>(codes, coeffs, rows, cols, x, y, st);
    default: return launch_bpdq<4>(codes, coeffs, rows, cols, x, y, st);
  }
}
