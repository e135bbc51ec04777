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
// gfx950 design.  A workgroup owns 16 rows; its 256 threads are 16 rows x 16
// column slices (slice j takes groups j, j+16, ...), so a wave instruction
// reads four 64-byte runs of a code row; neighbouring 16-row tiles are mapped
// to workgroups on the same XCD so each 128-byte line is fetched once per L2.
// Bits are never shifted into place: a mask keeps bit 2c (plane 0) or 2c+1
// (plane 1) of the columns c and c+8 of a word, and that masked word, read as
// two fp16 subnormals (2^(2c) or 2^(2c+1) times 2^-24), goes straight into
// v_dot2_f32_f16 against the pre-paired x; columns 5..7 use the word shifted
// by 10.  Ten fp32 accumulators (2 planes x 5 power-of-two scales) are rescaled
// exactly at the end of each group.  The 16 slice partials of a row are summed
// in LDS in a fixed order.

#include "common.h"

namespace lvq {

constexpr int kBpdqThreads = 256;
constexpr int kBpdqRows = 16;
constexpr int kBpdqSlices = 16;

template <int B>
__global__ void __launch_bounds__(kBpdqThreads)
bpdq_gemv_kernel(const uint32_t* __restrict__ codes, const uint16_t* __restrict__ coeffs,
                 int rows, int cols, const uint16_t* __restrict__ x, float* __restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int nwords = cols / 16, G = cols / 256;
  uint32_t* xp = (uint32_t*)smem;                    // [B][nwords*8] pairs
  float* gsum = (float*)(xp + (size_t)B * nwords * 8);  // [B][G]
  float* red = gsum + B * G;                          // [16 slices][16 rows][B]

  const int tid = threadIdx.x;
  for (int i = tid; i < B * nwords; i += kBpdqThreads) {
    const int bb = i / nwords, wi = i - bb * nwords;
    const uint16_t* s = x + (size_t)bb * cols + 16 * wi;
    uint32_t p[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) p[c] = (uint32_t)s[c] | ((uint32_t)s[c + 8] << 16);
    uint4* d = (uint4*)(xp + (size_t)bb * nwords * 8 + 8 * wi);
    d[0] = make_uint4(p[0], p[1], p[2], p[3]);
    d[1] = make_uint4(p[4], p[5], p[6], p[7]);
  }
  for (int i = tid; i < B * G; i += kBpdqThreads) {
    const int bb = i / G, g = i - bb * G;
    const uint16_t* s = x + (size_t)bb * cols + 256 * g;
    float a = 0.f;
    for (int c = 0; c < 256; ++c) a += (float)__builtin_bit_cast(_Float16, s[c]);
    gsum[i] = a;
  }
  __syncthreads();

  const int ntiles = (rows + kBpdqRows - 1) / kBpdqRows;
  int tile = blockIdx.x;
  if ((ntiles & 7) == 0) tile = (blockIdx.x & 7) * (ntiles >> 3) + (blockIdx.x >> 3);
  const int ir = tid % kBpdqRows, j = tid / kBpdqRows;
  const int r = tile * kBpdqRows + ir;
  float part[B];
#pragma unroll
  for (int bb = 0; bb < B; ++bb) part[bb] = 0.f;
  if (r < rows) {
    for (int g = j; g < G; g += kBpdqSlices) {
      float a0[B][5], a1[B][5];
#pragma unroll
      for (int bb = 0; bb < B; ++bb)
#pragma unroll
        for (int c = 0; c < 5; ++c) a0[bb][c] = a1[bb][c] = 0.f;
      const uint32_t* cw = codes + (size_t)(16 * g) * rows + r;
#pragma unroll 4
      for (int i = 0; i < 16; ++i) {
        const uint32_t u = cw[(size_t)i * rows];
        const uint32_t u10 = u >> 10;
#pragma unroll
        for (int bb = 0; bb < B; ++bb) {
          const uint4* xq = (const uint4*)(xp + (size_t)bb * nwords * 8 + 8 * (16 * g + i));
          const uint4 xa = xq[0], xb = xq[1];
          const uint32_t xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
          for (int c = 0; c < 5; ++c) {
            a0[bb][c] = dot2(u & (0x00010001u << (2 * c)), xv[c], a0[bb][c]);
            a1[bb][c] = dot2(u & (0x00020002u << (2 * c)), xv[c], a1[bb][c]);
          }
#pragma unroll
          for (int c = 0; c < 3; ++c) {
            a0[bb][c] = dot2(u10 & (0x00010001u << (2 * c)), xv[c + 5], a0[bb][c]);
            a1[bb][c] = dot2(u10 & (0x00020002u << (2 * c)), xv[c + 5], a1[bb][c]);
          }
        }
      }
      const float c0 = (float)__builtin_bit_cast(_Float16, coeffs[((size_t)g * 3 + 0) * rows + r]);
      const float c1 = (float)__builtin_bit_cast(_Float16, coeffs[((size_t)g * 3 + 1) * rows + r]);
      const float c2 = (float)__builtin_bit_cast(_Float16, coeffs[((size_t)g * 3 + 2) * rows + r]);
#pragma unroll
      for (int bb = 0; bb < B; ++bb) {
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int c = 0; c < 5; ++c) {
          const float sc = (float)(1u << (24 - 2 * c));  // exact powers of two
          s0 += a0[bb][c] * sc;
          s1 += a1[bb][c] * (sc * 0.5f);
        }
        part[bb] += c0 * s0 + c1 * s1 + c2 * gsum[bb * G + g];
      }
    }
  }
#pragma unroll
  for (int bb = 0; bb < B; ++bb) red[(j * kBpdqRows + ir) * B + bb] = part[bb];
  __syncthreads();
  if (j == 0 && r < rows) {
#pragma unroll
    for (int bb = 0; bb < B; ++bb) {
      float s = 0.f;
      for (int jj = 0; jj < kBpdqSlices; ++jj) s += red[(jj * kBpdqRows + ir) * B + bb];
      y[(size_t)bb * rows + r] = s;
    }
  }
}

int zero_output(float* y, size_t n, hipStream_t st);

template <int B>
int launch_bpdq(const uint32_t* codes, const uint16_t* coeffs, int rows, int cols,
                const uint16_t* x, float* y, hipStream_t st) {
  const size_t lds = (size_t)B * cols * 2 + (size_t)B * (cols / 256) * 4 +
                     (size_t)kBpdqSlices * kBpdqRows * B * 4;
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
