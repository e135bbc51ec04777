// Fused Leech-lattice dequantize-plus-matvec for gfx950 (lvq_gemv, lvq_decode).
//
// Source: arXiv 2609.02652, section 1, contribution C1: a fused kernel reads
// the unfolded layout with shifts, masks and a predicated table lookup, the
// same instruction sequence on every lane whatever the class, and the
// combinatorial index is never decoded inside the matvec.  The Tetra summary
// (arXiv 2609.35465, section 5.1) adds the epilogue: apply the row scale, then
// add the unquantized tail.
//
// gfx950 design.  One wave64 owns one row at a time (rows are grid-strided
// over all waves).  Lane l takes blocks l, l + 64, ... of the row, so every
// load instruction of a wave reads one contiguous run of the row's code words
// (12 bytes per lane) and class ids (2 bytes per lane).  x is staged in LDS
// once per workgroup in "pair order": for block b, code word w and view v the
// 32-bit pair (x[24b + 8w + v], x[24b + 8w + v + 4]), so one ds_read_b128
// feeds the four views of a code word.  The class table is staged in LDS as
// 8-byte byte-LUTs.  Per coordinate pair the decode is
//     rotate (v_alignbit), mask (v_and), byte LUT (v_perm)
// giving two signed magnitudes as exact fp16 subnormals (value * 2^-24), and
// one v_dot2_f32_f16 multiplies them with the x pair into an fp32
// accumulator; the 2^24 is folded into the row scale.  No MFMA: at batch 1
// this is a stream over HBM.  The wave reduction is a fixed butterfly, so the
// result does not depend on timing.

#include "common.h"
#include "layout.h"

namespace lvq {

constexpr int kGemvThreads = 256;
constexpr int kWavesPerWg = kGemvThreads / kWave;
constexpr int kUnroll = 4;  // blocks per lane loaded before they are decoded

struct LeechView {
  const uint64_t* table;
  const uint32_t* codes;
  const uint16_t* cls;
  const uint16_t* scale;
  const uint16_t* tail;
};

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

// LDS layout (dynamic): lut uint2[302] | xpair uint32[B][nb*12] | xtail fp16 [B][24]
template <int B>
__global__ void __launch_bounds__(kGemvThreads)
leech_gemv_kernel(LeechView v, int rows, int nb, int tau, int cols, const uint16_t* __restrict__ x,
                  float* __restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint2* lut = (uint2*)smem;
  uint32_t* xp = (uint32_t*)(smem + LVQ_NUM_CLASSES * 8);
  const int npair = nb * 12;
  uint16_t* xt = (uint16_t*)(xp + B * npair);

  const int tid = threadIdx.x;
  for (int c = tid; c < LVQ_NUM_CLASSES; c += kGemvThreads) lut[c] = leech_lut(v.table[c]);
  // stage x: one thread per group of 8 columns (one code word), 4 pairs out
  for (int bb = 0; bb < B; ++bb) {
    const uint16_t* xb = x + (size_t)bb * cols;
    for (int q = tid; q < nb * 3; q += kGemvThreads) {
      const uint16_t* s = xb + 8 * q;
      uint32_t p[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) p[k] = (uint32_t)s[k] | ((uint32_t)s[k + 4] << 16);
      *(uint4*)(xp + bb * npair + 4 * q) = make_uint4(p[0], p[1], p[2], p[3]);
    }
    for (int t = tid; t < tau; t += kGemvThreads) xt[bb * 24 + t] = xb[24 * nb + t];
  }
  __syncthreads();

  const int lane = tid & (kWave - 1);
  const int wave = blockIdx.x * kWavesPerWg + tid / kWave;
  const int nwaves = gridDim.x * kWavesPerWg;
  const int iters = (nb + kWave - 1) / kWave;

  for (int r = wave; r < rows; r += nwaves) {
    float acc[B][2];
#pragma unroll
    for (int bb = 0; bb < B; ++bb) acc[bb][0] = acc[bb][1] = 0.f;
    const uint32_t* crow = v.codes + (size_t)r * nb * 3;
    const uint16_t* clsrow = v.cls + (size_t)r * nb;
    for (int t0 = 0; t0 < iters; t0 += kUnroll) {
      uint32_t w[kUnroll][3];
      uint32_t c[kUnroll];
      int kk[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int k = (t0 + u) * kWave + lane;
        const bool ok = k < nb;
        kk[u] = ok ? k : 0;
        if (ok) {
          w[u][0] = crow[3 * k + 0];
          w[u][1] = crow[3 * k + 1];
          w[u][2] = crow[3 * k + 2];
          c[u] = min((uint32_t)clsrow[k], (uint32_t)(LVQ_NUM_CLASSES - 1));
        } else {
          w[u][0] = w[u][1] = w[u][2] = kZeroWord;  // origin block: decodes to +0
          c[u] = 0u;
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const uint2 l = lut[c[u]];
#pragma unroll
        for (int wi = 0; wi < 3; ++wi) {
          uint32_t d[4];
#pragma unroll
          for (int vi = 0; vi < 4; ++vi) d[vi] = leech_pair(w[u][wi], vi, l.x, l.y);
#pragma unroll
          for (int bb = 0; bb < B; ++bb) {
            const uint4 xq = *(const uint4*)(xp + bb * npair + 12 * kk[u] + 4 * wi);
            acc[bb][wi & 1] = dot2(d[0], xq.x, acc[bb][wi & 1]);
            acc[bb][wi & 1] = dot2(d[1], xq.y, acc[bb][wi & 1]);
            acc[bb][wi & 1] = dot2(d[2], xq.z, acc[bb][wi & 1]);
            acc[bb][wi & 1] = dot2(d[3], xq.w, acc[bb][wi & 1]);
          }
        }
      }
    }
    // epilogue: scale (with the 2^24 of the subnormal encoding), then the tail
    const float s = half_bits_to_float(v.scale[r]) * 16777216.0f;
    const uint16_t tv = lane < tau ? v.tail[(size_t)r * tau + lane] : (uint16_t)0;
#pragma unroll
    for (int bb = 0; bb < B; ++bb) {
      float part = (acc[bb][0] + acc[bb][1]) * s;
      if (lane < tau) part += half_bits_to_float(tv) * half_bits_to_float(xt[bb * 24 + lane]);
      const float tot = wave_sum(part);
      if (lane == 0) y[(size_t)bb * rows + r] = tot;
    }
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
      vals[8 * wi + vi] = (int8_t)((p & 0x8000u) ? -lo : lo);
      vals[8 * wi + vi + 4] = (int8_t)((p & 0x80000000u) ? -hi : hi);
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

int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

size_t device_lds_bytes() {
  static size_t cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 65536;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
        n <= 0)
      n = 65536;
    cached[dev] = (size_t)n;
  }
  return cached[dev];
}

int zero_output(float* y, size_t n, hipStream_t st) {
  if (!n) return LVQ_OK;
  clear_hip_error();
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, y, n);
  return launch_status();
}

template <int B>
int launch_leech(const LeechView& v, int rows, int cols, const uint16_t* x, float* y,
                 hipStream_t st) {
  const int nb = cols / 24, tau = cols % 24;
  const size_t lds = (size_t)LVQ_NUM_CLASSES * 8 + (size_t)B * nb * 48 + (size_t)B * 24 * 2;
  if (lds > device_lds_bytes()) return LVQ_E_SHAPE;
  const int waves_needed = rows;
  int wgs = (waves_needed + kWavesPerWg - 1) / kWavesPerWg;
  const int cap = 2 * device_cus();
  if (wgs > cap) wgs = cap;
  clear_hip_error();
  hipLaunchKernelGGL(leech_gemv_kernel<B>, dim3(wgs), dim3(kGemvThreads), lds, st, v, rows, nb,
                     tau, cols, x, y);
  return launch_status();
}

}  // namespace lvq

using namespace lvq;

extern "C" int lvq_gemv(const void* blob, int rows, int cols, const uint16_t* x, float* y,
                        int batch, void* stream) {
  if (rows < 0 || cols < 0) return LVQ_E_SHAPE;
  int e = check_batch(batch);
  if (e) return e;
  if (!blob || !y || (cols && !x)) return LVQ_E_NULL;
  if (!aligned16(blob) || !aligned16(x) || !aligned16(y)) return LVQ_E_ALIGN;
  if ((long long)batch * cols > 65536) return LVQ_E_SHAPE;
  hipStream_t st = (hipStream_t)stream;
  if (rows == 0) return LVQ_OK;
  if (cols == 0) return zero_output(y, (size_t)batch * rows, st);
  const LeechView v = leech_view(blob, (size_t)rows, (size_t)cols);
  switch (batch) {
    case 1: return launch_leech<1>(v, rows, cols, x, y, st);
    case 2: return launch_leech<2>(v, rows, cols, x, y, st);
    case 3: return launch_leech<3>(v, rows, cols, x, y, st);
    default: return launch_leech<4>(v, rows, cols, x, y, st);
  }
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
