// Dense fp16 control matvec (fp16_gemv).
//
// The control arm of arXiv 2609.02652 (section 1, contribution C2, and the
// performance-model paragraph of the related-work section): the same y = W x
// over an fp16 matrix; its bandwidth is the "byte bound" the lattice kernels
// are measured against.
//
// gfx950 design: one wave64 per row (rows grid-strided), each lane streams
// 16-byte chunks so a wave instruction reads 1 KiB of the row; x is staged in
// LDS once per workgroup; v_dot2_f32_f16 with fp32 accumulation; fixed
// butterfly reduction.

#include "common.h"

namespace lvq {

constexpr int kDenseThreads = 256;

template <int B>
__global__ void __launch_bounds__(kDenseThreads)
fp16_gemv_kernel(const uint16_t* __restrict__ W, int rows, int cols,
                 const uint16_t* __restrict__ x, float* __restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint4* xs = (uint4*)smem;  // [B][cols/8]
  const int n8 = cols / 8;
  const int tid = threadIdx.x;
  for (int i = tid; i < B * n8; i += kDenseThreads) {
    const int bb = i / n8, q = i - bb * n8;
    xs[i] = *(const uint4*)(x + (size_t)bb * cols + 8 * q);
  }
  __syncthreads();
  const int lane = tid & (kWave - 1);
  const int wave = blockIdx.x * (kDenseThreads / kWave) + tid / kWave;
  const int nwaves = gridDim.x * (kDenseThreads / kWave);
  for (int r = wave; r < rows; r += nwaves) {
    const uint4* wrow = (const uint4*)(W + (size_t)r * cols);
    float acc[B][2];
#pragma unroll
    for (int bb = 0; bb < B; ++bb) acc[bb][0] = acc[bb][1] = 0.f;
    int q = lane;
    for (; q + kWave < n8; q += 2 * kWave) {
      const uint4 a = wrow[q];
      const uint4 b = wrow[q + kWave];
#pragma unroll
      for (int bb = 0; bb < B; ++bb) {
        const uint4 xa = xs[bb * n8 + q];
        const uint4 xb = xs[bb * n8 + q + kWave];
        acc[bb][0] = dot2(a.x, xa.x, acc[bb][0]);
        acc[bb][1] = dot2(b.x, xb.x, acc[bb][1]);
        acc[bb][0] = dot2(a.y, xa.y, acc[bb][0]);
        acc[bb][1] = dot2(b.y, xb.y, acc[bb][1]);
        acc[bb][0] = dot2(a.z, xa.z, acc[bb][0]);
        acc[bb][1] = dot2(b.z, xb.z, acc[bb][1]);
        acc[bb][0] = dot2(a.w, xa.w, acc[bb][0]);
        acc[bb][1] = dot2(b.w, xb.w, acc[bb][1]);
      }
    }
    if (q < n8) {
      const uint4 a = wrow[q];
#pragma unroll
      for (int bb = 0; bb < B; ++bb) {
        const uint4 xa = xs[bb * n8 + q];
        acc[bb][0] = dot2(a.x, xa.x, acc[bb][0]);
        acc[bb][0] = dot2(a.y, xa.y, acc[bb][0]);
        acc[bb][0] = dot2(a.z, xa.z, acc[bb][0]);
        acc[bb][0] = dot2(a.w, xa.w, acc[bb][0]);
      }
    }
#pragma unroll
    for (int bb = 0; bb < B; ++bb) {
      const float tot = wave_sum_lane63(acc[bb][0] + acc[bb][1]);
      if (lane == kWave - 1) y[(size_t)bb * rows + r] = tot;
    }
  }
}

int zero_output(float* y, size_t n, hipStream_t st);

template <int B>
int launch_fp16(const uint16_t* W, int rows, int cols, const uint16_t* x, float* y,
                hipStream_t st) {
  const size_t lds = (size_t)B * cols * 2;
  if (lds > device_lds_bytes()) return LVQ_E_SHAPE;
  int wgs = (rows + 3) / 4;
  const int cap = 2 * device_cus();
  if (wgs > cap) wgs = cap;
  clear_hip_error();
  hipLaunchKernelGGL(fp16_gemv_kernel<B>, dim3(wgs), dim3(kDenseThreads), lds, st, W, rows, cols,
                     x, y);
  return launch_status();
}

}  // namespace lvq

using namespace lvq;

extern "C" int fp16_gemv(const uint16_t* W, int rows, int cols, const uint16_t* x, float* y,
                         int batch, void* stream) {
  if (rows < 0 || cols < 0 || cols % 8) return LVQ_E_SHAPE;
  int e = check_batch(batch);
  if (e) return e;
  if (!y || (rows && cols && (!W || !x))) return LVQ_E_NULL;
  if (!aligned16(W) || !aligned16(x) || !aligned16(y)) return LVQ_E_ALIGN;
  if ((long long)batch * cols > 65536) return LVQ_E_SHAPE;
  hipStream_t st = (hipStream_t)stream;
  if (rows == 0) return LVQ_OK;
  if (cols == 0) return zero_output(y, (size_t)batch * rows, st);
  switch (batch) {
    case 1: return launch_fp16<1>(W, rows, cols, x, y, st);
    case 2: return launch_fp16<2>(W, rows, cols, x, y, st);
    case 3: return launch_fp16<3>(W, rows, cols, x, y, st);
    default: return launch_fp16<4>(W, rows, cols, x, y, st);
  }
}
