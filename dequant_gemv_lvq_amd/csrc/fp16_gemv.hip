// Dense fp16 control matvec (fp16_gemv).
//
// The control arm of arXiv 2609.02652 (section 1, contribution C2, and the
// performance-model paragraph of the related-work section): the same y = W x
// over an fp16 matrix; its bandwidth is the "byte bound" the lattice kernels
// are measured against, so it has to stream as close to the hardware's
// achievable read bandwidth as a plain matvec can.
//
// gfx950 design.  One wave64 owns a row at a time (rows grid-strided over the
// waves of up to two 1024-thread workgroups per CU).  A row is cut into items
// of 64 lanes x 8 sixteen-byte chunks (8 KiB; 4 chunks at batch 3-4); lane l
// takes chunks l, l + 64, ... of the item, so each load instruction of the
// wave reads 1 KiB in one run.  Two register sets keep the next item in flight while the
// current one is multiplied, so ~16-32 MiB is requested across the chip at
// any time.  Loads are raw buffer loads (chunks past the row's end read 0);
// x is copied into LDS by buffer loads that write LDS directly.  Products are
// v_dot2_f32_f16 with fp32 accumulation; the row sum is a fixed DPP tree.

#include "common.h"

namespace lvq {

constexpr int kDenseThreads = 1024;
// 16-byte chunks per lane per item: 8 (8 KiB per wave) up to batch 2, 4 at
// batch 3-4, where the x reads and accumulators need the registers
constexpr int dense_chunks(int B) { return B <= 2 ? 8 : 4; }

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t dense_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

template <int CH>
struct DenseItem {
  u32x4_t w[CH];
};

template <int CH>
__device__ __forceinline__ void dense_load(const uint16_t* W, int cols, int r, int g, int lane,
                                           DenseItem<CH>& it) {
  // item g of row r: chunks 64 CH g .. 64 CH (g + 1) - 1 of the row
  const auto rw = dense_rsrc(W + (size_t)r * cols, (uint32_t)cols * 2);
  const int base = g * (kWave * CH);
#pragma unroll
  for (int i = 0; i < CH; ++i)
    it.w[i] = __builtin_bit_cast(
        u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, (base + lane + i * kWave) * 16, 0, 2));
}

template <int B, int CH>
__device__ __forceinline__ void dense_mul(const DenseItem<CH>& it, const uint4* xs, int n8, int g,
                                          int lane, float (&acc)[B][2]) {
  const int base = g * (kWave * CH);
#pragma unroll
  for (int i = 0; i < CH; ++i) {
#pragma unroll
    for (int bb = 0; bb < B; ++bb) {
      const uint4 xq = xs[bb * n8 + base + lane + i * kWave];
      float& a = acc[bb][i & 1];
      a = dot2(it.w[i].x, xq.x, a);
      a = dot2(it.w[i].y, xq.y, a);
      a = dot2(it.w[i].z, xq.z, a);
      a = dot2(it.w[i].w, xq.w, a);
    }
  }
}

template <int B>
__global__ void __launch_bounds__(kDenseThreads)
fp16_gemv_kernel(const uint16_t* __restrict__ W, int rows, int cols, int n8pad,
                 const uint16_t* __restrict__ x, float* __restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint4* xs = (uint4*)smem;  // [B][n8pad] 16-byte chunks of x, zero past cols
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wpb = blockDim.x / kWave;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave = blockIdx.x * wpb + wv;
  const int nwaves = gridDim.x * wpb;
  constexpr int CH = dense_chunks(B);
  const int n8 = cols / 8;
  const int G = (n8 + kWave * CH - 1) / (kWave * CH);
  const int myrows = wave < rows ? (rows - 1 - wave) / nwaves + 1 : 0;
  const int items = myrows * G;

  // x into LDS, 1 KiB (64 chunks) per wave instruction
  for (int bb = 0; bb < B; ++bb) {
    const auto rx = dense_rsrc(x + (size_t)bb * cols, (uint32_t)cols * 2);
    for (int q = wv; q * kWave < n8pad; q += wpb)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (__attribute__((address_space(3))) void*)(xs + (size_t)bb * n8pad + q * kWave), 16,
          lane * 16, q * kWave * 16, 0, 0);
  }
  // the first two items of this wave (a wave with fewer items loads its first
  // item again, so the prologue has no branches)
  DenseItem<CH> ia, ib;
  int ra = wave < rows ? wave : 0, ga = 0;
  int rb = ra, gb = 0;
  if (items > 1) { if (G > 1) gb = 1; else rb = ra + nwaves; }
  dense_load(W, cols, ra, ga, lane, ia);
  dense_load(W, cols, rb, gb, lane, ib);
  __syncthreads();
  if (items == 0) return;

  float acc[B][2];
#pragma unroll
  for (int bb = 0; bb < B; ++bb) acc[bb][0] = acc[bb][1] = 0.f;
  auto finish_row = [&](int r, int g) {
    if (g != G - 1) return;
#pragma unroll
    for (int bb = 0; bb < B; ++bb) {
      const float tot = wave_sum_lane63(acc[bb][0] + acc[bb][1]);
      if (lane == kWave - 1) y[(size_t)bb * rows + r] = tot;
      acc[bb][0] = acc[bb][1] = 0.f;
    }
  };
  auto advance2 = [&](int& r, int& g) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (g + 1 == G) { r += nwaves; g = 0; } else { ++g; }
    }
  };
  int j = 0;
  for (; j + 3 < items; j += 2) {
    dense_mul<B, CH>(ia, xs, n8pad, ga, lane, acc);
    finish_row(ra, ga);
    advance2(ra, ga);
    dense_load(W, cols, ra, ga, lane, ia);
    dense_mul<B, CH>(ib, xs, n8pad, gb, lane, acc);
    finish_row(rb, gb);
    advance2(rb, gb);
    dense_load(W, cols, rb, gb, lane, ib);
  }
  // the last one to three items
  dense_mul<B, CH>(ia, xs, n8pad, ga, lane, acc);
  finish_row(ra, ga);
  if (j + 2 < items) {
    advance2(ra, ga);
    dense_load(W, cols, ra, ga, lane, ia);
  }
  if (j + 1 < items) {
    dense_mul<B, CH>(ib, xs, n8pad, gb, lane, acc);
    finish_row(rb, gb);
  }
  if (j + 2 < items) {
    dense_mul<B, CH>(ia, xs, n8pad, ga, lane, acc);
    finish_row(ra, ga);
  }
}

int zero_output(float* y, size_t n, hipStream_t st);

template <int B>
int launch_fp16(const uint16_t* W, int rows, int cols, const uint16_t* x, float* y,
                hipStream_t st) {
  const int n8 = cols / 8;
  const int per_item = kWave * 8;  // a multiple of every item size and of a 1 KiB copy
  const int n8pad = (n8 + per_item - 1) / per_item * per_item;
  const size_t lds = (size_t)B * n8pad * 16;
  if (lds > device_lds_bytes()) return LVQ_E_SHAPE;
  const int cus = device_cus();
  int threads = kDenseThreads;
  while (threads > 256 && rows < cus * (threads / kWave)) threads /= 2;
  const int wpb = threads / kWave;
  static OccupancyCache occupancy;  // this instantiation's own
  const int occ = wgs_per_cu(occupancy, fp16_gemv_kernel<B>, threads, lds);
  long long wgs = ((long long)rows + wpb - 1) / wpb;
  if (wgs > (long long)occ * cus) wgs = (long long)occ * cus;
  if (wgs < 1) wgs = 1;
  clear_hip_error();
  hipLaunchKernelGGL(fp16_gemv_kernel<B>, dim3((unsigned)wgs), dim3(threads), lds, st, W, rows,
                     cols, n8pad, x, y);
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
