// Bitshift-trellis matvec (trellis_gemv), the trellis comparison arm.
//
// Source: blog "Qwen3.8-27B on a 12 GB card", section "A trellis is a codebook
// you walk": the state is the last L bits of the stream, each step shifts T
// new bits in, so decoding a position means reading one L-bit window and no
// step depends on the previous step's output.  Here L = 16, T = 2, one weight
// per step, a 65536-entry fp16 table and one scale per row; every 256 columns
// form a tail-biting packet.
//
// gfx950 design.  One 1024-thread workgroup per CU copies the 128 KiB table
// into LDS once and then loops over rows (one wave per row at a time).  Lane l
// takes code words l, l + 64, ... of the row; for each of the 16 symbols of
// its word the state is a single funnel shift (v_alignbit) of the previous
// and current word, masked to 16 bits, and the weight is one LDS read.  Two
// table values are packed into an fp16 pair for v_dot2_f32_f16 against the x
// pair; the row scale is applied after the fixed butterfly reduction.  The
// previous word of the first word of a packet is the packet's last word.

#include "common.h"

namespace lvq {

constexpr int kTrellisThreads = 1024;
constexpr int kTrellisWaves = kTrellisThreads / kWave;

template <int B>
__global__ void __launch_bounds__(kTrellisThreads)
trellis_gemv_kernel(const uint32_t* __restrict__ bits, const uint16_t* __restrict__ table,
                    const uint16_t* __restrict__ scale, int rows, int cols,
                    const uint16_t* __restrict__ x, float* __restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint16_t* tbl = (uint16_t*)smem;                 // [65536]
  uint32_t* xs = (uint32_t*)(smem + 65536 * 2);    // [B][cols/2] natural-order pairs
  const int tid = threadIdx.x;
  for (int i = tid; i < 65536 / 8; i += kTrellisThreads)
    ((uint4*)tbl)[i] = ((const uint4*)table)[i];
  for (int i = tid; i < B * cols / 8; i += kTrellisThreads)
    ((uint4*)xs)[i] = ((const uint4*)x)[i];
  __syncthreads();

  const int nw = cols / 16;
  const int lane = tid & (kWave - 1);
  const int wave = blockIdx.x * kTrellisWaves + tid / kWave;
  const int nwaves = gridDim.x * kTrellisWaves;
  for (int r = wave; r < rows; r += nwaves) {
    const uint32_t* brow = bits + (size_t)r * nw;
    float acc[B][2];
#pragma unroll
    for (int bb = 0; bb < B; ++bb) acc[bb][0] = acc[bb][1] = 0.f;
    for (int i = lane; i < nw; i += kWave) {
      const uint32_t cur = brow[i];
      const uint32_t prev = brow[(i & 15) ? i - 1 : i + 15];
#pragma unroll
      for (int p = 0; p < 16; p += 2) {
        const uint32_t s0 = __builtin_amdgcn_alignbit(prev, cur, 30 - 2 * p) & 0xFFFFu;
        const uint32_t s1 = __builtin_amdgcn_alignbit(prev, cur, 28 - 2 * p) & 0xFFFFu;
        const uint32_t w2 = (uint32_t)tbl[s0] | ((uint32_t)tbl[s1] << 16);
#pragma unroll
        for (int bb = 0; bb < B; ++bb)
          acc[bb][p >> 3] = dot2(w2, xs[(size_t)bb * (cols / 2) + 8 * i + (p >> 1)], acc[bb][p >> 3]);
      }
    }
    const float s = (float)__builtin_bit_cast(_Float16, scale[r]);
#pragma unroll
    for (int bb = 0; bb < B; ++bb) {
      const float tot = wave_sum_lane63(acc[bb][0] + acc[bb][1]);
      if (lane == kWave - 1) y[(size_t)bb * rows + r] = tot * s;
    }
  }
}

int zero_output(float* y, size_t n, hipStream_t st);

template <int B>
int launch_trellis(const uint32_t* bits, const uint16_t* table, const uint16_t* scale, int rows,
                   int cols, const uint16_t* x, float* y, hipStream_t st) {
  const size_t lds = 65536 * 2 + (size_t)B * cols * 2;
  if (lds > device_lds_bytes()) return LVQ_E_SHAPE;
  int wgs = (rows + kTrellisWaves - 1) / kTrellisWaves;
  if (wgs > device_cus()) wgs = device_cus();
  clear_hip_error();
  hipLaunchKernelGGL(trellis_gemv_kernel<B>, dim3(wgs), dim3(kTrellisThreads), lds, st, bits, table,
                     scale, rows, cols, x, y);
  return launch_status();
}

}  // namespace lvq

using namespace lvq;

extern "C" int trellis_gemv(const uint32_t* bits, const uint16_t* table, const uint16_t* scale,
                            int rows, int cols, const uint16_t* x, float* y, int batch,
                            void* stream) {
  if (rows < 0 || cols < 0 || cols % 256) return LVQ_E_SHAPE;
  int e = check_batch(batch);
  if (e) return e;
  if (!y || !table || (rows && (!scale || (cols && (!bits || !x))))) return LVQ_E_NULL;
  if (!aligned16(bits) || !aligned16(table) || !aligned16(scale) || !aligned16(x) ||
      !aligned16(y))
    return LVQ_E_ALIGN;
  if ((long long)batch * cols > 12288) return LVQ_E_SHAPE;
  hipStream_t st = (hipStream_t)stream;
  if (rows == 0) return LVQ_OK;
  if (cols == 0) return zero_output(y, (size_t)batch * rows, st);
  switch (batch) {
    case 1: return launch_trellis<1>(bits, table, scale, rows, cols, x, y, st);
    case 2: return launch_trellis<2>(bits, table, scale, rows, cols, x, y, st);
    case 3: return launch_trellis<3>(bits, table, scale, rows, cols, x, y, st);
    default: return launch_trellis<4>(bits, table, scale, rows, cols, x, y, st);
  }
}
