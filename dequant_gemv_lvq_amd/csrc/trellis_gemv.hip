// Bitshift-trellis matvec (trellis_gemv), the trellis comparison arm.
//
// Source: blog "Qwen3.8-27B on a 12 GB card", section "A trellis is a codebook
// you walk".  A position's decoder state is a fixed-width window of the code
// stream ending at that position's symbol, so each weight is one window read
// plus one table entry, and positions decode independently of each other.
// Here the window is 16 bits, a symbol 2 bits (one weight per symbol), the
// table holds 65536 fp16 values, each row has one scale, and each run of 256
// columns is a tail-biting packet.
//
// gfx950 design.  One 1024-thread workgroup per CU copies the 128 KiB table
// and x into LDS with buffer loads that write LDS directly, then its waves
// walk rows (one row per wave at a time).  Lane l takes code words l, l + 64,
// ... of the row; all of them are requested at once, so a row costs one
// memory round trip, and a wave's first row is requested before the staging
// barrier, so that round trip overlaps the 128 KiB table copy.  The word before word w in its packet (w - 1, or the
// packet's last word for its first word) is held by lane l - 1 or l + 15 and
// comes over with one lane shuffle.  For each of the 16 symbols of a word the
// table's byte address (state * 2) is one funnel shift of the previous and
// current word (v_alignbit) and one mask; the value is one LDS read.  Two
// table values are packed into an fp16 pair for v_dot2_f32_f16 against the
// x pair; the row scale is applied after a fixed DPP reduction.

#include "common.h"

namespace lvq {

constexpr int kTrellisThreads = 1024;
constexpr int kTrellisWaves = kTrellisThreads / kWave;
constexpr int kTrellisMaxWordsPerLane = 12;  // batch * cols <= 12288: <= 768 words per row

__device__ __forceinline__ __amdgpu_buffer_rsrc_t trellis_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// byte address in the table of the state after symbol p (0..15) of `cur`,
// whose predecessor word is `prev`: bits 30-2p .. 45-2p of prev:cur, times 2
__device__ __forceinline__ uint32_t trellis_addr(uint32_t prev, uint32_t cur, int p) {
  const uint32_t w = p < 15 ? __builtin_amdgcn_alignbit(prev, cur, 29 - 2 * p) : cur << 1;
  return w & 0x1FFFEu;
}

// The kernel declares no static LDS, so its dynamic LDS (the table first)
// starts at LDS address 0 and a table byte address is an LDS address: reading
// through it directly saves adding the base to every lookup.
typedef const _Float16 __attribute__((address_space(3))) lds_f16_t;
__device__ __forceinline__ lds_f16_t* lds_f16(uint32_t byte_addr) {
  return (lds_f16_t*)(uintptr_t)byte_addr;
}

template <int B>
__global__ void __launch_bounds__(kTrellisThreads)
trellis_gemv_kernel(const uint32_t* __restrict__ bits, const uint16_t* __restrict__ table,
                    const uint16_t* __restrict__ scale, int rows, int cols,
                    const uint16_t* __restrict__ x, float* __restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // smem: the table fp16 [65536] (byte address 2 * state), then x as
  // [B][2][nw] 16-byte units: unit (h, w) holds the pairs 4h .. 4h + 3 of
  // code word w's 16 columns, so the lanes of a wave (consecutive words)
  // read consecutive units
  uint32_t* xs = (uint32_t*)(smem + 65536 * 2);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nw = cols / 16;

  const int wave = blockIdx.x * kTrellisWaves + wv;
  const int nwaves = gridDim.x * kTrellisWaves;
  // one row's code words (every word at once; words past the row's end, or
  // a row past the last, read 0) and its scale
  uint32_t cw[kTrellisMaxWordsPerLane];
  uint32_t sbits = 0;
  auto load_row = [&](int r) {
    const bool ok = r < rows;
    const auto rb = trellis_rsrc(bits + (size_t)(ok ? r : 0) * nw, ok ? (uint32_t)nw * 4 : 0u);
    // no branch per load (a load past the row's range reads 0 and makes no
    // request), so the waits after it count exactly
#pragma unroll
    for (int j = 0; j < kTrellisMaxWordsPerLane; ++j)
      cw[j] = __builtin_amdgcn_raw_buffer_load_b32(rb, (lane + j * kWave) * 4, 0, 2);
    const auto rsc = trellis_rsrc(scale + (ok ? r : 0), ok ? 2u : 0u);
    sbits = __builtin_amdgcn_raw_buffer_load_b16(rsc, 0, 0, 0);
  };

  // table and x straight into LDS, 1 KiB per wave instruction; the first
  // row's code words are requested right behind them, so they arrive while
  // the table is copied (the barrier waits for the copies only)
  {
    const auto rt = trellis_rsrc(table, 65536 * 2);
    for (int q = wv; q < 128; q += kTrellisWaves)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rt, (__attribute__((address_space(3))) void*)(smem + q * 1024), 16, lane * 16, q * 1024,
          0, 0);
    // each lane of a copy fetches the natural unit its transposed LDS unit
    // holds (units past x read 0)
    const int xbytes = B * cols * 2;  // a multiple of 512
    const int units = 2 * nw;         // 16-byte units per batch row
    const auto rx = trellis_rsrc(x, (uint32_t)xbytes);
    for (int q = wv; q * 1024 < xbytes; q += kTrellisWaves) {
      const int u = q * kWave + lane, bb = u / units, k = u - bb * units;
      const int h = k >= nw ? 1 : 0, w = k - h * nw;
      const int src = u < B * units ? (bb * units + 2 * w + h) * 16 : xbytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (__attribute__((address_space(3))) void*)((uint8_t*)xs + q * 1024), 16, src, 0, 0,
          0);
    }
  }
  load_row(wave);
  __syncthreads();

  const int src = (lane & 15) ? lane - 1 : lane + 15;  // holder of the previous word
  for (int r = wave; r < rows; r += nwaves) {
    if (r != wave) load_row(r);
    float acc[B][2];
#pragma unroll
    for (int bb = 0; bb < B; ++bb) acc[bb][0] = acc[bb][1] = 0.f;
#pragma unroll
    for (int j = 0; j < kTrellisMaxWordsPerLane; ++j) {
      if (j * kWave >= nw) break;                  // uniform
      const int w = lane + j * kWave;
      const uint32_t cur = cw[j];
      const uint32_t prev = (uint32_t)__shfl((int)cur, src, kWave);
      if (w < nw) {
#pragma unroll
        for (int p = 0; p < 16; p += 2) {
          // the two table values land in the two halves of one register
          lvq_half2 h;
          h.x = *lds_f16(trellis_addr(prev, cur, p));
          h.y = *lds_f16(trellis_addr(prev, cur, p + 1));
          const uint32_t w2 = __builtin_bit_cast(uint32_t, h);
#pragma unroll
          for (int bb = 0; bb < B; ++bb) {
            const int pr = p >> 1;  // pair 0..7 of the word's 16 columns
            acc[bb][pr & 1] = dot2(
                w2, xs[(size_t)bb * (cols / 2) + ((pr >> 2) * nw + w) * 4 + (pr & 3)],
                acc[bb][pr & 1]);
          }
        }
      }
    }
    const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)sbits);
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
  // x rounded up to whole KiB: the last buffer-to-LDS copy writes a full KiB
  const size_t lds = 65536 * 2 + (((size_t)B * cols * 2 + 1023) & ~(size_t)1023);
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
