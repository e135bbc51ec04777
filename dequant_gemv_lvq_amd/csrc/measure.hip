// Read-only streaming kernels (lvq_stream_read, lvq_stream_read_geom): the
// achievable-bandwidth reference the GEMV kernels are compared with.  It reads every byte of a
// buffer once, with the same 16-byte non-temporal loads and the same grid
// shape rules as a weight stream, and folds the words into one checksum so
// the loads cannot be dropped.
//
// gfx950 design: 256-thread workgroups, at most eight per CU, grid-strided;
// each thread keeps four 16-byte loads in flight per trip.  The checksum is
// the XOR of all 32-bit words (order-free): reduced per wave by shuffles and
// per workgroup in LDS, then stored by each workgroup into its own sink word
// (no atomics: many atomics on one cache line serialize in L2 and would time
// the atomics, not the stream); the checksum is the XOR of the sink words.

#include "common.h"

namespace lvq {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kStreamThreads)
stream_read_kernel(const u32x4* __restrict__ src, size_t n16, const uint32_t* __restrict__ tail,
                   int ntail, uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * kStreamThreads * kStreamUnroll;
  uint32_t acc = 0;
  for (size_t base = (size_t)blockIdx.x * kStreamThreads * kStreamUnroll + threadIdx.x;
       base < n16; base += stride) {
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int i = 0; i < kStreamUnroll; ++i) {
      const size_t idx = base + (size_t)i * kStreamThreads;
      v[i] = idx < n16 ? __builtin_nontemporal_load(src + idx) : (u32x4){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < kStreamUnroll; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  }
  if (blockIdx.x == 0 && (int)threadIdx.x < ntail) acc ^= tail[threadIdx.x];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, kWave);
  __shared__ uint32_t part[kStreamThreads / kWave];
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
#pragma unroll
    for (int i = 0; i < kStreamThreads / kWave; ++i) a ^= part[i];
    sink[blockIdx.x] = a;
  }
}

// The same read with the launch shape as a parameter, for the sweep that
// establishes the ceiling: THREADS per workgroup, U 16-byte loads in flight
// per thread per trip, non-temporal or ordinary loads; the grid (resident
// workgroups grid-strided, or one trip per thread) is the caller's.
template <int THREADS, int U, bool NT>
__global__ void __launch_bounds__(THREADS)
stream_read_geom_kernel(const u32x4* __restrict__ src, size_t n16, const uint32_t* __restrict__ tail,
                        int ntail, uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * THREADS * U;
  uint32_t acc = 0;
  for (size_t base = (size_t)blockIdx.x * THREADS * U + threadIdx.x; base < n16; base += stride) {
    u32x4 v[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const size_t idx = base + (size_t)i * THREADS;
      v[i] = idx < n16 ? (NT ? __builtin_nontemporal_load(src + idx) : src[idx])
                       : (u32x4){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < U; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  }
  if (blockIdx.x == 0 && (int)threadIdx.x < ntail) acc ^= tail[threadIdx.x];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, kWave);
  __shared__ uint32_t part[THREADS / kWave];
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
#pragma unroll
    for (int i = 0; i < THREADS / kWave; ++i) a ^= part[i];
    sink[blockIdx.x] = a;
  }
}

template <int THREADS, int U, bool NT>
int launch_geom(const void* buf, size_t bytes, uint32_t* sink, int wgs_per_cu, hipStream_t st) {
  const size_t n16 = bytes / 16;
  const int ntail = (int)((bytes % 16) / 4);
  const size_t per = (size_t)THREADS * U;
  size_t wgs = (n16 + per - 1) / per;
  if (wgs_per_cu > 0 && wgs > (size_t)device_cus() * wgs_per_cu)
    wgs = (size_t)device_cus() * wgs_per_cu;
  if (wgs < 1) wgs = 1;
  if (wgs > LVQ_STREAM_GEOM_SINK_WORDS) return LVQ_E_SHAPE;
  clear_hip_error();
  hipLaunchKernelGGL((stream_read_geom_kernel<THREADS, U, NT>), dim3((unsigned)wgs), dim3(THREADS),
                     0, st, (const u32x4*)buf, n16,
                     (const uint32_t*)((const uint8_t*)buf + n16 * 16), ntail, sink);
  return launch_status();
}

template <int THREADS, int U>
int launch_geom_nt(const void* buf, size_t bytes, uint32_t* sink, int wgs_per_cu, bool nt,
                   hipStream_t st) {
  return nt ? launch_geom<THREADS, U, true>(buf, bytes, sink, wgs_per_cu, st)
            : launch_geom<THREADS, U, false>(buf, bytes, sink, wgs_per_cu, st);
}

template <int THREADS>
int launch_geom_u(const void* buf, size_t bytes, uint32_t* sink, int wgs_per_cu, int unroll,
                  bool nt, hipStream_t st) {
  switch (unroll) {
    case 1: return launch_geom_nt<THREADS, 1>(buf, bytes, sink, wgs_per_cu, nt, st);
    case 2: return launch_geom_nt<THREADS, 2>(buf, bytes, sink, wgs_per_cu, nt, st);
    case 4: return launch_geom_nt<THREADS, 4>(buf, bytes, sink, wgs_per_cu, nt, st);
    case 8: return launch_geom_nt<THREADS, 8>(buf, bytes, sink, wgs_per_cu, nt, st);
    default: return LVQ_E_SHAPE;
  }
}

}  // namespace lvq

using namespace lvq;

extern "C" int lvq_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!sink || (bytes && !buf)) return LVQ_E_NULL;
  if (!aligned16(buf) || ((uintptr_t)sink & 3) || (bytes & 3)) return LVQ_E_ALIGN;
  const size_t n16 = bytes / 16;
  const int ntail = (int)((bytes % 16) / 4);
  size_t wgs = (n16 + (size_t)kStreamThreads * kStreamUnroll - 1) / ((size_t)kStreamThreads * kStreamUnroll);
  size_t cap = (size_t)device_cus() * 8;
  if (cap > LVQ_STREAM_SINK_WORDS) cap = LVQ_STREAM_SINK_WORDS;
  if (wgs > cap) wgs = cap;
  if (wgs < 1) wgs = 1;
  clear_hip_error();
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)wgs), dim3(kStreamThreads), 0,
                     (hipStream_t)stream, (const u32x4*)buf, n16,
                     (const uint32_t*)((const uint8_t*)buf + n16 * 16), ntail, sink);
  return launch_status();
}

extern "C" int lvq_stream_read_geom(const void* buf, size_t bytes, uint32_t* sink, int threads,
                                    int wgs_per_cu, int unroll, int nontemporal, void* stream) {
  if (!sink || (bytes && !buf)) return LVQ_E_NULL;
  if (!aligned16(buf) || ((uintptr_t)sink & 3) || (bytes & 3)) return LVQ_E_ALIGN;
  if (wgs_per_cu < 0 || wgs_per_cu > 8) return LVQ_E_SHAPE;
  hipStream_t st = (hipStream_t)stream;
  const bool nt = nontemporal != 0;
  switch (threads) {
    case 256: return launch_geom_u<256>(buf, bytes, sink, wgs_per_cu, unroll, nt, st);
    case 512: return launch_geom_u<512>(buf, bytes, sink, wgs_per_cu, unroll, nt, st);
    case 1024: return launch_geom_u<1024>(buf, bytes, sink, wgs_per_cu, unroll, nt, st);
    default: return LVQ_E_SHAPE;
  }
}
