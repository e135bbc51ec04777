// Internal helpers shared by the gfx950 kernels and their host wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../include/lvq.h"

typedef _Float16 lvq_half2 __attribute__((ext_vector_type(2)));

namespace lvq {

constexpr int kWave = 64;

// ---------------------------------------------------------------- host side

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

inline int check_batch(int batch) {
  return (batch < 1 || batch > LVQ_MAX_BATCH) ? LVQ_E_BATCH : LVQ_OK;
}

// Clear an error left by an earlier, unrelated HIP call before a launch, so
// launch_status() reports only the launch itself.
inline void clear_hip_error() { (void)hipGetLastError(); }

inline int launch_status() {
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) return LVQ_OK;
  if (getenv("LVQ_VERBOSE")) fprintf(stderr, "liblvq: %s\n", hipGetErrorString(e));
  return LVQ_E_HIP;
}

// Number of compute units of the current device (cached per device id).
int device_cus();
// Largest dynamic LDS allocation a workgroup may request on the current device.
size_t device_lds_bytes();

constexpr int kMaxDevices = 64;

// Workgroups per CU (at most 2) that fit at once for one kernel, by the occupancy query,
// kept in that kernel's own cache (`cache`, one per kernel instantiation) per
// device and per (workgroup size, LDS above 64 KiB).  The entries are ints
// written whole with the same value by any thread that races on them.
typedef int OccupancyCache[kMaxDevices][3][2];
template <typename K>
int wgs_per_cu(OccupancyCache& cache, K kernel, int threads, size_t lds) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  const int ti = threads == 1024 ? 0 : threads == 512 ? 1 : 2, li = lds > 64 * 1024;
  int n = __atomic_load_n(&cache[dev][ti][li], __ATOMIC_RELAXED);
  if (!n) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, lds) != hipSuccess ||
        n < 1)
      n = 1;
    n = n > 2 ? 2 : n;
    __atomic_store_n(&cache[dev][ti][li], n, __ATOMIC_RELAXED);
  }
  return n;
}

// ---------------------------------------------------------------- device side

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float v) {
  // v + (the value DPP routes to this lane; 0 where the row is masked off)
  const int moved = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK,
                                                0xF, false);
  return v + __builtin_bit_cast(float, moved);
}

// Sum over the 64 lanes of a wave in a fixed order (so the result never
// depends on timing): quad swaps, half-row and row mirrors give each row of 16
// its sum, then two row broadcasts carry rows 0..2 into row 3.  The total is
// valid in lane 63.
__device__ __forceinline__ float wave_sum_lane63(float v) {
  v = dpp_add<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_add<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_add<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_add<0x140, 0xF>(v);  // row_mirror
  v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
  // fixed butterfly: every lane ends with the same, order-independent sum
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ lvq_half2 as_half2(uint32_t u) {
  return __builtin_bit_cast(lvq_half2, u);
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(as_half2(a), as_half2(b), c, false);
}

// Leech decode of one coordinate pair.  `word` is a code word of a block; view
// v (0..3) selects its slots v (low half) and v + 4 (high half), which carry
// the adjacent coordinates 8w + 2v and 8w + 2v + 1.  After the
// rotation by 4v, bits 0..2 and 16..18 hold the two table slots (rank + 1)
// and bits 11 and 27 the two "non-negative" flags, so masking with 0x08070807
// leaves the selector bytes  slot, 8*nonneg, slot, 8*nonneg.  v_perm_b32 reads
// them against the block's 8-byte LUT
//   byte 0 = 0x80, bytes 1..5 = the ascending magnitudes (ranks 0..4),
// where selector 8 yields the sign-extension of byte 1 (a magnitude <= 13,
// so 0x00).  Each 16-bit half is then the fp16 pattern sign | magnitude: the
// signed coordinate times 2^-24 as an exact fp16 subnormal.
__device__ __forceinline__ uint32_t leech_pair(uint32_t word, int v, uint32_t lut_lo,
                                               uint32_t lut_hi) {
  uint32_t r = v ? __builtin_amdgcn_alignbit(word, word, 4 * v) : word;
  return __builtin_amdgcn_perm(lut_hi, lut_lo, r & 0x08070807u);
}

// LUT words of a class-table entry (bytes 0..4 ascending magnitudes).
__device__ __forceinline__ uint2 leech_lut(uint64_t entry) {
  uint2 l;
  l.x = (uint32_t)(entry << 8) | 0x80u;
  l.y = (uint32_t)(entry >> 24) & 0xFFFFu;
  return l;
}

}  // namespace lvq
