// Load-time unfolding of 48-bit block words (lvq_unfold): word -> the 24
// integer coordinates of its Leech-lattice point and its gain bit.
//
// Source: arXiv 2609.02652 serves the source method's 48 bits per 24-weight
// block, a 47-bit index into the m <= 12 ball plus one gain bit, and unfolds
// them into its GPU layouts at load time (quality-protocol, published-results
// and validity-envelope paragraphs).  The enumeration order is this library's
// (see index.h); the tables are built on the host by index.cpp.
//
// gfx950 design.  One thread per word.  The (type, codeword) block of the
// index is found by binary search over the 8193 block offsets, then the 24
// coordinates are chosen one at a time: for each candidate value in ascending
// order the number of completions of the remaining coordinates is read from
// the counting table (about 1 MB of 64-bit counts, L2-resident) and
// subtracted until the index falls inside.  At most 7 candidates per
// coordinate, all loads of one coordinate independent of each other.  The
// tables live in device globals of the code object (no allocation), uploaded
// once per device on the first call.

#include <mutex>

#include "common.h"
#include "index.h"

namespace lvq {

__device__ uint64_t g_idx_f[kIdxFSize];
__device__ uint64_t g_idx_offs[kIdxBlocks + 1];
__device__ uint32_t g_idx_cw[4096];

__global__ void __launch_bounds__(256)
unfold_kernel(const uint64_t* __restrict__ words, size_t n, int8_t* __restrict__ coords,
              uint8_t* __restrict__ gain) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint64_t w = words[i];
  const uint64_t idx = w & kIdxMask;
  uint32_t out[6] = {0, 0, 0, 0, 0, 0};
  uint8_t status = 0xFF;
  if ((w >> 48) == 0 && idx < g_idx_offs[kIdxBlocks]) {
    // block: the last offset <= idx
    int lo = 0, hi = kIdxBlocks;  // offs[lo] <= idx < offs[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (g_idx_offs[mid] <= idx) lo = mid; else hi = mid;
    }
    const int t = lo >> 12;
    const uint32_t c = g_idx_cw[lo & 4095];
    uint64_t rem = idx - g_idx_offs[lo];
    int nb = __builtin_popcount(c), na = 24 - nb, q = t ? 21 : 48, p = t;
    for (int j = 0; j < 24; ++j) {
      const int ci = (c >> j) & 1;
      if (ci) --nb; else --na;
      const int r = t ? 1 + 2 * ci : 2 * ci;
      int v = r - 16;  // the smallest value = r (mod 4) that is >= -13
      if (v < -13) v += 4;
      int chosen = 13;
      for (int s = 0; s < 7; ++s, v += 4) {
        if (v > 13) break;
        const int cst = t ? (v * v - 1) >> 3 : (v * v) >> 2;
        if (cst > q) continue;
        const int zp = ((v - r) >> 2) & 1;
        const uint64_t cnt = g_idx_f[idx_f(t, na, nb, q - cst, p ^ zp)];
        if (rem < cnt) {
          chosen = v;
          q -= cst;
          p ^= zp;
          break;
        }
        rem -= cnt;
      }
      out[j >> 2] |= (uint32_t)(uint8_t)(int8_t)chosen << (8 * (j & 3));
    }
    status = (uint8_t)((w >> 47) & 1);
  }
  uint32_t* dst = (uint32_t*)(coords + i * 24);  // 8-byte aligned: 24 i
#pragma unroll
  for (int k = 0; k < 6; ++k) dst[k] = out[k];
  gain[i] = status;
}

namespace {
std::mutex g_upload_mu;
bool g_uploaded[kMaxDevices] = {};
}  // namespace

int upload_index_tables() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LVQ_E_HIP;
  std::lock_guard<std::mutex> lock(g_upload_mu);
  if (g_uploaded[dev]) return LVQ_OK;
  const IndexTables& T = index_tables();
  if (hipMemcpyToSymbol(HIP_SYMBOL(g_idx_f), T.f, sizeof(T.f)) != hipSuccess ||
      hipMemcpyToSymbol(HIP_SYMBOL(g_idx_offs), T.offs, sizeof(T.offs)) != hipSuccess ||
      hipMemcpyToSymbol(HIP_SYMBOL(g_idx_cw), T.cw, sizeof(T.cw)) != hipSuccess)
    return LVQ_E_HIP;
  g_uploaded[dev] = true;
  return LVQ_OK;
}

}  // namespace lvq

using namespace lvq;

extern "C" int lvq_unfold(const uint64_t* words, size_t nblocks, int8_t* coords_out,
                          uint8_t* gain_out, void* stream) {
  if (nblocks && (!words || !coords_out || !gain_out)) return LVQ_E_NULL;
  if (!aligned16(words) || !aligned16(coords_out) || !aligned16(gain_out)) return LVQ_E_ALIGN;
  if (!nblocks) return LVQ_OK;
  int e = upload_index_tables();
  if (e) return e;
  const size_t wgs = (nblocks + 255) / 256;
  if (wgs > 0x7FFFFFFF) return LVQ_E_SHAPE;
  clear_hip_error();
  hipLaunchKernelGGL(unfold_kernel, dim3((unsigned)wgs), dim3(256), 0, (hipStream_t)stream, words,
                     nblocks, coords_out, gain_out);
  return launch_status();
}
