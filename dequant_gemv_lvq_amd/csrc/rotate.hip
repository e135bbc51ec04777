// Activation rotation (lvq_rotate): y = (H kron Q)(S x) before a GEMV.
//
// Sources: arXiv 2609.02652 keeps the weights in an incoherence-rotated basis,
// so each projection's input goes through a Walsh-Hadamard transform first, a
// transform that needs the whole activation resident in one block's shared
// memory (served-path setup, and the section on the rotated basis and the
// shared-memory wall: the widest activation of the largest model needed
// 102,400 B of f32 and did not fit that card).  The Tetra summary (section
// "What the kernel does per token") gives the form for widths that are not
// powers of two: (H kron Q)(S x), S random signs, H a power-of-two
// Walsh-Hadamard transform, Q a small orthogonal matrix.
//
// n = K m, K a power of two, coordinate a m + b; H = K^-1/2 times the Sylvester
// matrix ((-1)^popcount(a & c)); Q is m x m (identity when none is given).
//
// gfx950 design.  The m interleaved sequences are independent once Q has mixed
// each group, so one workgroup takes one (batch row, b) pair and one K-point
// transform (K <= 32768).  A lane produces 8 consecutive values of its
// sequence: for m = 1 one 16-byte load of x, for m > 1 the Q mix
// w[c] = sum_d Q[b][d] x'[c m + d] from the row of x staged in LDS with row b
// of Q in scalar registers; the signs are XORed into the fp16 sign bits
// (exact).  Butterfly stages 0-2 run in the lane's registers, stages 3-8
// across the 64 lanes of its wave by lane exchanges, so a wave finishes
// 512-point transforms without touching LDS.  For K <= 512 the results are
// scaled, rounded to fp16 and stored from registers.  Otherwise they go to
// LDS once (f32), and after one barrier a single pass does the remaining
// stages 9 .. log2 K - 1 (up to 64 values per thread, coordinates 512 apart,
// consecutive threads at consecutive addresses: no bank conflicts) and
// stores.  LDS: 4 K bytes (+ 2 n for the staged x when m > 1); the largest
// Qwen3-family width, 25600 (the one that did not fit the pages' card as
// f32), takes 54 KiB.

#include "common.h"
#include "rotate_dev.h"

namespace lvq {

constexpr int kRotThreads = 1024;
constexpr int kRotMaxM = 32;





// Stages s .. s + R - 1 over buf: coordinates 2^s apart, consecutive threads
// at consecutive addresses (for s >= 4).  The last pass scales, rounds and
// stores.
template <int R>
__device__ __forceinline__ void rot_high_pass(float* buf, int k, int s, bool last, int mm, int b,
                                              float scale, uint16_t* yr, int tid, int nthr) {
  constexpr int kR = 1 << R;
  const int nsets = k >> R;
  const int low = (1 << s) - 1;
  for (int set = tid; set < nsets; set += nthr) {
    const int base = ((set & ~low) << R) | (set & low);
    float v[kR];
#pragma unroll
    for (int t = 0; t < kR; ++t) v[t] = buf[base + (t << s)];
#pragma unroll
    for (int h = 1; h < kR; h <<= 1) {
#pragma unroll
      for (int t = 0; t < kR; ++t) {
        if (t & h) continue;
        const float lo = v[t], hi = v[t + h];
        v[t] = lo + hi;
        v[t + h] = lo - hi;
      }
    }
    if (last) {
#pragma unroll
      for (int t = 0; t < kR; ++t) yr[(size_t)(base + (t << s)) * mm + b] = rot_out(v[t], scale);
    } else {
#pragma unroll
      for (int t = 0; t < kR; ++t) buf[base + (t << s)] = v[t];
    }
  }
}

// Workgroup (b, batch row): y[c m + b] for c < K.
template <int MMAX>
__global__ void __launch_bounds__(kRotThreads)
rotate_kernel(const uint16_t* x, const uint32_t* __restrict__ signs,
              const float* __restrict__ q, int n, int m, int logk, float scale, uint16_t* y) {
  // y may be x when m = 1: a row's one workgroup reads all of it before its
  // barrier and writes after it (for m > 1 the host refuses overlap)
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & (kWave - 1);
  const int b = MMAX == 1 ? 0 : blockIdx.x;
  const int mm = MMAX == 1 ? 1 : m;
  const int k = n / mm;
  const uint16_t* xr = x + (size_t)blockIdx.y * n;
  uint16_t* yr = y + (size_t)blockIdx.y * n;
  // LDS: the staged row of x (m > 1), then the f32 sequence (K > 512)
  uint16_t* xs = (uint16_t*)smem;
  float* buf = (float*)(smem + (MMAX > 1 ? (((size_t)n * 2 + 15) & ~(size_t)15) : 0));
  if (MMAX == 1 && q) scale *= q[0];  // a 1 x 1 Q is a scale (+-1 when orthogonal)

  // m > 1: the row of x, signs applied, into LDS (four 16-byte loads per
  // thread in flight), then every thread mixes groups with row b of Q into
  // the f32 sequence
  if (MMAX > 1) {
    if ((n & 7) == 0) {
      const int n8 = n >> 3;
      for (int j0 = 0; j0 < n8; j0 += 4 * nthr) {
        uint4 v[4];
        uint32_t s8[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int j8 = j0 + u * nthr + tid;
          v[u] = j8 < n8 ? *(const uint4*)(xr + (size_t)j8 * 8) : make_uint4(0, 0, 0, 0);
          s8[u] = signs && j8 < n8 ? signs[j8 >> 2] >> ((j8 & 3) * 8) : 0u;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int j8 = j0 + u * nthr + tid;
          if (j8 < n8) *(uint4*)(xs + j8 * 8) = rot_apply_signs(v[u], s8[u]);
        }
      }
    } else {
      for (int j = tid; j < n; j += nthr)
        xs[j] = xr[j] ^ (signs ? (uint16_t)(((signs[j >> 5] >> (j & 31)) & 1u) << 15) : 0);
    }
    // row b of Q: uniform, so scalar loads
    float qrow[MMAX];
#pragma unroll
    for (int d = 0; d < MMAX; ++d)
      qrow[d] = d < m ? (q ? q[b * m + d] : (d == b ? 1.f : 0.f)) : 0.f;
    __syncthreads();
    for (int c = tid; c < k; c += nthr) {
      float a = 0.f;
#pragma unroll
      for (int d = 0; d < MMAX; ++d)
        if (d < m) a = __builtin_fmaf(qrow[d], rot_half(xs[c * m + d]), a);
      buf[c] = a;
    }
    __syncthreads();
  }

  // 1. 8 consecutive values per lane (fewer when K < 8), stages 0 .. 8
  const int cw = k < 8 ? k : 8;              // values per lane
  const int nch = k / cw;                    // lanes with values
  const int lo_bits = logk < 9 ? logk : 9;   // stages done before LDS
  for (int ch0 = 0; ch0 < nch; ch0 += nthr) {
    const int ch = ch0 + tid;
    float v[8];
    if (MMAX == 1) {
      if (cw == 8) {
        uint4 u = ch < nch ? *(const uint4*)(xr + (size_t)ch * 8) : make_uint4(0, 0, 0, 0);
        const uint32_t s8 = signs && ch < nch ? signs[ch >> 2] >> ((ch & 3) * 8) : 0u;
        u = rot_apply_signs(u, s8);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = rot_half((uint16_t)w[i]);
          v[2 * i + 1] = rot_half((uint16_t)(w[i] >> 16));
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int j = ch * cw + i;
          v[i] = 0.f;
          if (i < cw && ch < nch)
            v[i] = rot_half(xr[j] ^ (signs ? (uint16_t)(((signs[j >> 5] >> (j & 31)) & 1u) << 15)
                                           : 0));
        }
      }
    } else if (cw == 8) {
      const float4 lo = ch < nch ? *(const float4*)(buf + ch * 8) : make_float4(0, 0, 0, 0);
      const float4 hi = ch < nch ? *(const float4*)(buf + ch * 8 + 4) : make_float4(0, 0, 0, 0);
      v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
      v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = i < cw && ch < nch ? buf[ch * cw + i] : 0.f;
    }
    // stages 0-2 in registers
#pragma unroll
    for (int e = 0; e < 3; ++e) {
      const int h = 1 << e;
      if (h >= cw) break;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if (t & h) continue;
        const float lo = v[t], hi = v[t + h];
        v[t] = lo + hi;
        v[t + h] = lo - hi;
      }
    }
    // stages 3 .. lo_bits - 1 across lanes (lane bit j = chunk bit j)
    for (int j = 0; (8 << j) <= (1 << lo_bits) && cw == 8; ++j) {
      if ((8 << j) == (1 << lo_bits)) break;
#pragma unroll
      for (int t = 0; t < 8; ++t) v[t] = rot_lane_bfly(v[t], 1 << j, lane);
    }
    if (ch < nch) {
      if (logk <= 9) {
        if (MMAX == 1 && cw == 8) {
          uint32_t w[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            w[i] = rot_out(v[2 * i], scale) | ((uint32_t)rot_out(v[2 * i + 1], scale) << 16);
          *(uint4*)(yr + (size_t)ch * 8) = make_uint4(w[0], w[1], w[2], w[3]);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (i < cw) yr[(size_t)(ch * cw + i) * mm + b] = rot_out(v[i], scale);
        }
      } else {
        *(float4*)(buf + ch * 8) = make_float4(v[0], v[1], v[2], v[3]);
        *(float4*)(buf + ch * 8 + 4) = make_float4(v[4], v[5], v[6], v[7]);
      }
    }
  }
  if (logk <= 9) return;  // uniform
  __syncthreads();

  // 2. stages 9 .. log2 K - 1, up to four per pass; the last pass scales,
  //    rounds and stores
  for (int s = 9; s < logk; s += 4) {
    const int r = logk - s < 4 ? logk - s : 4;
    const bool last = s + r == logk;
    if (r == 4) rot_high_pass<4>(buf, k, s, last, mm, b, scale, yr, tid, nthr);
    else if (r == 3) rot_high_pass<3>(buf, k, s, last, mm, b, scale, yr, tid, nthr);
    else if (r == 2) rot_high_pass<2>(buf, k, s, last, mm, b, scale, yr, tid, nthr);
    else rot_high_pass<1>(buf, k, s, last, mm, b, scale, yr, tid, nthr);
    if (!last) __syncthreads();
  }
}

// Workgroup (b, batch row) for K >= 16 and m = MM <= 8: y[c m + b] for c < K.
// A thread takes 16 consecutive values of sequence b: for m = 1 two 16-byte
// loads of x, for m > 1 the Q mix of the 16 groups (32 m contiguous bytes of
// x, read as 16-byte loads, eight groups at a time) in registers, in the same
// fma order as the general kernel; the signs are XORed into each 16-byte
// unit as it arrives.  Stages 0-3 in registers, the 16 values to LDS, then
// radix passes for stages 4 and up with consecutive threads on consecutive
// addresses; the last pass scales, rounds and stores.  Each stage applies
// the same butterflies to the same operands as the general kernel, so both
// give the same bits.  No staging of x and no lane exchanges: one barrier per
// pass.  LDS: 4 K bytes.
template <int MM>
__global__ void __launch_bounds__(kRotThreads)
rotate16_kernel(const uint16_t* x, const uint32_t* __restrict__ signs,
                const float* __restrict__ q, int n, int logk, float scale, uint16_t* y) {
  // y may be x when m = 1: every read of the row happens before the first
  // barrier and every write after the last one (for m > 1 the host refuses
  // overlap)
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float* buf = (float*)smem;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int b = MM == 1 ? 0 : blockIdx.x;
  const uint16_t* xr = x + (size_t)blockIdx.y * n;
  uint16_t* yr = y + (size_t)blockIdx.y * n;
  if (MM == 1 && q) scale *= q[0];
  float qrow[MM];
#pragma unroll
  for (int d = 0; d < MM; ++d) qrow[d] = MM == 1 ? 1.f : (q ? q[b * MM + d] : (d == b ? 1.f : 0.f));
  // coordinates 8 j8 .. 8 j8 + 7 of the row, signs applied
  auto unit = [&](int j8) {
    const uint4 u = *(const uint4*)(xr + (size_t)8 * j8);
    return signs ? rot_apply_signs(u, signs[j8 >> 2] >> ((j8 & 3) * 8)) : u;
  };
  const int nck = 1 << (logk - 4);
  for (int c16 = tid; c16 < nck; c16 += nthr) {
    float v[16];
    if (MM == 1) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint4 u = unit(2 * c16 + h);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[8 * h + 2 * i] = rot_half((uint16_t)w[i]);
          v[8 * h + 2 * i + 1] = rot_half((uint16_t)(w[i] >> 16));
        }
      }
    } else {
      auto mix8 = [&](int g0, float* o) {  // groups g0 .. g0 + 7
        uint32_t w[4 * MM];
#pragma unroll
        for (int i = 0; i < MM; ++i) {
          const uint4 u = unit(g0 * MM / 8 + i);
          w[4 * i] = u.x;
          w[4 * i + 1] = u.y;
          w[4 * i + 2] = u.z;
          w[4 * i + 3] = u.w;
        }
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          float a = 0.f;
#pragma unroll
          for (int d = 0; d < MM; ++d) {
            const int e = g * MM + d;
            a = __builtin_fmaf(qrow[d], rot_half((uint16_t)(w[e >> 1] >> (16 * (e & 1)))), a);
          }
          o[g] = a;
        }
      };
      mix8(16 * c16, v);
      mix8(16 * c16 + 8, v + 8);
    }
#pragma unroll
    for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        if (t & h) continue;
        const float lo = v[t], hi = v[t + h];
        v[t] = lo + hi;
        v[t + h] = lo - hi;
      }
    }
    if (logk == 4) {
#pragma unroll
      for (int t = 0; t < 16; ++t) yr[(size_t)(16 * c16 + t) * MM + b] = rot_out(v[t], scale);
    } else {
      float4* f = (float4*)(buf + 16 * c16);
#pragma unroll
      for (int i = 0; i < 4; ++i) f[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
    }
  }
  if (logk == 4) return;  // uniform
  __syncthreads();
  const int k = 1 << logk;
  for (int st = 4; st < logk; st += 4) {
    const int r = logk - st < 4 ? logk - st : 4;
    const bool last = st + r == logk;
    if (r == 4) rot_high_pass<4>(buf, k, st, last, MM, b, scale, yr, tid, nthr);
    else if (r == 3) rot_high_pass<3>(buf, k, st, last, MM, b, scale, yr, tid, nthr);
    else if (r == 2) rot_high_pass<2>(buf, k, st, last, MM, b, scale, yr, tid, nthr);
    else rot_high_pass<1>(buf, k, st, last, MM, b, scale, yr, tid, nthr);
    if (!last) __syncthreads();
  }
}

template <int MM>
int launch_rotate16(const uint16_t* x, const uint32_t* signs, const float* q, int n, uint16_t* y,
                    int batch, hipStream_t st) {
  const int k = n / MM;
  int logk = 0;
  while ((1 << logk) < k) ++logk;
  if (logk > 15) return LVQ_E_SHAPE;
  const size_t lds = (size_t)k * 4;
  if (lds > device_lds_bytes()) return LVQ_E_SHAPE;
  // one thread per 16 values (and per radix set of the passes), whole waves
  int threads = ((k >> 4) + kWave - 1) / kWave * kWave;
  if (threads > kRotThreads) threads = kRotThreads;
  const float scale = (float)(1.0 / __builtin_sqrt((double)k));
  clear_hip_error();
  hipLaunchKernelGGL(rotate16_kernel<MM>, dim3(MM, batch), dim3(threads), lds, st, x, signs, q, n,
                     logk, scale, y);
  return launch_status();
}

template <int MMAX>
int launch_rotate(const uint16_t* x, const uint32_t* signs, const float* q, int n, int m,
                  uint16_t* y, int batch, hipStream_t st) {
  const int k = n / m;
  int logk = 0;
  while ((1 << logk) < k) ++logk;
  if (logk > 15) return LVQ_E_SHAPE;
  const size_t lds = (MMAX > 1 ? (((size_t)n * 2 + 15) & ~(size_t)15) + (size_t)k * 4
                               : (logk > 9 ? (size_t)k * 4 : 0));
  if (lds > device_lds_bytes()) return LVQ_E_SHAPE;
  // one lane per 8 values (and for m > 1 enough to stage x), whole waves
  const int cw = k < 8 ? k : 8;
  int want = k / cw;
  if (MMAX > 1 && k > want) want = k;
  if (logk > 9 && (k >> (logk - 9 < 4 ? logk - 9 : 4)) > want)
    want = k >> (logk - 9 < 4 ? logk - 9 : 4);
  int threads = (want + kWave - 1) / kWave * kWave;
  if (threads < kWave) threads = kWave;
  if (threads > kRotThreads) threads = kRotThreads;
  const float scale = (float)(1.0 / __builtin_sqrt((double)k));
  clear_hip_error();
  hipLaunchKernelGGL(rotate_kernel<MMAX>, dim3(MMAX == 1 ? 1 : m, batch), dim3(threads), lds, st,
                     x, signs, q, n, m, logk, scale, y);
  return launch_status();
}

}  // namespace lvq

using namespace lvq;

extern "C" int lvq_rotate(const uint16_t* x, const uint32_t* sign_words, const float* q, int n,
                          int m, uint16_t* y, int batch, void* stream) {
  if (n < 0 || m < 1 || m > kRotMaxM) return LVQ_E_SHAPE;
  int e = check_batch(batch);
  if (e) return e;
  if (n % m) return LVQ_E_SHAPE;
  const int k = n / m;
  if (n && (k & (k - 1))) return LVQ_E_SHAPE;
  if (n && (!x || !y)) return LVQ_E_NULL;
  if (!aligned16(x) || !aligned16(y) || !aligned16(sign_words) || !aligned16(q))
    return LVQ_E_ALIGN;
  // with m > 1 the m workgroups of a row each read all of x and write every
  // m-th element of y, so y must not overlap x
  if (m > 1 && n && (const void*)y < (const void*)(x + (size_t)batch * n) &&
      (const void*)x < (const void*)(y + (size_t)batch * n))
    return LVQ_E_SHAPE;
  if (n == 0) return LVQ_OK;
  hipStream_t st = (hipStream_t)stream;
  if (k >= 16 && m <= 8) {
    switch (m) {
      case 1: return launch_rotate16<1>(x, sign_words, q, n, y, batch, st);
      case 2: return launch_rotate16<2>(x, sign_words, q, n, y, batch, st);
      case 3: return launch_rotate16<3>(x, sign_words, q, n, y, batch, st);
      case 4: return launch_rotate16<4>(x, sign_words, q, n, y, batch, st);
      case 5: return launch_rotate16<5>(x, sign_words, q, n, y, batch, st);
      case 6: return launch_rotate16<6>(x, sign_words, q, n, y, batch, st);
      case 7: return launch_rotate16<7>(x, sign_words, q, n, y, batch, st);
      default: return launch_rotate16<8>(x, sign_words, q, n, y, batch, st);
    }
  }
  if (m == 1) return launch_rotate<1>(x, sign_words, q, n, 1, y, batch, st);
  if (m <= 8) return launch_rotate<8>(x, sign_words, q, n, m, y, batch, st);
  return launch_rotate<kRotMaxM>(x, sign_words, q, n, m, y, batch, st);
}
