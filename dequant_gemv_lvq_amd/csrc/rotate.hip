// Activation rotation (lvq_rotate): y = (H kron Q)(S x) before a GEMV.
//
// Sources: arXiv 2609.02652 keeps the weights in an incoherence-rotated basis,
// so each projection's input goes through a Walsh-Hadamard transform first, a
// transform that needs the whole activation resident in one block's shared
// memory (served-path setup, and the section on the rotated basis and the
// shared-memory wall: the widest activation of the largest model needed
// 102,400 B of f32 and did not fit that card).  That fixes the power-of-two
// case (m = 1).  Widths that are not powers of two borrow the form another
// system uses: the blog post "Qwen3.8-27B on a 12 GB card" (section "What the
// kernel does per token") gives Mirai S's runtime rotation as (H kron Q)(S x),
// S random signs, H a power-of-two Walsh-Hadamard transform, Q a small
// orthogonal matrix.
//
// n = K m, K a power of two, coordinate a m + b; H = K^-1/2 times the Sylvester
// matrix ((-1)^popcount(a & c)); Q is m x m (identity when none is given).
//
// gfx950 design.  The m interleaved sequences are independent once Q has mixed
// each group, so one workgroup takes one (batch row, b) pair and one K-point
// transform (K <= 32768); the signs are XORed into the fp16 sign bits as x
// arrives (exact).  Two kernels, which apply every stage's butterflies to the
// same operands in the same order and so give the same bits:
// - K >= 16 and m <= 8 (rotate16_kernel, every Qwen3-family width but the
//   wide ones): a thread takes 16 consecutive values of its sequence, forms
//   their Q mix in registers straight from global memory, runs stages 0-3 in
//   registers, and radix passes over an f32 copy in LDS do the rest.
// - m > 8 or K < 16 (rotate_kernel): the row of x is staged in LDS, each
//   thread forms one output of the Q mix into an f32 sequence in LDS, then
//   stages 0-3 with 16 consecutive values per thread and radix passes; for
//   K < 16 one lane holds the whole sequence.
// The passes for stages 4 and up have consecutive threads on consecutive
// addresses (no bank conflicts) and one barrier each; the last one scales,
// rounds to fp16 and stores.  LDS: 4 K bytes (+ 2 n where x is staged); the widest
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

// Workgroup (b, batch row): y[c m + b] for c < K, for the shapes the 16-value
// kernel below does not take: m > 8, and K < 16.
template <int MMAX>
__global__ void __launch_bounds__(kRotThreads)
rotate_kernel(const uint16_t* x, const uint32_t* __restrict__ signs,
              const float* __restrict__ q, int n, int m, int logk, float scale, uint16_t* y) {
  // y may be x when m = 1: a row's one workgroup reads all of it before its
  // barrier and writes after it (for m > 1 the host refuses overlap)
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int b = MMAX == 1 ? 0 : blockIdx.x;
  const int mm = MMAX == 1 ? 1 : m;
  const int k = n / mm;
  const uint16_t* xr = x + (size_t)blockIdx.y * n;
  uint16_t* yr = y + (size_t)blockIdx.y * n;
  // LDS (m > 1): the staged row of x, then the f32 sequence
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
      for (int j = tid; j < n; j += nthr) xs[j] = xr[j] ^ rot_sign_bit(signs, j);
    }
    // row b of Q: uniform, so scalar loads
    float qrow[MMAX];
#pragma unroll
    for (int d = 0; d < MMAX; ++d)
      qrow[d] = d < m ? (q ? q[b * m + d] : (d == b ? 1.f : 0.f)) : 0.f;
    __syncthreads();
    if (MMAX > 8) {
      // wide groups: a lane reads its group as aligned words (one more than
      // half of MMAX), shifts each pair of halves into place by its own
      // parity, and runs all MMAX terms, those past m masked to +0 (with q 0
      // adding +0 leaves the sum as it is): no branch per term, every read in
      // flight at once.  The reads past the group stay inside the LDS
      // allocation (the host adds 64 bytes after the f32 sequence).
      const uint32_t* xs32 = (const uint32_t*)xs;
      for (int c = tid; c < k; c += nthr) {
        const int h0 = c * m;
        const int w0 = h0 >> 1;
        const uint32_t sh = (uint32_t)(h0 & 1) * 16;
        uint32_t dw[MMAX / 2 + 1];
#pragma unroll
        for (int j = 0; j <= MMAX / 2; ++j) dw[j] = xs32[w0 + j];
        float a = 0.f;
#pragma unroll
        for (int j = 0; j < MMAX / 2; ++j) {
          const uint32_t keep = 2 * j + 1 < m ? 0xFFFFFFFFu : 2 * j < m ? 0xFFFFu : 0u;  // uniform
          const uint32_t pr = __builtin_amdgcn_alignbit(dw[j + 1], dw[j], sh) & keep;
          a = __builtin_fmaf(qrow[2 * j], rot_half((uint16_t)pr), a);
          a = __builtin_fmaf(qrow[2 * j + 1], rot_half((uint16_t)(pr >> 16)), a);
        }
        buf[c] = a;
      }
    } else {
      for (int c = tid; c < k; c += nthr) {
        float a = 0.f;
#pragma unroll
        for (int d = 0; d < MMAX; ++d)
          if (d < m) a = __builtin_fmaf(qrow[d], rot_half(xs[c * m + d]), a);
        buf[c] = a;
      }
    }
    __syncthreads();
    if (logk >= 4) {  // uniform
      // stages 0-3 with 16 consecutive values per thread (16-byte LDS
      // accesses), then radix passes with consecutive threads on consecutive
      // addresses: a barrier per pass, no lane exchanges
      for (int set = tid; set < (k >> 4); set += nthr) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 f = *(const float4*)(buf + 16 * set + 4 * i);
          v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
        }
        rot_set_stages<4>(v);
        if (logk == 4) {
#pragma unroll
          for (int t = 0; t < 16; ++t) yr[(size_t)(16 * set + t) * mm + b] = rot_out(v[t], scale);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            *(float4*)(buf + 16 * set + 4 * i) =
                make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
        }
      }
      for (int s = 4; s < logk; s += 4) {
        __syncthreads();
        const int r = logk - s < 4 ? logk - s : 4;
        const bool last = s + r == logk;
        if (r == 4) rot_high_pass<4>(buf, k, s, last, mm, b, scale, yr, tid, nthr);
        else if (r == 3) rot_high_pass<3>(buf, k, s, last, mm, b, scale, yr, tid, nthr);
        else if (r == 2) rot_high_pass<2>(buf, k, s, last, mm, b, scale, yr, tid, nthr);
        else rot_high_pass<1>(buf, k, s, last, mm, b, scale, yr, tid, nthr);
      }
      return;
    }
  }

  // K < 16: one lane holds the whole sequence (K <= 8 values) and runs every
  // stage in its registers (m = 1 reads x itself, with the signs; m > 1 the
  // Q mix)
  if (tid == 0) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] = 0.f;
      if (i < k)
        v[i] = MMAX == 1 ? rot_half(xr[i] ^ rot_sign_bit(signs, i)) : buf[i];
    }
    rot_reg_stages(v, k);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < k) yr[(size_t)i * mm + b] = rot_out(v[i], scale);
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
  if (MMAX == 1 && k >= 16) return LVQ_E_SHAPE;  // the 16-value kernel's
  // m > 8: 64 bytes after the f32 sequence for the Q mix's reads past x
  const size_t lds =
      MMAX > 1 ? (((size_t)n * 2 + 15) & ~(size_t)15) + (size_t)k * 4 + (MMAX > 8 ? 64 : 0) : 0;
  if (lds > device_lds_bytes()) return LVQ_E_SHAPE;
  // m > 1: one thread per Q-mix output (whole waves); m = 1 (K < 16): one wave
  int threads = MMAX > 1 ? (k + kWave - 1) / kWave * kWave : kWave;
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
