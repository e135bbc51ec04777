"""f64 activation rotation (oracle; test infrastructure).

Sources.  arXiv 2609.02652 keeps the weights in an incoherence-rotated basis,
so every projection first applies a Walsh-Hadamard transform to its input
activation, held whole in one thread block's shared memory (setup paragraph
of the served-path section, and the paragraph on the rotated basis and the
shared-memory wall).  That fixes the power-of-two case only: one
Walsh-Hadamard transform over the whole input (m = 1 below).  For widths that
are not powers of two (9,728, 17,408 and 25,600 in the Qwen3 family) this
module borrows the form of another system: the blog post "Qwen3.8-27B on a
12 GB card" (section "What the kernel does per token") gives the runtime
rotation of Mirai S, a QTIP-style trellis model, as x_rot = (H kron Q)(S x),
with S random signs, H a 1024- or 2048-point Walsh-Hadamard transform and Q
a small orthogonal matrix (5 x 5 for 5120 = 5 x 1024, 3 x 3 for
6144 = 3 x 2048).  The paper names none of S, Q or that factorisation.

Reading (the pages fix neither the normalisation nor the index order):
  n = K * m with K a power of two; coordinate i = a * m + b (a < K, b < m);
  H is the Sylvester matrix H[a][c] = (-1)^popcount(a & c), scaled by
  1 / sqrt(K) so that the transform is orthogonal when Q is;
  (H kron Q)[(a, b), (c, d)] = H[a][c] * Q[b][d]  (numpy.kron's order);
  S negates coordinate j when bit j % 32 of sign word j / 32 is set;
  Q = identity when none is given (then the transform is block-diagonal with
  m interleaved K-point transforms).

  y[a*m + b] = K^-1/2 * sum_c H[a][c] * sum_d Q[b][d] * s_(c*m+d) * x_(c*m+d)

The Walsh-Hadamard step is the textbook butterfly recursion (pairs at distance
h, 2h, 4h, ... replaced by their sum and difference); Q is applied with numpy's
float64 matmul.  Pinned in tests/test_oracle_rotate.py against scipy's
Hadamard matrix, numpy.kron, H H^T = K I, orthogonality and involution.
"""
import numpy as np

from .gemv import f16


def is_pow2(k: int) -> bool:
    return k >= 1 and (k & (k - 1)) == 0


def sign_vector(sign_words, n: int) -> np.ndarray:
    """+1 / -1 per coordinate from the packed sign words (None: all +1)."""
    if sign_words is None:
        return np.ones(n)
    w = np.asarray(sign_words, dtype=np.uint32)
    j = np.arange(n)
    bits = (w[j // 32] >> (j % 32).astype(np.uint32)) & 1
    return np.where(bits == 1, -1.0, 1.0)


def fwht(v: np.ndarray, axis: int = -1) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform along `axis` (length a power of
    two), float64: for h = 1, 2, 4, ..., every pair (i, i + h) inside each
    block of 2h becomes (v_i + v_(i+h), v_i - v_(i+h))."""
    v = np.moveaxis(np.array(v, dtype=np.float64), axis, -1)
    k = v.shape[-1]
    assert is_pow2(k)
    lead = v.shape[:-1]
    h = 1
    while h < k:
        blocks = v.reshape(lead + (k // (2 * h), 2, h))
        lo, hi = blocks[..., 0, :].copy(), blocks[..., 1, :].copy()
        blocks[..., 0, :] = lo + hi
        blocks[..., 1, :] = lo - hi
        v = blocks.reshape(lead + (k,))
        h *= 2
    return np.moveaxis(v, -1, axis)


def rotate(x_bits, n: int, m: int = 1, sign_words=None, q=None) -> tuple:
    """x fp16 bits [batch][n] -> (y, bound), float64 [batch][n]:
    y = (H kron Q)(S x) with H = K^-1/2 Sylvester, and
    bound = K^-1/2 * sum_c sum_d |Q[b][d]| |x_(c*m+d)|, the sum of the
    magnitudes of the terms of each output (the scale of its rounding error)."""
    assert m >= 1 and n % m == 0 and is_pow2(n // m)
    k = n // m
    x = f16(x_bits).reshape(-1, n)
    qm = np.eye(m) if q is None else np.asarray(q, dtype=np.float64).reshape(m, m)
    z = (x * sign_vector(sign_words, n)).reshape(-1, k, m)
    z = z @ qm.T                      # z[c][b] = sum_d Q[b][d] (Sx)[c*m + d]
    y = fwht(z, axis=1) / np.sqrt(k)  # across the K groups, for each b
    za = np.abs(x).reshape(-1, k, m) @ np.abs(qm).T
    bound = np.broadcast_to(za.sum(axis=1, keepdims=True), za.shape) / np.sqrt(k)
    return y.reshape(-1, n), np.array(bound).reshape(-1, n)


def ulp16(v) -> np.ndarray:
    """Spacing of fp16 numbers at |v| (2^-24 below the normal range)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


# fp32 arithmetic on the device: about log2(K) + m roundings per output, each
# at most 2^-24 of the running magnitude; 1e-5 of the bound leaves margin
ROT_REL_TOL = 1e-5


def rotate_check(y_dev_bits, y64, bound) -> float:
    """Largest |y_dev - y64| / (ulp16(y64) + 1e-5 * bound) over the outputs;
    the device result is an fp16 rounding of an fp32 computation, so the bar
    (<= 1) allows one fp16 ulp of rounding plus the fp32 error."""
    y = f16(y_dev_bits).reshape(y64.shape)
    tol = ulp16(y64) + ROT_REL_TOL * bound
    r = np.abs(y - y64) / tol
    return float(r.max()) if r.size else 0.0
