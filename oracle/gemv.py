"""f64 reconstruction of W for every arm, the matvec, and the per-row bound
(oracle; test infrastructure).

The method computes exactly y = W x (only faster), so the oracle is that
definition written out: rebuild W in float64 from the stored values (int8
lattice coordinates, fp16 scales, tails, coefficients and tables, each
converted exactly) and multiply by x (fp16 converted exactly).  numpy's float64
matmul is the one library primitive used; for tiny shapes the tests re-derive
y in exact rational arithmetic.

Arms and their sources:
  leech    arXiv 2609.02652, section 1: 24-weight blocks are Leech points with
           one scale per row; the Tetra summary (arXiv 2609.35465, section 5.1)
           says the kernel applies the row scale and then adds the unquantized
           tail.  Reading: w = s_r * x_int, the tail (K mod 24 columns) is fp16
           and unscaled.
  bpdq     model card "Qwen3-8B - 2-bit BPDQ (packed)", section Format:
           w[r,c] = sum_i coeffs[g(c), r, i] * bit_i(r, c) + coeffs[g(c), r, 2],
           two bit planes, group size 256, the "Elsewhere" layout
           codes int32 [in/16, out] with a column's two bits interleaved into
           one 2-bit code that is peeled low bits first.  Reading: bit_i is bit
           i of that code; coeffs are fp16 [groups, 3, out].
  trellis  blog "Qwen3.8-27B on a 12 GB card", section "A trellis is a codebook
           you walk": a position's state is the L-bit window of the code
           stream that ends at its symbol (T bits per symbol, V weights per
           symbol).  Here L=16, T=2, V=1; a weight is s_r * table[state];
           packets restart every 256 columns.
           Readings (parity unpinned beyond the pins listed in the tests):
           symbols are read MSB-first within each 32-bit word, and a packet is
           tail-biting (the 7 symbols before symbol 0 are the packet's last 7).
  fp16     the dense control: w = W[r, c].
"""
import numpy as np

REL_TOL = 1e-4


def f16(bits) -> np.ndarray:
    """uint16 fp16 bit patterns -> float64 values (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


# --------------------------------------------------------------------------
# Leech
# --------------------------------------------------------------------------

def leech_weights(coords, scale_bits, tail_bits, cols: int) -> np.ndarray:
    """coords int8 [R][nb][24], scale fp16 bits [R], tail fp16 bits [R][cols%24]."""
    coords = np.asarray(coords)
    rows = coords.shape[0]
    nb = cols // 24
    tau = cols - 24 * nb
    assert coords.shape == (rows, nb, 24)
    w = np.empty((rows, cols), dtype=np.float64)
    s = f16(scale_bits).reshape(rows, 1)
    w[:, : 24 * nb] = coords.reshape(rows, 24 * nb).astype(np.float64) * s
    if tau:
        w[:, 24 * nb:] = f16(tail_bits).reshape(rows, tau)
    return w


# --------------------------------------------------------------------------
# BPDQ
# --------------------------------------------------------------------------

def bpdq_codes(codes, rows: int, cols: int) -> np.ndarray:
    """The 2-bit code of every weight, [R][K]: column c of row r sits in word
    codes[c // 16, r] at bits 2*(c % 16) .. 2*(c % 16) + 1."""
    codes = np.asarray(codes, dtype=np.uint32)
    assert codes.shape == (cols // 16, rows)
    out = np.empty((rows, cols), dtype=np.uint8)
    for c in range(16):
        out[:, c::16] = ((codes >> np.uint32(2 * c)) & np.uint32(3)).T
    return out


def bpdq_weights(codes, coeff_bits, rows: int, cols: int, group: int = 256) -> np.ndarray:
    code = bpdq_codes(codes, rows, cols)
    coeffs = f16(coeff_bits).reshape(cols // group, 3, rows)
    g = np.arange(cols) // group
    c0 = coeffs[g, 0, :].T
    c1 = coeffs[g, 1, :].T
    c2 = coeffs[g, 2, :].T
    b0 = (code & 1).astype(np.float64)
    b1 = ((code >> 1) & 1).astype(np.float64)
    return c0 * b0 + c1 * b1 + c2


# --------------------------------------------------------------------------
# bitshift trellis
# --------------------------------------------------------------------------

TRELLIS_L = 16
TRELLIS_T = 2
TRELLIS_PACKET = 256


def shift_state(prev: int, symbol: int, t_bits: int = TRELLIS_T, l_bits: int = TRELLIS_L) -> int:
    """One trellis step: shift T new bits into an L-bit state (newest lowest)."""
    return ((prev << t_bits) | symbol) & ((1 << l_bits) - 1)


def trellis_symbols(bits, rows: int, cols: int) -> np.ndarray:
    """2-bit symbols [R][K]: symbol k of a row is read MSB-first from word k//16."""
    words = np.asarray(bits, dtype=np.uint32).reshape(rows, cols // 16)
    out = np.empty((rows, cols), dtype=np.uint8)
    for p in range(16):
        out[:, p::16] = (words >> np.uint32(30 - 2 * p)) & np.uint32(3)
    return out


def trellis_states(bits, rows: int, cols: int) -> np.ndarray:
    """16-bit state of every weight, [R][K], as the window of the last 8
    symbols of the (circular) 256-symbol packet ending at that weight."""
    sym = trellis_symbols(bits, rows, cols).astype(np.uint32)
    per = TRELLIS_L // TRELLIS_T
    pk = sym.reshape(rows, cols // TRELLIS_PACKET, TRELLIS_PACKET)
    state = np.zeros_like(pk)
    for i in range(per):  # symbol k-i lands at bits 2i..2i+1
        state |= np.roll(pk, i, axis=2) << np.uint32(TRELLIS_T * i)
    return state.reshape(rows, cols)


def trellis_states_walk(packet_symbols) -> list:
    """The same states by walking the shift register (tail-biting start);
    plain Python, for small cross-checks."""
    n = len(packet_symbols)
    per = TRELLIS_L // TRELLIS_T
    state = 0
    out = []
    for k in range(-(per - 1), n):
        state = shift_state(state, int(packet_symbols[k % n]))
        if k >= 0:
            out.append(state)
    return out


def trellis_weights(bits, table_bits, scale_bits, rows: int, cols: int) -> np.ndarray:
    table = f16(table_bits)
    assert table.shape == (1 << TRELLIS_L,)
    st = trellis_states(bits, rows, cols)
    return table[st] * f16(scale_bits).reshape(rows, 1)


# --------------------------------------------------------------------------
# dense control
# --------------------------------------------------------------------------

def fp16_weights(w_bits, rows: int, cols: int) -> np.ndarray:
    return f16(w_bits).reshape(rows, cols)


# --------------------------------------------------------------------------
# matvec and the per-row bound
# --------------------------------------------------------------------------

def gemv(w: np.ndarray, x_bits) -> tuple:
    """y[b, r] = sum_c w[r, c] x[b, c] and bound[b, r] = sum_c |w[r, c] x[b, c]|,
    both in float64; x is fp16 bits [batch][K]."""
    x = f16(x_bits)
    x = x.reshape(-1, w.shape[1])
    y = x @ w.T
    bound = np.abs(x) @ np.abs(w).T
    return y, bound


def parity_ratio(y_dev, y64, bound, rel: float = REL_TOL) -> np.ndarray:
    """|y_dev - y64| / (rel * bound) per element; rows with bound 0 must be
    exactly 0 (ratio 0), any other value there gives inf."""
    y_dev = np.asarray(y_dev, dtype=np.float64).reshape(y64.shape)
    err = np.abs(y_dev - y64)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = err / (rel * bound)
    zero = bound == 0
    r[zero] = np.where(y_dev[zero] == 0, 0.0, np.inf)
    return r


def check(y_dev, y64, bound, rel: float = REL_TOL) -> float:
    """Largest parity ratio; the bar is met when it is <= 1."""
    r = parity_ratio(y_dev, y64, bound, rel)
    return float(r.max()) if r.size else 0.0
