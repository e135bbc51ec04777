"""Python binding of liblvq.so (argument marshalling only).

Every computation runs in the library: the C++ expander on the host and the
gfx950 kernels on the device.  This module only converts arguments (numpy
arrays, torch tensors or raw integer pointers) into the C ABI of
include/lvq.h and raises LvqError on a negative status.  PyTorch, when used,
provides device memory and the current stream.  There is no fallback: if the
library is missing, importing this package raises.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblvq.so")

NUM_CLASSES = 302
STREAM_SINK_WORDS = 4096
STREAM_GEOM_SINK_WORDS = 65536
MAX_FUSED = 4
MAX_BATCH = 4

LVQ_OK = 0
LVQ_E_NULL = -1
LVQ_E_SHAPE = -2
LVQ_E_ALIGN = -3
LVQ_E_NOT_LEECH = -4
LVQ_E_NORM = -5
LVQ_E_BATCH = -6
LVQ_E_HIP = -7
LVQ_E_LAYOUT = -8


class LvqError(RuntimeError):
    def __init__(self, code, message, index=None):
        super().__init__("%s (status %d)%s" % (
            message, code, "" if index is None else " at row %d, block %d" % index))
        self.code = code
        self.index = index


def _load():
    # One HIP runtime per process: PyTorch ships its own libamdhip64 (same
    # soname).  Loading torch first makes liblvq.so bind to that runtime, so
    # torch's device pointers and streams are valid in the library.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError("liblvq.so is not built (%s); run python dequant_gemv_lvq_amd/build.py"
                          % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    sig = {
        "lvq_strerror": (ctypes.c_char_p, [i]),
        "lvq_last_error_index": (i, [ctypes.POINTER(i), ctypes.POINTER(i)]),
        "lvq_class_table": (i, [vp]),
        "lvq_layout_bytes": (sz, [i, i]),
        "lvq_expand": (i, [vp, vp, vp, i, i, vp]),
        "lvq_expand_gain": (i, [vp, vp, vp, vp, i, i, vp]),
        "lvq_layout_bytes_lp2": (sz, [i, i]),
        "lvq_expand_lp2": (i, [vp, vp, vp, i, i, vp]),
        "lvq_gemv_lp2": (i, [vp, i, i, vp, vp, i, vp]),
        "lvq_lp2x_exceptions": (i, [vp, i, i, vp]),
        "lvq_layout_bytes_lp2x": (sz, [i, i, sz]),
        "lvq_expand_lp2x": (i, [vp, vp, vp, i, i, sz, vp]),
        "lvq_gemv_lp2x": (i, [vp, i, i, sz, vp, vp, i, vp]),
        "lvq_layout_bytes_direct": (sz, [i, i]),
        "lvq_expand_direct": (i, [vp, vp, vp, i, i, vp]),
        "lvq_gemv_direct": (i, [vp, i, i, vp, vp, i, vp]),
        "lvq_layout_bytes_onehot": (sz, [i, i]),
        "lvq_expand_onehot": (i, [vp, vp, vp, i, i, vp]),
        "lvq_gemv_onehot": (i, [vp, i, i, vp, vp, i, vp]),
        "lvq_rank": (i, [vp, sz, vp]),
        "lvq_unfold": (i, [vp, sz, vp, vp, vp]),
        "lvq_gemv_gain": (i, [vp, i, i, ctypes.c_float, ctypes.c_float, vp, vp, i, vp]),
        "lvq_gemv": (i, [vp, i, i, vp, vp, i, vp]),
        "lvq_gemv_fused": (i, [i, vp, vp, i, vp, vp, i, vp]),
        "lvq_gemv_noweights": (i, [vp, i, i, vp, vp, i, vp]),
        "lvq_decode": (i, [vp, i, i, vp, vp]),
        "bpdq_gemv": (i, [vp, vp, i, i, vp, vp, i, vp]),
        "trellis_gemv": (i, [vp, vp, vp, i, i, vp, vp, i, vp]),
        "fp16_gemv": (i, [vp, i, i, vp, vp, i, vp]),
        "lvq_rotate": (i, [vp, vp, vp, i, i, vp, i, vp]),
        "lvq_gemv_rotated": (i, [vp, i, i, vp, vp, i, vp, vp, i, vp]),
        "lvq_stream_read": (i, [vp, sz, vp, vp]),
        "lvq_stream_read_geom": (i, [vp, sz, vp, i, i, i, i, vp]),
        "lvq_gemv_launch_info": (i, [i, i, i, i, i, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()
EXPORTED = ("lvq_strerror", "lvq_last_error_index", "lvq_class_table", "lvq_layout_bytes",
            "lvq_expand", "lvq_expand_gain", "lvq_layout_bytes_lp2", "lvq_expand_lp2",
            "lvq_gemv_lp2", "lvq_lp2x_exceptions", "lvq_layout_bytes_lp2x", "lvq_expand_lp2x",
            "lvq_gemv_lp2x", "lvq_layout_bytes_direct", "lvq_expand_direct", "lvq_gemv_direct",
            "lvq_layout_bytes_onehot", "lvq_expand_onehot", "lvq_gemv_onehot",
            "lvq_rank", "lvq_gemv", "lvq_gemv_gain",
            "lvq_unfold", "lvq_gemv_fused", "lvq_gemv_noweights", "lvq_decode",
            "bpdq_gemv", "trellis_gemv", "fp16_gemv", "lvq_rotate", "lvq_gemv_rotated",
            "lvq_stream_read", "lvq_stream_read_geom", "lvq_gemv_launch_info")


def library():
    return _lib


def strerror(code: int) -> str:
    return _lib.lvq_strerror(int(code)).decode()


def _check(code: int, index=None):
    if code != LVQ_OK:
        raise LvqError(code, strerror(code), index)


def _ptr(a):
    """Device or host address of a torch tensor, numpy array, int or None."""
    if a is None:
        return None
    if isinstance(a, int):
        return a
    if isinstance(a, np.ndarray):
        if not a.flags["C_CONTIGUOUS"]:
            raise ValueError("array must be C-contiguous")
        return a.ctypes.data
    if hasattr(a, "data_ptr"):
        if not a.is_contiguous():
            raise ValueError("tensor must be contiguous")
        return a.data_ptr()
    raise TypeError("unsupported argument type %r" % type(a))


def _stream(stream):
    if stream is None:
        try:
            import torch
            return torch.cuda.current_stream().cuda_stream
        except Exception:
            return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ------------------------------------------------------------------ host side

def class_table() -> np.ndarray:
    out = np.zeros(NUM_CLASSES, dtype=np.uint64)
    _check(_lib.lvq_class_table(out.ctypes.data))
    return out


def layout_bytes(rows: int, cols: int) -> int:
    return int(_lib.lvq_layout_bytes(int(rows), int(cols)))


def _host_inputs(coords, scale, tail, rows: int, cols: int):
    """The host expanders' inputs as contiguous arrays of the exact sizes the
    C expanders read (coords int8 rows*(cols//24)*24, scale uint16 rows, tail
    uint16 rows*(cols%24) or None when cols%24 == 0); LvqError(LVQ_E_SHAPE)
    otherwise, before any native call, so a short array is never read past."""
    if rows < 0 or cols < 0:
        _check(LVQ_E_SHAPE)
    coords = np.ascontiguousarray(coords, dtype=np.int8)
    scale = np.ascontiguousarray(scale, dtype=np.uint16)
    tau = cols % 24
    if tau and tail is None:
        _check(LVQ_E_SHAPE)
    tail = None if tau == 0 else np.ascontiguousarray(tail, dtype=np.uint16)
    if coords.size != rows * (cols // 24) * 24 or scale.size != rows or (
            tail is not None and tail.size != rows * tau):
        _check(LVQ_E_SHAPE)
    return coords, scale, tail


def expand(coords, scale, tail, rows: int, cols: int) -> np.ndarray:
    """Host expansion: coords int8 [rows][cols//24][24], scale/tail fp16 bits
    (uint16) -> packed blob (uint8, lvq_layout_bytes long)."""
    coords, scale, tail = _host_inputs(coords, scale, tail, rows, cols)
    blob = np.empty(_lib.lvq_layout_bytes(int(rows), int(cols)), dtype=np.uint8)
    code = _lib.lvq_expand(_ptr(coords), _ptr(scale), _ptr(tail), int(rows), int(cols),
                           blob.ctypes.data)
    if code != LVQ_OK:
        r, b = ctypes.c_int(), ctypes.c_int()
        _lib.lvq_last_error_index(ctypes.byref(r), ctypes.byref(b))
        _check(code, (r.value, b.value))
    return blob


def layout_bytes_lp2(rows: int, cols: int) -> int:
    return int(_lib.lvq_layout_bytes_lp2(int(rows), int(cols)))


def expand_lp2(coords, scale, tail, rows: int, cols: int) -> np.ndarray:
    """Host expansion into the LP2 layout (two rank planes, class in the record)."""
    coords, scale, tail = _host_inputs(coords, scale, tail, rows, cols)
    blob = np.empty(_lib.lvq_layout_bytes_lp2(int(rows), int(cols)), dtype=np.uint8)
    code = _lib.lvq_expand_lp2(_ptr(coords), _ptr(scale), _ptr(tail), int(rows), int(cols),
                               blob.ctypes.data)
    if code != LVQ_OK:
        r, b = ctypes.c_int(), ctypes.c_int()
        _lib.lvq_last_error_index(ctypes.byref(r), ctypes.byref(b))
        _check(code, (r.value, b.value))
    return blob


def layout_bytes_direct(rows: int, cols: int) -> int:
    return int(_lib.lvq_layout_bytes_direct(int(rows), int(cols)))


def layout_bytes_onehot(rows: int, cols: int) -> int:
    return int(_lib.lvq_layout_bytes_onehot(int(rows), int(cols)))


def expand_onehot(coords, scale, tail, rows: int, cols: int) -> np.ndarray:
    """Host expansion into the one-hot layout (rank-indicator masks)."""
    return _expand_with(_lib.lvq_expand_onehot, _lib.lvq_layout_bytes_onehot, coords, scale,
                        tail, rows, cols)


def expand_direct(coords, scale, tail, rows: int, cols: int) -> np.ndarray:
    """Host expansion into the direct layout (|x| = 2e + parity, no table)."""
    return _expand_with(_lib.lvq_expand_direct, _lib.lvq_layout_bytes_direct, coords, scale,
                        tail, rows, cols)


def _expand_with(expand, nbytes, coords, scale, tail, rows: int, cols: int) -> np.ndarray:
    coords, scale, tail = _host_inputs(coords, scale, tail, rows, cols)
    blob = np.empty(nbytes(int(rows), int(cols)), dtype=np.uint8)
    code = expand(_ptr(coords), _ptr(scale), _ptr(tail), int(rows), int(cols), blob.ctypes.data)
    if code != LVQ_OK:
        r, b = ctypes.c_int(), ctypes.c_int()
        _lib.lvq_last_error_index(ctypes.byref(r), ctypes.byref(b))
        _check(code, (r.value, b.value))
    return blob


def expand_lp2x(coords, scale, tail, rows: int, cols: int) -> tuple:
    """Host expansion into LP2X; returns (blob, number of side-channel blocks)."""
    coords, scale, tail = _host_inputs(coords, scale, tail, rows, cols)
    n = ctypes.c_size_t()
    code = _lib.lvq_lp2x_exceptions(_ptr(coords), int(rows), int(cols), ctypes.byref(n))
    if code == LVQ_OK:
        blob = np.empty(_lib.lvq_layout_bytes_lp2x(int(rows), int(cols), n.value), dtype=np.uint8)
        code = _lib.lvq_expand_lp2x(_ptr(coords), _ptr(scale), _ptr(tail), int(rows), int(cols),
                                    n.value, blob.ctypes.data)
    if code != LVQ_OK:
        r, b = ctypes.c_int(), ctypes.c_int()
        _lib.lvq_last_error_index(ctypes.byref(r), ctypes.byref(b))
        _check(code, (r.value, b.value))
    return blob, n.value


def expand_gain(coords, gain_bits, scale, tail, rows: int, cols: int) -> np.ndarray:
    """lvq_expand with a shape-gain bit per block (uint8 [rows][cols//24])."""
    coords, scale, tail = _host_inputs(coords, scale, tail, rows, cols)
    gain_bits = np.ascontiguousarray(gain_bits, dtype=np.uint8)
    if gain_bits.size != rows * (cols // 24):
        _check(LVQ_E_SHAPE)
    blob = np.empty(_lib.lvq_layout_bytes(int(rows), int(cols)), dtype=np.uint8)
    code = _lib.lvq_expand_gain(_ptr(coords), _ptr(gain_bits), _ptr(scale), _ptr(tail),
                                int(rows), int(cols), blob.ctypes.data)
    if code != LVQ_OK:
        r, b = ctypes.c_int(), ctypes.c_int()
        _lib.lvq_last_error_index(ctypes.byref(r), ctypes.byref(b))
        _check(code, (r.value, b.value))
    return blob


def rank(coords) -> np.ndarray:
    """47-bit index of each block: int8 [..., 24] -> uint64 [...]."""
    coords = np.ascontiguousarray(coords, dtype=np.int8)
    n = coords.size // 24
    out = np.empty(n, dtype=np.uint64)
    _check(_lib.lvq_rank(_ptr(coords), n, out.ctypes.data))
    return out.reshape(coords.shape[:-1])


def last_error_index():
    r, b = ctypes.c_int(), ctypes.c_int()
    _check(_lib.lvq_last_error_index(ctypes.byref(r), ctypes.byref(b)))
    return r.value, b.value


# ------------------------------------------------------------------ device side

def gemv(blob, rows: int, cols: int, x, y, batch: int = 1, stream=None):
    _check(_lib.lvq_gemv(_ptr(blob), int(rows), int(cols), _ptr(x), _ptr(y), int(batch),
                         _stream(stream)))


def gemv_fused(blobs, rows, cols: int, x, ys, batch: int = 1, stream=None):
    """One launch for len(blobs) matrices sharing x: ys[m] = W_m x."""
    n = len(blobs)
    if len(rows) != n or len(ys) != n:
        raise ValueError("blobs, rows and ys must have the same length")
    bp = (ctypes.c_void_p * max(n, 1))(*[_ptr(b) for b in blobs])
    rp = (ctypes.c_int * max(n, 1))(*[int(r) for r in rows])
    yp = (ctypes.c_void_p * max(n, 1))(*[_ptr(y) for y in ys])
    _check(_lib.lvq_gemv_fused(int(n), bp, rp, int(cols), _ptr(x), yp, int(batch),
                               _stream(stream)))


def gemv_noweights(blob, rows: int, cols: int, x, y, batch: int = 1, stream=None):
    """No-weights control: lvq_gemv's launch for this shape reading no weight
    bytes (y = 0); blob only supplies the class table."""
    _check(_lib.lvq_gemv_noweights(_ptr(blob), int(rows), int(cols), _ptr(x), _ptr(y),
                                   int(batch), _stream(stream)))


def gemv_lp2(blob, rows: int, cols: int, x, y, batch: int = 1, stream=None):
    _check(_lib.lvq_gemv_lp2(_ptr(blob), int(rows), int(cols), _ptr(x), _ptr(y), int(batch),
                             _stream(stream)))


def gemv_onehot(blob, rows: int, cols: int, x, y, batch: int = 1, stream=None):
    _check(_lib.lvq_gemv_onehot(_ptr(blob), int(rows), int(cols), _ptr(x), _ptr(y), int(batch),
                                _stream(stream)))


def gemv_direct(blob, rows: int, cols: int, x, y, batch: int = 1, stream=None):
    _check(_lib.lvq_gemv_direct(_ptr(blob), int(rows), int(cols), _ptr(x), _ptr(y), int(batch),
                                _stream(stream)))


def gemv_lp2x(blob, rows: int, cols: int, n_exceptions: int, x, y, batch: int = 1,
              stream=None):
    _check(_lib.lvq_gemv_lp2x(_ptr(blob), int(rows), int(cols), int(n_exceptions), _ptr(x),
                              _ptr(y), int(batch), _stream(stream)))


def gemv_gain(blob, rows: int, cols: int, gain0: float, gain1: float, x, y, batch: int = 1,
              stream=None):
    _check(_lib.lvq_gemv_gain(_ptr(blob), int(rows), int(cols), float(gain0), float(gain1),
                              _ptr(x), _ptr(y), int(batch), _stream(stream)))


def unfold(words, nblocks: int, coords_out, gain_out, stream=None):
    """48-bit words (device uint64) -> coordinates int8 [n][24] and gain bits
    (0xFF marks an invalid word)."""
    _check(_lib.lvq_unfold(_ptr(words), int(nblocks), _ptr(coords_out), _ptr(gain_out),
                           _stream(stream)))


def decode(blob, rows: int, cols: int, out, stream=None):
    _check(_lib.lvq_decode(_ptr(blob), int(rows), int(cols), _ptr(out), _stream(stream)))


def bpdq_gemv(codes, coeffs, rows: int, cols: int, x, y, batch: int = 1, stream=None):
    _check(_lib.bpdq_gemv(_ptr(codes), _ptr(coeffs), int(rows), int(cols), _ptr(x), _ptr(y),
                          int(batch), _stream(stream)))


def trellis_gemv(bits, table, scale, rows: int, cols: int, x, y, batch: int = 1, stream=None):
    _check(_lib.trellis_gemv(_ptr(bits), _ptr(table), _ptr(scale), int(rows), int(cols), _ptr(x),
                             _ptr(y), int(batch), _stream(stream)))


def fp16_gemv(w, rows: int, cols: int, x, y, batch: int = 1, stream=None):
    _check(_lib.fp16_gemv(_ptr(w), int(rows), int(cols), _ptr(x), _ptr(y), int(batch),
                          _stream(stream)))


def rotate(x, n: int, m: int, sign_words, q, y, batch: int = 1, stream=None):
    """y = (H kron Q)(S x) per batch row (fp16 in, fp16 out; y may be x)."""
    _check(_lib.lvq_rotate(_ptr(x), _ptr(sign_words), _ptr(q), int(n), int(m), _ptr(y),
                           int(batch), _stream(stream)))


def gemv_rotated(blob, rows: int, cols: int, sign_words, q, m: int, x, y, batch: int = 1,
                 stream=None):
    """y = W (H kron Q)(S x) in one launch (the rotation of rotate())."""
    _check(_lib.lvq_gemv_rotated(_ptr(blob), int(rows), int(cols), _ptr(sign_words), _ptr(q),
                                 int(m), _ptr(x), _ptr(y), int(batch), _stream(stream)))


def stream_read(buf, nbytes: int, sink, stream=None):
    """Measurement hook: read nbytes of buf once; the XOR of the STREAM_SINK_WORDS
    words of sink (cleared by the caller) is the XOR of the buffer's words."""
    _check(_lib.lvq_stream_read(_ptr(buf), int(nbytes), _ptr(sink), _stream(stream)))


def stream_read_geom(buf, nbytes: int, sink, threads: int, wgs_per_cu: int, unroll: int,
                     nontemporal: bool, stream=None):
    """Measurement hook: the read of stream_read with the launch shape given
    (threads per workgroup, workgroups per CU or 0 for one trip per thread,
    16-byte loads in flight per thread, non-temporal loads or not); sink has
    STREAM_GEOM_SINK_WORDS words, cleared by the caller."""
    _check(_lib.lvq_stream_read_geom(_ptr(buf), int(nbytes), _ptr(sink), int(threads),
                                     int(wgs_per_cu), int(unroll), int(bool(nontemporal)),
                                     _stream(stream)))


LAUNCH_KINDS = {"gemv": 0, "rotated": 1, "direct": 2, "onehot": 3, "lp2": 4, "gain": 5,
                "noweights": 6}


def gemv_launch_info(kind: str, rows: int, cols: int, batch: int = 1, m: int = 1) -> dict:
    """The launch a Leech GEMV entry point makes for this shape (nothing is
    launched): threads, workgroups, blocks per lane, ring depth, LDS bytes."""
    out = (ctypes.c_int * 5)()
    _check(_lib.lvq_gemv_launch_info(LAUNCH_KINDS[kind], int(rows), int(cols), int(batch),
                                     int(m), out))
    return {"threads": out[0], "workgroups": out[1], "blocks_per_lane": out[2],
            "ring": out[3], "lds_bytes": out[4]}
