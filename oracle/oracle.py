"""ctypes binding of the fp64 CPU oracle in nvfp4_oracle.c (test infrastructure only).

Every function here marshals numpy arrays into the C oracle and back; the
arithmetic is all in nvfp4_oracle.c, which states what it computes and why.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build():
    """Compile the oracle with gcc: plain -O2, no fast-math, OpenMP."""
    cmd = ["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Wextra", _SRC, "-o", _LIB_PATH + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.nvo_e2m1.restype = ctypes.c_double
    lib.nvo_e2m1.argtypes = [ctypes.c_uint32]
    lib.nvo_e4m3.restype = ctypes.c_double
    lib.nvo_e4m3.argtypes = [ctypes.c_uint32]
    lib.nvo_bf16.restype = ctypes.c_double
    lib.nvo_bf16.argtypes = [ctypes.c_uint16]
    lib.nvo_silu.restype = ctypes.c_double
    lib.nvo_silu.argtypes = [ctypes.c_double]
    lib.nvo_dequant.restype = None
    lib.nvo_dequant.argtypes = [P, P, i64, i64, ctypes.c_float, P]
    lib.nvo_gemm.restype = None
    lib.nvo_gemm.argtypes = [P, P, i64, i64, ctypes.c_float, P, i64, i64, P, i64, P, P, ctypes.c_int]
    lib.nvo_route.restype = None
    lib.nvo_route.argtypes = [P, i64, i64, i64, P, P]
    lib.nvo_group.restype = None
    lib.nvo_group.argtypes = [P, i64, i64, i64, P, P, P, P]
    lib.nvo_moe.restype = None
    lib.nvo_moe.argtypes = [P, P, P, P, P, P, P, P, P, P, P, i64, i64, i64, i64, i64, P, P, P, P, ctypes.c_int]
    lib.nvo_tensor_scale.restype = ctypes.c_float
    lib.nvo_tensor_scale.argtypes = [P, ctypes.c_int, i64, i64, i64]
    lib.nvo_quantize.restype = None
    lib.nvo_quantize.argtypes = [P, ctypes.c_int, i64, i64, i64, ctypes.c_float, P, P]
    lib.nvo_mx_from_nvfp4.restype = None
    lib.nvo_mx_from_nvfp4.argtypes = [P, P, i64, i64, P, P]
    lib.nvo_mx_from_bf16.restype = None
    lib.nvo_mx_from_bf16.argtypes = [P, i64, i64, i64, P, P]
    lib.nvo_mx_gemm.restype = None
    lib.nvo_mx_gemm.argtypes = [P, P, i64, i64, ctypes.c_float, P, P, i64, P, i64, P, P, ctypes.c_int]
    lib.nvo_max_threads.restype = ctypes.c_int
    lib.nvo_max_threads.argtypes = []
    _lib = lib
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def max_threads():
    return int(_load().nvo_max_threads())


def _threads(nthreads):
    if nthreads is None:
        try:
            return len(os.sched_getaffinity(0))
        except AttributeError:  # pragma: no cover
            return os.cpu_count() or 1
    return int(nthreads)


def e2m1(codes):
    """Decode 4-bit E2M1 codes (any integer array with values 0..15) to fp64."""
    lib = _load()
    c = np.asarray(codes)
    return np.array([lib.nvo_e2m1(int(v)) for v in c.ravel()], dtype=np.float64).reshape(c.shape)


def e4m3(byts):
    """Decode E4M3FN bytes to fp64 (NaN for 0x7F / 0xFF)."""
    lib = _load()
    b = np.asarray(byts)
    return np.array([lib.nvo_e4m3(int(v)) for v in b.ravel()], dtype=np.float64).reshape(b.shape)


def bf16_to_f64(bits):
    lib = _load()
    b = np.asarray(bits)
    return np.array([lib.nvo_bf16(int(v)) for v in b.ravel()], dtype=np.float64).reshape(b.shape)


def silu(z):
    lib = _load()
    z = np.asarray(z, dtype=np.float64)
    return np.array([lib.nvo_silu(float(v)) for v in z.ravel()], dtype=np.float64).reshape(z.shape)


def dequant(codes, scales, tensor_scale):
    """W[n][k] = s_t * e2m1 * e4m3 in fp64 from canonical codes [N][K/2] and scales [N][K/16]."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    n, kh = codes.shape
    k = 2 * kh
    assert scales.shape == (n, k // 16)
    w = np.empty((n, k), dtype=np.float64)
    _load().nvo_dequant(_ptr(codes), _ptr(scales), n, k, float(tensor_scale), _ptr(w))
    return w


def gemm(codes, scales, tensor_scale, x_bits, rows=None, nthreads=None):
    """y[m][j] = sum_k W[rows[j]][k] x[m][k] and s[m][j] = sum_k |W x| (fp64).

    x_bits: uint16 bf16 bit patterns, [M][K] (or [K] for one row).
    rows: optional int64 list of output rows to evaluate (default: all).
    Returns (y, s), each [M][nrows].
    """
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    n, kh = codes.shape
    k = 2 * kh
    assert scales.shape == (n, k // 16)
    x = _c(np.atleast_2d(x_bits), np.uint16)
    assert x.shape[1] == k, (x.shape, k)
    m = x.shape[0]
    if rows is None:
        nrows, rp = n, None
    else:
        rows = _c(np.asarray(rows, dtype=np.int64), np.int64)
        assert rows.size == 0 or (rows.min() >= 0 and rows.max() < n)
        nrows, rp = rows.size, _ptr(rows)
    y = np.empty((m, nrows), dtype=np.float64)
    s = np.empty((m, nrows), dtype=np.float64)
    _load().nvo_gemm(_ptr(codes), _ptr(scales), n, k, float(tensor_scale), _ptr(x), m, k,
                     rp, nrows, _ptr(y), _ptr(s), _threads(nthreads))
    return y, s


def route(logits, top_k):
    """Top-k experts per token (descending logit, ties to smaller id) and fp64 softmax weights."""
    logits = _c(logits, np.float32)
    t, e = logits.shape
    assert 1 <= top_k <= e
    ids = np.empty((t, top_k), dtype=np.int32)
    g = np.empty((t, top_k), dtype=np.float64)
    _load().nvo_route(_ptr(logits), t, e, top_k, _ptr(ids), _ptr(g))
    return ids, g


def group(ids, experts):
    """counts [E], offsets [E+1], perm [T*k], pos [T*k] of the stable expert grouping."""
    ids = _c(ids, np.int32)
    t, k = ids.shape
    assert ids.size == 0 or (ids.min() >= 0 and ids.max() < experts)
    counts = np.empty(experts, dtype=np.int32)
    offsets = np.empty(experts + 1, dtype=np.int32)
    perm = np.empty(t * k, dtype=np.int32)
    pos = np.empty(t * k, dtype=np.int32)
    _load().nvo_group(_ptr(ids), t, k, experts, _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(pos))
    return counts, offsets, perm, pos


def moe(gate, up, down, x_bits, logits, top_k, nthreads=None):
    """The whole expert layer in fp64.

    gate, up: (codes [E][I][H/2], scales [E][I][H/16], s_t [E] float32)
    down:     (codes [E][H][I/2], scales [E][H][I/16], s_t [E] float32)
    Returns ids, g, y [T][H], ybound [T][H] (= sum_j g_j sum_i |Wd h_j|).
    """
    gc, gs, sg = (_c(gate[0], np.uint8), _c(gate[1], np.uint8), _c(gate[2], np.float32))
    uc, us, su = (_c(up[0], np.uint8), _c(up[1], np.uint8), _c(up[2], np.float32))
    dc, ds, sd = (_c(down[0], np.uint8), _c(down[1], np.uint8), _c(down[2], np.float32))
    x = _c(x_bits, np.uint16)
    logits = _c(logits, np.float32)
    e, inter, hh = gc.shape
    hidden = 2 * hh
    t = x.shape[0]
    assert x.shape == (t, hidden) and logits.shape == (t, e)
    assert uc.shape == gc.shape and dc.shape == (e, hidden, inter // 2)
    ids = np.empty((t, top_k), dtype=np.int32)
    g = np.empty((t, top_k), dtype=np.float64)
    y = np.empty((t, hidden), dtype=np.float64)
    yb = np.empty((t, hidden), dtype=np.float64)
    _load().nvo_moe(_ptr(gc), _ptr(gs), _ptr(sg), _ptr(uc), _ptr(us), _ptr(su),
                    _ptr(dc), _ptr(ds), _ptr(sd), _ptr(x), _ptr(logits),
                    t, e, top_k, hidden, inter, _ptr(ids), _ptr(g), _ptr(y), _ptr(yb),
                    _threads(nthreads))
    return ids, g, y, yb


def quantize(w, tensor_scale=None, bf16=None):
    """NVFP4-encode an [N][K] matrix: returns (codes [N][K/2] u8, scales [N][K/16] u8, s_t float32).

    w: float32 values, or uint16 bf16 bit patterns (bf16 defaults to w's dtype
    being uint16).  tensor_scale: use this s_t instead of the matrix's own.
    """
    if bf16 is None:
        bf16 = np.asarray(w).dtype == np.uint16
    w = _c(w, np.uint16 if bf16 else np.float32)
    n, k = w.shape
    assert k % 16 == 0
    lib = _load()
    st = np.float32(lib.nvo_tensor_scale(_ptr(w), int(bf16), n, k, k)) if tensor_scale is None \
        else np.float32(tensor_scale)
    codes = np.zeros((n, k // 2), dtype=np.uint8)
    scales = np.zeros((n, k // 16), dtype=np.uint8)
    lib.nvo_quantize(_ptr(w), int(bf16), n, k, k, float(st), _ptr(codes), _ptr(scales))
    return codes, scales, st


def mx_from_nvfp4(codes, scales):
    """MX FP4 requantisation of an NVFP4 matrix (s_t left out): (codes [N][K/2], E8M0 scales [N][K/32])."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    n, kh = codes.shape
    k = 2 * kh
    assert k % 32 == 0 and scales.shape == (n, k // 16)
    mc = np.zeros((n, k // 2), np.uint8)
    ms = np.zeros((n, k // 32), np.uint8)
    _load().nvo_mx_from_nvfp4(_ptr(codes), _ptr(scales), n, k, _ptr(mc), _ptr(ms))
    return mc, ms


def mx_from_bf16(x_bits):
    """MX FP4 quantisation of bf16 activations [M][K]: (codes [M][K/2], E8M0 scales [M][K/32])."""
    x = _c(x_bits, np.uint16)
    m, k = x.shape
    assert k % 32 == 0
    mc = np.zeros((m, k // 2), np.uint8)
    ms = np.zeros((m, k // 32), np.uint8)
    _load().nvo_mx_from_bf16(_ptr(x), m, k, k, _ptr(mc), _ptr(ms))
    return mc, ms


def mx_gemm(wc, ws, tensor_scale, xc, xs, rows=None, nthreads=None):
    """y[m][j] = s_t * sum_k w'[rows[j]][k] x'[m][k] and s = s_t * sum |w' x'| (fp64) over MX operands."""
    wc, ws, xc, xs = _c(wc, np.uint8), _c(ws, np.uint8), _c(xc, np.uint8), _c(xs, np.uint8)
    n, kh = wc.shape
    m = xc.shape[0]
    k = 2 * kh
    r = None if rows is None else _c(rows, np.int64)
    nr = n if r is None else r.size
    y = np.empty((m, nr), np.float64)
    s = np.empty((m, nr), np.float64)
    _load().nvo_mx_gemm(_ptr(wc), _ptr(ws), n, k, float(tensor_scale), _ptr(xc), _ptr(xs), m,
                        None if r is None else _ptr(r), nr, _ptr(y), _ptr(s), _threads(nthreads))
    return y, s
