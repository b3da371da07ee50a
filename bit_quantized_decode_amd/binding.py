"""Python binding of libnvfp4.so: the functions of include/nvfp4.h, same names.

Argument marshalling only: torch tensors supply device memory and the current
stream; every step of the computation runs in the library's HIP kernels.  If
the library is not built, every call raises -- there is no fallback path.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

NVFP4_OK = 0
NVFP4_ERR_NULL = 1
NVFP4_ERR_SHAPE = 2
NVFP4_ERR_ALIGN = 3
NVFP4_ERR_DTYPE = 4
NVFP4_ERR_WORKSPACE = 5
NVFP4_ERR_ARG = 6
NVFP4_ERR_HIP = 7
NVFP4_F32 = 0
NVFP4_BF16 = 1

EXPORTED = (
    "nvfp4_abi_version", "nvfp4_status_str", "nvfp4_last_error", "nvfp4_packed_bytes", "nvfp4_pack",
    "nvfp4_unpack", "nvfp4_gemv_workspace_bytes", "nvfp4_gemv", "nvfp4_gemm_workspace_bytes", "nvfp4_gemm",
    "nvfp4_gemv_batched_workspace_bytes", "nvfp4_gemv_batched", "nvfp4_gemm_batched_workspace_bytes",
    "nvfp4_gemm_batched", "nvfp4_moe_workspace_bytes", "nvfp4_moe_grouped", "nvfp4_quantize_workspace_bytes",
    "nvfp4_quantize", "nvfp4_expert_cache_reset", "nvfp4_moe_streamed", "nvfp4_mx_packed_bytes", "nvfp4_mx_pack",
    "nvfp4_mx_unpack", "nvfp4_w4a4_workspace_bytes", "nvfp4_w4a4_gemm", "nvfp4_w4a4_batched_workspace_bytes",
    "nvfp4_w4a4_batched", "nvfp4_gemv_batched_noalloc",
)


class Nvfp4Error(RuntimeError):
    def __init__(self, status, message):
        super().__init__(message)
        self.status = status


class Problem(ctypes.Structure):
    """Mirror of struct nvfp4_problem."""
    _fields_ = [
        ("packed", ctypes.c_void_p), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
        ("tensor_scale", ctypes.c_float), ("x", ctypes.c_void_p), ("ldx", ctypes.c_int64),
        ("y", ctypes.c_void_p), ("ldy", ctypes.c_int64),
    ]


class MoeArgs(ctypes.Structure):
    """Mirror of struct nvfp4_moe_args."""
    _fields_ = [
        ("tokens", ctypes.c_int64), ("experts", ctypes.c_int64), ("top_k", ctypes.c_int64),
        ("hidden", ctypes.c_int64), ("inter", ctypes.c_int64),
        ("x", ctypes.c_void_p), ("router_logits", ctypes.c_void_p),
        ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
        ("stride_gate", ctypes.c_size_t), ("stride_up", ctypes.c_size_t), ("stride_down", ctypes.c_size_t),
        ("scale_gate", ctypes.c_void_p), ("scale_up", ctypes.c_void_p), ("scale_down", ctypes.c_void_p),
        ("y", ctypes.c_void_p), ("y_dtype", ctypes.c_int),
        ("topk_ids", ctypes.c_void_p), ("topk_weights", ctypes.c_void_p),
        ("expert_counts", ctypes.c_void_p), ("expert_offsets", ctypes.c_void_p), ("perm", ctypes.c_void_p),
        ("dbg_gate", ctypes.c_void_p), ("dbg_up", ctypes.c_void_p), ("dbg_h", ctypes.c_void_p),
        ("dbg_down", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
    ]


class ExpertCache(ctypes.Structure):
    """Mirror of struct nvfp4_expert_cache."""
    _fields_ = [
        ("experts", ctypes.c_int64), ("slots", ctypes.c_int64),
        ("host_gate", ctypes.c_void_p), ("host_up", ctypes.c_void_p), ("host_down", ctypes.c_void_p),
        ("dev_gate", ctypes.c_void_p), ("dev_up", ctypes.c_void_p), ("dev_down", ctypes.c_void_p),
        ("stride_gate", ctypes.c_size_t), ("stride_up", ctypes.c_size_t), ("stride_down", ctypes.c_size_t),
        ("dev_slot_of", ctypes.c_void_p), ("host_counts", ctypes.c_void_p), ("host_slot_stage", ctypes.c_void_p),
        ("slot_of", ctypes.c_void_p), ("expert_in", ctypes.c_void_p), ("last_use", ctypes.c_void_p),
        ("clock", ctypes.c_uint64),
        ("last_active", ctypes.c_int64), ("last_fetched", ctypes.c_int64), ("last_bytes", ctypes.c_size_t),
    ]


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m bit_quantized_decode_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, i64, sz, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    sig = {
        "nvfp4_abi_version": (I, []),
        "nvfp4_status_str": (ctypes.c_char_p, [I]),
        "nvfp4_last_error": (ctypes.c_char_p, []),
        "nvfp4_packed_bytes": (I, [i64, i64, ctypes.POINTER(sz)]),
        "nvfp4_pack": (I, [P, P, i64, i64, P, P]),
        "nvfp4_unpack": (I, [P, i64, i64, P, P, P]),
        "nvfp4_gemv_workspace_bytes": (I, [i64, i64, ctypes.POINTER(sz)]),
        "nvfp4_gemv": (I, [P, i64, i64, ctypes.c_float, P, P, P, sz, P]),
        "nvfp4_gemm_workspace_bytes": (I, [i64, i64, i64, ctypes.POINTER(sz)]),
        "nvfp4_gemm": (I, [P, i64, i64, ctypes.c_float, P, i64, i64, P, i64, I, P, sz, P]),
        "nvfp4_gemv_batched_workspace_bytes": (I, [ctypes.POINTER(Problem), I, ctypes.POINTER(sz)]),
        "nvfp4_gemv_batched": (I, [ctypes.POINTER(Problem), I, P, sz, P]),
        "nvfp4_gemv_batched_noalloc": (I, [ctypes.POINTER(Problem), I, P]),
        "nvfp4_gemm_batched_workspace_bytes": (I, [ctypes.POINTER(Problem), I, i64, ctypes.POINTER(sz)]),
        "nvfp4_gemm_batched": (I, [ctypes.POINTER(Problem), I, i64, I, P, sz, P]),
        "nvfp4_moe_workspace_bytes": (I, [ctypes.POINTER(MoeArgs), ctypes.POINTER(sz)]),
        "nvfp4_moe_grouped": (I, [ctypes.POINTER(MoeArgs), P]),
        "nvfp4_quantize_workspace_bytes": (I, [ctypes.POINTER(sz)]),
        "nvfp4_quantize": (I, [P, I, i64, i64, i64, P, P, P, P, sz, P]),
        "nvfp4_expert_cache_reset": (I, [ctypes.POINTER(ExpertCache)]),
        "nvfp4_moe_streamed": (I, [ctypes.POINTER(MoeArgs), ctypes.POINTER(ExpertCache), P]),
        "nvfp4_mx_packed_bytes": (I, [i64, i64, ctypes.POINTER(sz)]),
        "nvfp4_mx_pack": (I, [P, P, i64, i64, P, P]),
        "nvfp4_mx_unpack": (I, [P, i64, i64, P, P, P]),
        "nvfp4_w4a4_workspace_bytes": (I, [i64, i64, ctypes.POINTER(sz)]),
        "nvfp4_w4a4_gemm": (I, [P, i64, i64, ctypes.c_float, P, i64, i64, P, i64, I, P, sz, P]),
        "nvfp4_w4a4_batched_workspace_bytes": (I, [ctypes.POINTER(Problem), I, i64, ctypes.POINTER(sz)]),
        "nvfp4_w4a4_batched": (I, [ctypes.POINTER(Problem), I, i64, I, P, sz, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def check(status):
    if status != NVFP4_OK:
        L = lib()
        raise Nvfp4Error(status, f"{L.nvfp4_status_str(status).decode()}: {L.nvfp4_last_error().decode()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# Zero-initialised workspaces, one per (device, kind), reused across calls in
# stream order.  "split" serves the GEMV / GEMM split-K reductions, whose
# counters every call leaves at zero; "moe" holds the MoE intermediates.  The
# two kinds never share memory, so MoE scratch cannot disturb the counters.
_workspaces = {}


def workspace(nbytes, device, kind="split"):
    if nbytes == 0:
        return None
    key = (str(device), kind)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def abi_version():
    return lib().nvfp4_abi_version()


def packed_bytes(n, k):
    out = ctypes.c_size_t()
    check(lib().nvfp4_packed_bytes(n, k, ctypes.byref(out)))
    return out.value


def pack(codes, scales, stream=None):
    """codes uint8 [n][k/2], scales uint8 [n][k/16] (device) -> packed uint8 buffer."""
    n, kh = codes.shape
    k = 2 * kh
    packed = torch.empty(packed_bytes(n, k), dtype=torch.uint8, device=codes.device)
    check(lib().nvfp4_pack(_ptr(codes), _ptr(scales), n, k, _ptr(packed), _stream(stream)))
    return packed


def mx_packed_bytes(rows, k):
    out = ctypes.c_size_t()
    check(lib().nvfp4_mx_packed_bytes(rows, k, ctypes.byref(out)))
    return out.value


def mx_pack(codes, scales, stream=None):
    """Canonical NVFP4 codes [n][k/2], scales [n][k/16] (device) -> MX tiles for nvfp4_w4a4_gemm."""
    n, kh = codes.shape
    k = 2 * kh
    out = torch.empty(mx_packed_bytes(n, k), dtype=torch.uint8, device=codes.device)
    check(lib().nvfp4_mx_pack(_ptr(codes), _ptr(scales), n, k, _ptr(out), _stream(stream)))
    return out


def mx_unpack(mx, rows, k, stream=None):
    codes = torch.empty((rows, k // 2), dtype=torch.uint8, device=mx.device)
    scales = torch.empty((rows, k // 32), dtype=torch.uint8, device=mx.device)
    check(lib().nvfp4_mx_unpack(_ptr(mx), rows, k, _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def w4a4_workspace_bytes(m, k):
    out = ctypes.c_size_t()
    check(lib().nvfp4_w4a4_workspace_bytes(m, k, ctypes.byref(out)))
    return out.value


def w4a4_x_tiles(ws, m, k):
    """The MX tiles of x that the last nvfp4_w4a4_gemm left in workspace ws."""
    off = w4a4_workspace_bytes(m, k) - mx_packed_bytes(m, k)
    return ws[off:off + mx_packed_bytes(m, k)]


def w4a4_gemm(mx, n, k, tensor_scale, x, y=None, y_dtype=torch.bfloat16, ws=None, stream=None):
    """y[m][n] = s_t * x' W'^T over MX FP4 operands (see nvfp4_w4a4_gemm); ws (zeroed
    before its first use) receives the schedule's counters and x's MX tiles."""
    m = x.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=y_dtype, device=x.device)
    if ws is None:
        ws = workspace(w4a4_workspace_bytes(m, k), x.device, kind="w4a4")
    dt = NVFP4_BF16 if y.dtype == torch.bfloat16 else NVFP4_F32
    check(lib().nvfp4_w4a4_gemm(_ptr(mx), n, k, float(tensor_scale), _ptr(x), m, x.stride(0), _ptr(y), y.stride(0),
                                dt, _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))
    return y


def w4a4_batched_workspace_bytes(items, m):
    """Workspace bytes nvfp4_w4a4_batched needs for these problems at m activation rows."""
    need = ctypes.c_size_t()
    check(lib().nvfp4_w4a4_batched_workspace_bytes(problems(items), len(items), m, ctypes.byref(need)))
    return need.value


def w4a4_batched(items, ws=None, stream=None):
    """Several W4A4 products sharing m and the output dtype:
    items = [(mx_tiles, n, k, tensor_scale, x [m][ldx], y [m][ldy])]."""
    arr = problems(items)
    m = items[0][4].shape[0] if items else 0
    dt = NVFP4_BF16 if items and items[0][5].dtype == torch.bfloat16 else NVFP4_F32
    if ws is None and items:
        ws = workspace(w4a4_batched_workspace_bytes(items, m), items[0][4].device, kind="w4a4")
    check(lib().nvfp4_w4a4_batched(arr, len(items), m, dt, _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))


def w4a4_batched_prepared(items, ws=None, stream=None):
    """nvfp4_w4a4_batched with its arguments marshalled once: returns a
    zero-argument callable that only makes the library call."""
    arr = problems(items)
    m = items[0][4].shape[0] if items else 0
    dt = NVFP4_BF16 if items and items[0][5].dtype == torch.bfloat16 else NVFP4_F32
    if ws is None and items:
        ws = workspace(w4a4_batched_workspace_bytes(items, m), items[0][4].device, kind="w4a4")
    fn, n, wsp, wsb = lib().nvfp4_w4a4_batched, len(items), _ptr(ws), 0 if ws is None else ws.numel()
    keep = (items, ws)

    def call():
        check(fn(arr, n, m, dt, wsp, wsb, _stream(stream)))
        return keep

    return call


def quantize_workspace_bytes():
    out = ctypes.c_size_t()
    check(lib().nvfp4_quantize_workspace_bytes(ctypes.byref(out)))
    return out.value


def quantize(w, codes=None, scales=None, tensor_scale=None, ws=None, stream=None):
    """NVFP4-encode w (device, float32 or bfloat16, [n][k], rows may be strided):
    returns (codes uint8 [n][k/2], scales uint8 [n][k/16], tensor_scale float32 [1])."""
    n, k = w.shape
    dtype = {torch.float32: NVFP4_F32, torch.bfloat16: NVFP4_BF16}[w.dtype]
    dev = w.device
    if codes is None:
        codes = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((n, k // 16), dtype=torch.uint8, device=dev)
    if tensor_scale is None:
        tensor_scale = torch.empty(1, dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(quantize_workspace_bytes(), dev, kind="quantize")
    check(lib().nvfp4_quantize(_ptr(w), dtype, n, k, w.stride(0) if n > 0 else k, _ptr(codes), _ptr(scales),
                               _ptr(tensor_scale), _ptr(ws), ws.numel(), _stream(stream)))
    return codes, scales, tensor_scale


def unpack(packed, n, k, stream=None):
    codes = torch.empty((n, k // 2), dtype=torch.uint8, device=packed.device)
    scales = torch.empty((n, k // 16), dtype=torch.uint8, device=packed.device)
    check(lib().nvfp4_unpack(_ptr(packed), n, k, _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def gemv_workspace_bytes(n, k):
    out = ctypes.c_size_t()
    check(lib().nvfp4_gemv_workspace_bytes(n, k, ctypes.byref(out)))
    return out.value


def gemv(packed, n, k, tensor_scale, x, y=None, ws=None, stream=None):
    """y[n] fp32 = s_t * W x, x bf16 [k] (device)."""
    if y is None:
        y = torch.empty(n, dtype=torch.float32, device=x.device)
    need = gemv_workspace_bytes(n, k)
    if ws is None:
        ws = workspace(need, x.device)
    check(lib().nvfp4_gemv(_ptr(packed), n, k, float(tensor_scale), _ptr(x), _ptr(y), _ptr(ws),
                           0 if ws is None else ws.numel(), _stream(stream)))
    return y


def gemm_workspace_bytes(m, n, k):
    out = ctypes.c_size_t()
    check(lib().nvfp4_gemm_workspace_bytes(m, n, k, ctypes.byref(out)))
    return out.value


def gemm(packed, n, k, tensor_scale, x, y=None, y_dtype=torch.bfloat16, ws=None, stream=None):
    """y[m][n] = s_t * x W^T, x bf16 [m][ldx] (device, row stride x.stride(0))."""
    m = x.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=y_dtype, device=x.device)
    dt = NVFP4_BF16 if y.dtype == torch.bfloat16 else NVFP4_F32
    need = gemm_workspace_bytes(m, n, k)
    if ws is None:
        ws = workspace(need, x.device)
    check(lib().nvfp4_gemm(_ptr(packed), n, k, float(tensor_scale), _ptr(x), m, x.stride(0), _ptr(y), y.stride(0),
                           dt, _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))
    return y


def problems(items):
    """ctypes array of Problem from (packed, n, k, tensor_scale, x, y) tuples of tensors."""
    arr = (Problem * len(items))()
    for i, (packed, n, k, st, x, y) in enumerate(items):
        arr[i].packed = packed.data_ptr()
        arr[i].n, arr[i].k, arr[i].tensor_scale = n, k, float(st)
        arr[i].x = x.data_ptr()
        arr[i].ldx = x.stride(0) if x.dim() == 2 else k
        arr[i].y = y.data_ptr()
        arr[i].ldy = y.stride(0) if y.dim() == 2 else n
    return arr


def gemv_batched(items, ws=None, stream=None):
    """Several GEMVs in one launch: items = [(packed, n, k, tensor_scale, x [k], y fp32 [n]), ...]."""
    arr = problems(items)
    L = lib()
    need = ctypes.c_size_t()
    check(L.nvfp4_gemv_batched_workspace_bytes(arr, len(items), ctypes.byref(need)))
    if ws is None and items:
        ws = workspace(need.value, items[0][4].device)
    check(L.nvfp4_gemv_batched(arr, len(items), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))


def gemv_batched_noalloc(items, stream=None):
    """nvfp4_gemv_batched_noalloc: the batched GEMV with the library's static
    device scratch instead of a workspace (same items as gemv_batched)."""
    arr = problems(items)
    check(lib().nvfp4_gemv_batched_noalloc(arr, len(items), _stream(stream)))


def gemv_batched_prepared(items, ws=None, stream=None):
    """nvfp4_gemv_batched with its arguments marshalled once: returns a
    zero-argument callable that only makes the library call (for tight
    launch loops)."""
    arr = problems(items)
    L = lib()
    need = ctypes.c_size_t()
    check(L.nvfp4_gemv_batched_workspace_bytes(arr, len(items), ctypes.byref(need)))
    if ws is None and items:
        ws = workspace(need.value, items[0][4].device)
    fn, n, wsp, wsb = L.nvfp4_gemv_batched, len(items), _ptr(ws), 0 if ws is None else ws.numel()
    keep = (items, ws)  # the tensors must outlive the callable

    def call():
        # The stream is looked up per call (None: the current one), so that a
        # call under graph capture lands on the capturing stream.
        check(fn(arr, n, wsp, wsb, _stream(stream)))
        return keep

    return call


def gemm_batched_workspace_bytes(items, m):
    """Workspace bytes nvfp4_gemm_batched needs for these problems at m activation rows."""
    arr = problems(items)
    need = ctypes.c_size_t()
    check(lib().nvfp4_gemm_batched_workspace_bytes(arr, len(items), m, ctypes.byref(need)))
    return need.value


def gemm_batched(items, ws=None, stream=None):
    """Several GEMMs sharing m and the output dtype: items = [(packed, n, k, tensor_scale, x [m][ldx], y [m][ldy])]."""
    arr = problems(items)
    L = lib()
    m = items[0][4].shape[0] if items else 0
    dt = NVFP4_BF16 if items and items[0][5].dtype == torch.bfloat16 else NVFP4_F32
    need = ctypes.c_size_t()
    check(L.nvfp4_gemm_batched_workspace_bytes(arr, len(items), m, ctypes.byref(need)))
    if ws is None and items:
        ws = workspace(need.value, items[0][4].device)
    check(L.nvfp4_gemm_batched(arr, len(items), m, dt, _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))


def gemm_batched_prepared(items, ws=None, stream=None):
    """nvfp4_gemm_batched with its arguments marshalled once: returns a
    zero-argument callable that only makes the library call."""
    arr = problems(items)
    L = lib()
    m = items[0][4].shape[0] if items else 0
    dt = NVFP4_BF16 if items and items[0][5].dtype == torch.bfloat16 else NVFP4_F32
    need = ctypes.c_size_t()
    check(L.nvfp4_gemm_batched_workspace_bytes(arr, len(items), m, ctypes.byref(need)))
    if ws is None and items:
        ws = workspace(need.value, items[0][4].device)
    fn, n, wsp, wsb = L.nvfp4_gemm_batched, len(items), _ptr(ws), 0 if ws is None else ws.numel()
    keep = (items, ws)

    def call():
        check(fn(arr, n, m, dt, wsp, wsb, _stream(stream)))
        return keep

    return call


def moe_args(**kw):
    a = MoeArgs()
    for key, val in kw.items():
        if isinstance(val, torch.Tensor):
            val = val.data_ptr()
        setattr(a, key, val)
    return a


def moe_workspace_bytes(tokens, experts, top_k, hidden, inter):
    a = moe_args(tokens=tokens, experts=experts, top_k=top_k, hidden=hidden, inter=inter)
    out = ctypes.c_size_t()
    check(lib().nvfp4_moe_workspace_bytes(ctypes.byref(a), ctypes.byref(out)))
    return out.value


def moe_grouped(x, logits, top_k, w_gate, w_up, w_down, stride_gate, stride_up, stride_down,
                scale_gate, scale_up, scale_down, inter, y_dtype=torch.float32, debug=False, ws=None,
                outputs=None, stream=None):
    """The routed expert layer.  Returns a dict of the outputs (see nvfp4_moe_grouped).
    w_gate may be an ExpertStream (then w_up, w_down and the strides are taken from it)."""
    streamed = w_gate if isinstance(w_gate, ExpertStream) else None
    if streamed is not None:
        w_gate, w_up, w_down = streamed.dev
        stride_gate, stride_up, stride_down = streamed.strides
    tokens, hidden = x.shape
    experts = logits.shape[1]
    dev = x.device
    o = outputs if outputs is not None else {}
    flat = tokens * top_k
    o.setdefault("y", torch.empty((tokens, hidden), dtype=y_dtype, device=dev))
    o.setdefault("topk_ids", torch.empty((tokens, top_k), dtype=torch.int32, device=dev))
    o.setdefault("topk_weights", torch.empty((tokens, top_k), dtype=torch.float32, device=dev))
    o.setdefault("expert_counts", torch.empty(experts, dtype=torch.int32, device=dev))
    o.setdefault("expert_offsets", torch.empty(experts + 1, dtype=torch.int32, device=dev))
    o.setdefault("perm", torch.empty(flat, dtype=torch.int32, device=dev))
    if debug:
        o.setdefault("dbg_gate", torch.empty((flat, inter), dtype=torch.float32, device=dev))
        o.setdefault("dbg_up", torch.empty((flat, inter), dtype=torch.float32, device=dev))
        o.setdefault("dbg_h", torch.empty((flat, inter), dtype=torch.bfloat16, device=dev))
        o.setdefault("dbg_down", torch.empty((flat, hidden), dtype=torch.float32, device=dev))
    if ws is None:
        ws = workspace(moe_workspace_bytes(tokens, experts, top_k, hidden, inter), dev, kind="moe")
    a = moe_args(
        tokens=tokens, experts=experts, top_k=top_k, hidden=hidden, inter=inter, x=x, router_logits=logits,
        w_gate=w_gate, w_up=w_up, w_down=w_down, stride_gate=stride_gate, stride_up=stride_up,
        stride_down=stride_down, scale_gate=scale_gate, scale_up=scale_up, scale_down=scale_down,
        y=o["y"], y_dtype=NVFP4_BF16 if o["y"].dtype == torch.bfloat16 else NVFP4_F32,
        topk_ids=o["topk_ids"], topk_weights=o["topk_weights"], expert_counts=o["expert_counts"],
        expert_offsets=o["expert_offsets"], perm=o["perm"],
        dbg_gate=o.get("dbg_gate"), dbg_up=o.get("dbg_up"), dbg_h=o.get("dbg_h"), dbg_down=o.get("dbg_down"),
        workspace=ws, workspace_bytes=0 if ws is None else ws.numel(),
    )
    if streamed is not None:
        check(lib().nvfp4_moe_streamed(ctypes.byref(a), ctypes.byref(streamed.cache), _stream(stream)))
    else:
        check(lib().nvfp4_moe_grouped(ctypes.byref(a), _stream(stream)))
    return o


class ExpertStream:
    """Routed experts streamed from pinned host memory through a device cache
    of `slots` expert slots (nvfp4_moe_streamed).  pool_*: the packed expert
    pools (uint8 tensors, expert e at e * stride_*, any device); they are
    copied once into pinned host memory.  Pass the object as w_gate to
    moe_grouped (w_up / w_down / strides: None); its device slot pools then
    stand in for the weights."""

    def __init__(self, pool_gate, pool_up, pool_down, stride_gate, stride_up, stride_down, experts, slots, device):
        import numpy as np
        self.host = [torch.empty(p.numel(), dtype=torch.uint8, pin_memory=True) for p in (pool_gate, pool_up, pool_down)]
        for h, p in zip(self.host, (pool_gate, pool_up, pool_down)):
            h.copy_(p.reshape(-1))
        strides = (stride_gate, stride_up, stride_down)
        self.dev = [torch.empty(slots * st, dtype=torch.uint8, device=device) for st in strides]
        self.dev_slot_of = torch.zeros(experts, dtype=torch.int32, device=device)
        self.host_counts = torch.zeros(experts, dtype=torch.int32, pin_memory=True)
        self.host_stage = torch.zeros(experts, dtype=torch.int32, pin_memory=True)
        self.slot_of = np.full(experts, -1, np.int32)
        self.expert_in = np.full(slots, -1, np.int32)
        self.last_use = np.zeros(slots, np.uint64)
        c = ExpertCache()
        c.experts, c.slots = experts, slots
        c.host_gate, c.host_up, c.host_down = (h.data_ptr() for h in self.host)
        c.dev_gate, c.dev_up, c.dev_down = (d.data_ptr() for d in self.dev)
        c.stride_gate, c.stride_up, c.stride_down = strides
        c.dev_slot_of = self.dev_slot_of.data_ptr()
        c.host_counts = self.host_counts.data_ptr()
        c.host_slot_stage = self.host_stage.data_ptr()
        c.slot_of = self.slot_of.ctypes.data
        c.expert_in = self.expert_in.ctypes.data
        c.last_use = self.last_use.ctypes.data
        self.cache = c
        self.strides = strides
        self.reset()

    def reset(self):
        check(lib().nvfp4_expert_cache_reset(ctypes.byref(self.cache)))

    def stats(self):
        c = self.cache
        return {"active": c.last_active, "fetched": c.last_fetched, "bytes": c.last_bytes}


def moe_grouped_prepared(*args, **kw):
    """moe_grouped with its arguments marshalled once (same arguments):
    returns (call, outputs), call() making only the library call."""
    o = moe_grouped(*args, **kw)   # one real call builds and validates everything
    x, logits, top_k = args[0], args[1], args[2]
    tokens, hidden = x.shape
    experts = logits.shape[1]
    inter = args[12]
    ws = kw.get("ws")
    if ws is None:
        ws = workspace(moe_workspace_bytes(tokens, experts, top_k, hidden, inter), x.device, kind="moe")
    a = moe_args(
        tokens=tokens, experts=experts, top_k=top_k, hidden=hidden, inter=inter, x=x, router_logits=logits,
        w_gate=args[3], w_up=args[4], w_down=args[5], stride_gate=args[6], stride_up=args[7],
        stride_down=args[8], scale_gate=args[9], scale_up=args[10], scale_down=args[11],
        y=o["y"], y_dtype=NVFP4_BF16 if o["y"].dtype == torch.bfloat16 else NVFP4_F32,
        topk_ids=o["topk_ids"], topk_weights=o["topk_weights"], expert_counts=o["expert_counts"],
        expert_offsets=o["expert_offsets"], perm=o["perm"],
        dbg_gate=o.get("dbg_gate"), dbg_up=o.get("dbg_up"), dbg_h=o.get("dbg_h"), dbg_down=o.get("dbg_down"),
        workspace=ws, workspace_bytes=ws.numel(),
    )
    fn, ref, stream = lib().nvfp4_moe_grouped, ctypes.byref(a), kw.get("stream")
    keep = (args, kw, o, ws, a)

    def call():
        check(fn(ref, _stream(stream)))
        return keep

    return call, o
