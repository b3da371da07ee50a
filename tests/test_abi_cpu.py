"""The C ABI without a GPU: the library loads, exports every declared symbol,
and refuses invalid arguments with the documented status before touching HIP."""
import ctypes
import os
import re

import pytest

from bit_quantized_decode_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        from bit_quantized_decode_amd import build
        build.build()
    return B.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) == 28, names
    assert set(names) == set(B.EXPORTED)
    for name in names:
        assert hasattr(L, name), name


def test_version_and_status_strings(L):
    assert L.nvfp4_abi_version() == 1
    assert L.nvfp4_status_str(0) == b"NVFP4_OK"
    assert L.nvfp4_status_str(5) == b"NVFP4_ERR_WORKSPACE"
    assert L.nvfp4_status_str(99) == b"unknown status"


@pytest.mark.parametrize("n,k,expect", [
    (1024, 1024, 589_824),             # 1024 x 1024 weights at 0.5625 B each
    (17408, 5120, 50_135_040),         # gate / up of the 27B-class layer
    (5120, 17408, 50_135_040),         # down
    (7168, 5120, 20_643_840),          # QKV
    (512, 2048, 589_824),              # one MoE expert matrix
    (1, 16, 9216),                     # one padded tile
    (65, 272, 4 * 9216),               # 2 row tiles x 2 k tiles
    (0, 0, 0),
])
def test_packed_bytes(n, k, expect):
    assert B.packed_bytes(n, k) == expect


def status_of(fn, *args):
    return fn(*args)


def test_shape_and_pointer_validation(L):
    sz = ctypes.c_size_t()
    assert L.nvfp4_packed_bytes(4, 24, ctypes.byref(sz)) == B.NVFP4_ERR_SHAPE
    assert L.nvfp4_packed_bytes(-1, 16, ctypes.byref(sz)) == B.NVFP4_ERR_SHAPE
    assert L.nvfp4_packed_bytes(4, 16, None) == B.NVFP4_ERR_NULL
    assert b"multiple of 16" in L.nvfp4_last_error() or True
    A = ctypes.c_void_p(0x10000)   # 16-byte aligned fake device address (never dereferenced)
    M = ctypes.c_void_p(0x10008)   # misaligned
    # pack
    assert L.nvfp4_pack(None, A, 4, 16, A, None) == B.NVFP4_ERR_NULL
    assert L.nvfp4_pack(M, A, 4, 16, A, None) == B.NVFP4_ERR_ALIGN
    assert L.nvfp4_pack(A, A, 4, 20, A, None) == B.NVFP4_ERR_SHAPE
    assert L.nvfp4_pack(None, None, 0, 16, None, None) == B.NVFP4_OK      # empty: no work
    assert L.nvfp4_unpack(A, 4, 16, None, A, None) == B.NVFP4_ERR_NULL
    # gemv
    assert L.nvfp4_gemv(A, 4, 16, 1.0, None, A, None, 0, None) == B.NVFP4_ERR_NULL
    assert L.nvfp4_gemv(A, 4, 16, 1.0, M, A, None, 0, None) == B.NVFP4_ERR_ALIGN
    assert L.nvfp4_gemv(A, 4, 17, 1.0, A, A, None, 0, None) == B.NVFP4_ERR_SHAPE
    assert L.nvfp4_gemv(None, 0, 16, 1.0, None, None, None, 0, None) == B.NVFP4_OK
    need = B.gemv_workspace_bytes(5120, 17408)
    assert need > 0
    assert L.nvfp4_gemv(A, 5120, 17408, 1.0, A, A, None, 0, None) == B.NVFP4_ERR_WORKSPACE
    assert L.nvfp4_gemv(A, 5120, 17408, 1.0, A, A, A, need - 1, None) == B.NVFP4_ERR_WORKSPACE
    # gemm
    assert L.nvfp4_gemm(A, 64, 64, 1.0, A, 32, 64, A, 64, 7, None, 0, None) == B.NVFP4_ERR_DTYPE
    assert L.nvfp4_gemm(A, 64, 64, 1.0, A, 32, 60, A, 64, 1, None, 0, None) == B.NVFP4_ERR_SHAPE   # ldx < k
    assert L.nvfp4_gemm(A, 64, 64, 1.0, A, 32, 64, A, 60, 1, None, 0, None) == B.NVFP4_ERR_SHAPE   # ldy < n
    assert L.nvfp4_gemm(A, 64, 64, 1.0, A, -1, 64, A, 64, 1, None, 0, None) == B.NVFP4_ERR_SHAPE
    assert L.nvfp4_gemm(A, 64, 64, 1.0, A, 0, 64, A, 64, 1, None, 0, None) == B.NVFP4_OK          # m = 0
    assert L.nvfp4_gemm(A, 64, 64, 1.0, None, 32, 64, A, 64, 1, None, 0, None) == B.NVFP4_ERR_NULL
    assert L.nvfp4_gemm(A, 64, 64, 1.0, A, 32, 64, M, 64, 1, None, 0, None) == B.NVFP4_ERR_ALIGN
    need = B.gemm_workspace_bytes(32, 5120, 17408)
    assert need > 0
    assert L.nvfp4_gemm(A, 5120, 17408, 1.0, A, 32, 17408, A, 5120, 1, A, need - 16, None) == B.NVFP4_ERR_WORKSPACE
    # One row past the largest n a product call takes (65536 row tiles of 64).
    big = 4194304 + 1
    assert L.nvfp4_gemv(A, big, 1280, 1.0, A, A, A, 1 << 40, None) == B.NVFP4_ERR_SHAPE
    assert L.nvfp4_gemm(A, big, 1280, 1.0, A, 32, 1280, A, big, 1, A, 1 << 40, None) == B.NVFP4_ERR_SHAPE
    assert L.nvfp4_gemm(A, big, 256, 1.0, A, 64, 256, A, big, 1, A, 1 << 40, None) == B.NVFP4_ERR_SHAPE
    # k up to 32768, where the accumulation bound is proven; one block past it is refused.
    sz = ctypes.c_size_t()
    assert L.nvfp4_gemv_workspace_bytes(64, 32768, ctypes.byref(sz)) == B.NVFP4_OK
    assert L.nvfp4_gemv_workspace_bytes(64, 32784, ctypes.byref(sz)) == B.NVFP4_ERR_SHAPE
    assert L.nvfp4_gemv(A, 64, 32784, 1.0, A, A, A, 1 << 40, None) == B.NVFP4_ERR_SHAPE
    for m in (2, 32, 64):
        assert L.nvfp4_gemm_workspace_bytes(m, 64, 32768, ctypes.byref(sz)) == B.NVFP4_OK
        assert L.nvfp4_gemm(A, 64, 32784, 1.0, A, m, 32784, A, 64, 1, A, 1 << 40, None) == B.NVFP4_ERR_SHAPE
    assert L.nvfp4_w4a4_gemm(A, 64, 32800, 1.0, A, 64, 32800, A, 64, 1, A, 1 << 40, None) == B.NVFP4_ERR_SHAPE
    arr = (B.Problem * 1)()
    arr[0].packed, arr[0].n, arr[0].k, arr[0].x, arr[0].y, arr[0].ldx, arr[0].ldy = A, 64, 32784, A, A, 32784, 64
    assert L.nvfp4_gemv_batched(arr, 1, A, 1 << 40, None) == B.NVFP4_ERR_SHAPE
    assert L.nvfp4_gemm_batched(arr, 1, 32, 1, A, 1 << 40, None) == B.NVFP4_ERR_SHAPE
    # packing and quantising are not products: no such limit
    assert L.nvfp4_packed_bytes(64, 65536, ctypes.byref(sz)) == B.NVFP4_OK


def test_quantize_validation(L):
    A, M = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x10008)
    T = ctypes.c_void_p(0x10004)                 # 4-byte aligned (the tensor scale's requirement)
    need = B.quantize_workspace_bytes()
    assert need >= 4
    q = L.nvfp4_quantize
    assert q(A, B.NVFP4_BF16, 0, 64, 64, None, None, None, None, 0, None) == B.NVFP4_OK        # n = 0: no-op
    assert q(A, B.NVFP4_BF16, 4, 0, 0, None, None, None, None, 0, None) == B.NVFP4_OK          # k = 0: no-op
    assert q(A, 7, 4, 64, 64, A, A, T, A, need, None) == B.NVFP4_ERR_DTYPE
    assert q(A, B.NVFP4_F32, 4, 40, 40, A, A, T, A, need, None) == B.NVFP4_ERR_SHAPE           # k % 16
    assert q(A, B.NVFP4_F32, 4, 64, 60, A, A, T, A, need, None) == B.NVFP4_ERR_SHAPE           # ldw < k
    assert q(A, B.NVFP4_F32, 4, 64, 68, A, A, T, A, need, None) == B.NVFP4_ERR_SHAPE           # ldw % 8
    assert q(None, B.NVFP4_F32, 4, 64, 64, A, A, T, A, need, None) == B.NVFP4_ERR_NULL
    assert q(A, B.NVFP4_F32, 4, 64, 64, A, A, None, A, need, None) == B.NVFP4_ERR_NULL
    assert q(M, B.NVFP4_F32, 4, 64, 64, A, A, T, A, need, None) == B.NVFP4_ERR_ALIGN
    assert q(A, B.NVFP4_F32, 4, 64, 64, A, A, ctypes.c_void_p(0x10002), A, need, None) == B.NVFP4_ERR_ALIGN
    assert q(A, B.NVFP4_F32, 4, 64, 64, A, A, T, None, 0, None) == B.NVFP4_ERR_WORKSPACE
    assert q(A, B.NVFP4_F32, 4, 64, 64, A, A, T, A, need - 1, None) == B.NVFP4_ERR_WORKSPACE


def moe_template(**over):
    A = 0x10000
    kw = dict(tokens=32, experts=512, top_k=10, hidden=2048, inter=512, x=A, router_logits=A, w_gate=A, w_up=A,
              w_down=A, stride_gate=589_824, stride_up=589_824, stride_down=589_824, scale_gate=A, scale_up=A,
              scale_down=A, y=A, y_dtype=B.NVFP4_F32, topk_ids=A, topk_weights=A, expert_counts=A,
              expert_offsets=A, perm=A, workspace=A, workspace_bytes=1 << 30)
    kw.update(over)
    return B.moe_args(**kw)


@pytest.mark.parametrize("over,status", [
    (dict(top_k=0), B.NVFP4_ERR_ARG),
    (dict(top_k=513), B.NVFP4_ERR_ARG),
    (dict(top_k=65, experts=100), B.NVFP4_ERR_ARG),
    (dict(experts=4096), B.NVFP4_ERR_ARG),
    (dict(experts=2049), B.NVFP4_ERR_ARG),       # one past the largest expert count
    (dict(top_k=65, experts=2048), B.NVFP4_ERR_ARG),
    (dict(hidden=2040), B.NVFP4_ERR_SHAPE),
    (dict(inter=-16), B.NVFP4_ERR_SHAPE),
    (dict(hidden=32784), B.NVFP4_ERR_SHAPE),     # past the products' k limit (gate / up)
    (dict(inter=32784), B.NVFP4_ERR_SHAPE),      # (down)
    (dict(tokens=-1), B.NVFP4_ERR_SHAPE),
    (dict(stride_down=589_808), B.NVFP4_ERR_ARG),
    (dict(stride_gate=589_832), B.NVFP4_ERR_ALIGN),
    (dict(x=0), B.NVFP4_ERR_NULL),
    (dict(perm=0), B.NVFP4_ERR_NULL),
    (dict(x=0x10004), B.NVFP4_ERR_ALIGN),
    (dict(topk_ids=0x10002), B.NVFP4_ERR_ALIGN),
    (dict(y_dtype=3), B.NVFP4_ERR_DTYPE),
    (dict(workspace_bytes=1024), B.NVFP4_ERR_WORKSPACE),
])
def test_moe_validation(L, over, status):
    a = moe_template(**over)
    assert L.nvfp4_moe_grouped(ctypes.byref(a), None) == status
    assert L.nvfp4_last_error() != b""


def test_moe_zero_tokens_is_a_noop(L):
    a = moe_template(tokens=0, x=0, y=0, workspace=0, workspace_bytes=0)
    assert L.nvfp4_moe_grouped(ctypes.byref(a), None) == B.NVFP4_OK
    assert L.nvfp4_moe_grouped(None, None) == B.NVFP4_ERR_NULL


def test_moe_workspace_size_covers_intermediates():
    need = B.moe_workspace_bytes(32, 512, 10, 2048, 512)
    # h (bf16 320 x 512) + d (fp32 320 x 2048) + indices
    assert need >= 320 * 512 * 2 + 320 * 2048 * 4


def test_batched_validation(L):
    A, M = 0x10000, 0x10008
    arr = (B.Problem * 3)()
    for i in range(3):
        arr[i].packed, arr[i].n, arr[i].k, arr[i].tensor_scale = A, 64, 256, 1.0
        arr[i].x, arr[i].ldx, arr[i].y, arr[i].ldy = A, 256, A + 0x1000 * (i + 1), 64
    sz = ctypes.c_size_t()
    assert L.nvfp4_gemv_batched_workspace_bytes(arr, 3, ctypes.byref(sz)) == B.NVFP4_OK
    assert L.nvfp4_gemv_batched(None, 2, None, 0, None) == B.NVFP4_ERR_NULL
    assert L.nvfp4_gemv_batched(arr, -1, None, 0, None) == B.NVFP4_ERR_ARG
    assert L.nvfp4_gemv_batched(arr, 0, None, 0, None) == B.NVFP4_OK
    arr[1].k = 40
    assert L.nvfp4_gemv_batched(arr, 3, None, 0, None) == B.NVFP4_ERR_SHAPE
    arr[1].k = 256
    arr[2].x = M
    assert L.nvfp4_gemv_batched(arr, 3, None, 0, None) == B.NVFP4_ERR_ALIGN
    arr[2].x = A
    arr[2].y = arr[0].y
    assert L.nvfp4_gemv_batched(arr, 3, None, 0, None) == B.NVFP4_ERR_ARG      # shared output
    arr[2].y = A + 0x9000
    assert L.nvfp4_gemm_batched(arr, 3, 32, 9, None, 0, None) == B.NVFP4_ERR_DTYPE
    arr[0].ldx = 100
    assert L.nvfp4_gemm_batched(arr, 3, 32, 1, None, 0, None) == B.NVFP4_ERR_SHAPE
    arr[0].ldx = 256
    assert L.nvfp4_gemm_batched(arr, 3, 0, 1, None, 0, None) == B.NVFP4_OK     # m = 0
    big = (B.Problem * 1)()
    big[0].packed, big[0].n, big[0].k, big[0].x, big[0].y = A, 5120, 17408, A, A
    big[0].ldx, big[0].ldy = 17408, 5120
    assert L.nvfp4_gemm_batched_workspace_bytes(big, 1, 32, ctypes.byref(sz)) == B.NVFP4_OK and sz.value > 0
    assert L.nvfp4_gemm_batched(big, 1, 32, 1, None, 0, None) == B.NVFP4_ERR_WORKSPACE


def test_gemv_noalloc_validation(L):
    """The static-scratch GEMV batch refuses, before any HIP call, batches its
    scratch cannot hold, more than 64 problems, and what nvfp4_gemv_batched refuses."""
    A = 0x10000
    arr = (B.Problem * 65)()
    for i in range(65):
        arr[i].packed, arr[i].n, arr[i].k, arr[i].tensor_scale = A, 64, 2048, 1.0
        arr[i].x, arr[i].y = A, A + 0x1000 * (i + 1)
    assert L.nvfp4_gemv_batched_noalloc(arr, 65, None) == B.NVFP4_ERR_ARG
    assert L.nvfp4_gemv_batched_noalloc(arr, 0, None) == B.NVFP4_OK
    arr[0].n = 1 << 20                                  # 2 k-groups x 2^20 rows x 4 B = 8 MiB of partials
    arr[1].n = 64
    assert L.nvfp4_gemv_batched_noalloc(arr, 2, None) == B.NVFP4_ERR_WORKSPACE
    assert b"static scratch" in L.nvfp4_last_error()
    arr[0].n = 64
    arr[1].k = 40
    assert L.nvfp4_gemv_batched_noalloc(arr, 2, None) == B.NVFP4_ERR_SHAPE
    arr[1].k = 2048
    arr[1].y = arr[0].y
    assert L.nvfp4_gemv_batched_noalloc(arr, 2, None) == B.NVFP4_ERR_ARG     # shared output
    arr[1].y = A + 0x9000
    arr[1].x = A + 8
    assert L.nvfp4_gemv_batched_noalloc(arr, 2, None) == B.NVFP4_ERR_ALIGN


def test_w4a4_validation(L):
    A = 0x10000
    sz, one = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.nvfp4_w4a4_workspace_bytes(512, 5120, ctypes.byref(one)) == B.NVFP4_OK
    assert L.nvfp4_mx_packed_bytes(512, 5120, ctypes.byref(sz)) == B.NVFP4_OK
    stream_k = one.value - sz.value                   # counters and partial sums ahead of x's MX tiles
    assert stream_k > 0
    assert L.nvfp4_w4a4_workspace_bytes(64, 96, ctypes.byref(one)) == B.NVFP4_OK
    assert L.nvfp4_mx_packed_bytes(64, 96, ctypes.byref(sz)) == B.NVFP4_OK
    assert one.value - sz.value == stream_k           # the same offset for every shape
    assert L.nvfp4_w4a4_workspace_bytes(64, 48, ctypes.byref(one)) == B.NVFP4_ERR_SHAPE   # k % 32
    arr = (B.Problem * 2)()
    for i in range(2):
        arr[i].packed, arr[i].n, arr[i].k, arr[i].tensor_scale = A, 64, 256, 1.0
        arr[i].x, arr[i].ldx, arr[i].y, arr[i].ldy = A, 256, A + 0x1000 * (i + 1), 64
    assert L.nvfp4_w4a4_batched_workspace_bytes(arr, 2, 300, ctypes.byref(sz)) == B.NVFP4_OK
    assert L.nvfp4_mx_packed_bytes(300, 256, ctypes.byref(one)) == B.NVFP4_OK
    assert sz.value == stream_k + 2 * one.value       # each problem's x tiles after the stream-K area
    arr[1].k = 48
    assert L.nvfp4_w4a4_batched_workspace_bytes(arr, 2, 300, ctypes.byref(sz)) == B.NVFP4_ERR_SHAPE
    arr[1].k = 256
    assert L.nvfp4_w4a4_batched(arr, 2, -1, 1, None, 0, None) == B.NVFP4_ERR_SHAPE
    assert L.nvfp4_w4a4_batched(arr, 2, 1 << 25, 1, None, 0, None) == B.NVFP4_ERR_SHAPE
    assert L.nvfp4_w4a4_batched(arr, 2, 300, 9, None, 0, None) == B.NVFP4_ERR_DTYPE
    assert L.nvfp4_w4a4_batched(arr, 2, 300, 1, None, 0, None) == B.NVFP4_ERR_WORKSPACE
    assert L.nvfp4_w4a4_batched(arr, 2, 0, 1, None, 0, None) == B.NVFP4_OK      # m = 0
    arr[1].y = arr[0].y
    assert L.nvfp4_w4a4_batched(arr, 2, 300, 1, None, 0, None) == B.NVFP4_ERR_ARG   # shared output
    # single product: shape, dtype, stride, pointer, alignment and workspace checks before any launch
    W, X, Y = A, A + 0x1000, A + 0x2000
    g = L.nvfp4_w4a4_gemm
    assert g(W, 64, 48, 1.0, X, 4, 48, Y, 64, 1, None, 0, None) == B.NVFP4_ERR_SHAPE      # k % 32
    assert g(W, 64, 64, 1.0, X, 4, 64, Y, 64, 7, None, 0, None) == B.NVFP4_ERR_DTYPE
    assert g(W, 64, 64, 1.0, X, 4, 60, Y, 64, 1, None, 0, None) == B.NVFP4_ERR_SHAPE      # ldx < k
    assert g(W, 64, 64, 1.0, X, 4, 64, Y, 32, 1, None, 0, None) == B.NVFP4_ERR_SHAPE      # ldy < n
    assert g(None, 64, 64, 1.0, X, 4, 64, Y, 64, 1, None, 0, None) == B.NVFP4_ERR_NULL
    assert g(W + 8, 64, 64, 1.0, X, 4, 64, Y, 64, 1, None, 0, None) == B.NVFP4_ERR_ALIGN
    assert g(W, 64, 64, 1.0, X, 4, 64, Y, 64, 1, None, 0, None) == B.NVFP4_ERR_WORKSPACE
    assert g(W, 64, 64, 1.0, X, 0, 64, Y, 64, 1, None, 0, None) == B.NVFP4_OK              # m = 0
    assert g(W, 0, 64, 1.0, X, 4, 64, Y, 64, 1, None, 0, None) == B.NVFP4_OK               # n = 0
    assert g(W, 64, 64, 1.0, X, -1, 64, Y, 64, 1, None, 0, None) == B.NVFP4_ERR_SHAPE


def test_expert_cache_validation(L):
    import numpy as np
    c = B.ExpertCache()
    assert L.nvfp4_expert_cache_reset(None) == B.NVFP4_ERR_NULL
    c.experts, c.slots = 8, 0
    assert L.nvfp4_expert_cache_reset(ctypes.byref(c)) == B.NVFP4_ERR_ARG
    c.slots = 4
    assert L.nvfp4_expert_cache_reset(ctypes.byref(c)) == B.NVFP4_ERR_NULL      # no state arrays
    slot_of = np.zeros(8, np.int32)
    expert_in = np.zeros(4, np.int32)
    last_use = np.ones(4, np.uint64)
    c.slot_of, c.expert_in, c.last_use = slot_of.ctypes.data, expert_in.ctypes.data, last_use.ctypes.data
    c.clock = 99
    assert L.nvfp4_expert_cache_reset(ctypes.byref(c)) == B.NVFP4_OK
    assert (slot_of == -1).all() and (expert_in == -1).all() and (last_use == 0).all() and c.clock == 0
    # nvfp4_moe_streamed refuses before any launch: no cache, or pools that are not the cache's.
    a = moe_template()
    assert L.nvfp4_moe_streamed(ctypes.byref(a), None, None) == B.NVFP4_ERR_NULL
    c.experts = 512
    c.dev_gate = c.dev_up = c.dev_down = 0x20000
    c.stride_gate = c.stride_up = c.stride_down = 589_824
    assert L.nvfp4_moe_streamed(ctypes.byref(a), ctypes.byref(c), None) == B.NVFP4_ERR_ARG


def test_failed_streamed_call_leaves_the_cache_unchanged(L):
    """A streamed call whose first launch fails (here: no GPU) returns
    NVFP4_ERR_HIP and leaves the cache exactly as it was: the cache's new
    state is committed only after every copy of the call is enqueued.  Runs
    only where no GPU is visible (it would otherwise launch on fake pointers)."""
    import numpy as np
    import torch
    if torch.cuda.device_count() != 0:
        pytest.skip("a GPU is visible: this call would launch kernels on placeholder pointers")
    c = B.ExpertCache()
    c.experts, c.slots = 512, 4
    slot_of = np.full(512, -1, np.int32)
    expert_in = np.array([7, -1, 300, 2], np.int32)
    last_use = np.array([5, 0, 9, 3], np.uint64)
    slot_of[[7, 300, 2]] = [0, 2, 3]
    c.slot_of, c.expert_in, c.last_use = slot_of.ctypes.data, expert_in.ctypes.data, last_use.ctypes.data
    c.clock = 9
    c.dev_gate = c.dev_up = c.dev_down = 0x20000
    c.stride_gate = c.stride_up = c.stride_down = 589_824
    c.host_gate = c.host_up = c.host_down = 0x40000
    c.dev_slot_of, c.host_counts, c.host_slot_stage = 0x50000, 0x60000, 0x70000
    a = moe_template(w_gate=0x20000, w_up=0x20000, w_down=0x20000, stride_gate=589_824, stride_up=589_824,
                     stride_down=589_824)
    before = (slot_of.copy(), expert_in.copy(), last_use.copy())
    assert L.nvfp4_moe_streamed(ctypes.byref(a), ctypes.byref(c), None) == B.NVFP4_ERR_HIP
    assert np.array_equal(slot_of, before[0]) and np.array_equal(expert_in, before[1])
    assert np.array_equal(last_use, before[2]) and c.clock == 9
