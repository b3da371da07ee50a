// The skinny-product core shared by the decode-batch GEMM (a3) and the
// mixture-of-experts expert GEMMs (a6, a7): a workgroup of four wavefronts
// multiplies four 64-row NVFP4 tiles (one per wavefront, possibly of different
// matrices), over a common range of 256-k tiles, by the same <= 32 bf16
// activation rows, on the bf16 matrix cores.
//
// Data flow per 256-k tile:
//  - the activation tile (32 rows x 256 k, 16 KB) is loaded once per
//    workgroup into LDS (double-buffered, one barrier per tile), so every
//    wavefront reads it from LDS instead of from memory;
//  - each wavefront keeps the next weight tile's nine 16-byte loads in flight
//    while it multiplies the current one;
//  - one 1 KB wavefront load of a tile chunk (64 rows x 32 k) is already the
//    A operands of four v_mfma_f32_32x32x16_bf16 (rows 0-31 and 32-63, two k
//    steps of 16): lane l holds 8 consecutive k of rows l%32 and 32 + l%32
//    at k offset 8*(l/32), that instruction's operand layout;
//  - every weight is dequantised exactly: E2M1 -> fp32, times its E4M3 block
//    scale in fp32 (at most 6 significant bits, so exact), and the upper
//    half of that fp32 is its bf16.  The activations are the B operand: lane
//    l supplies activation row l%32's 8 values at the same k offset.
// Accumulation is two-level: each 256-k tile accumulates in a fresh fp32
// accumulator (16 MFMA steps), then is added to the running sum.
#pragma once

#include "device_common.h"

namespace nvfp4 {

constexpr int kXStride = kTileK + 8;  // bf16 per LDS activation row (16-byte pad: conflict-free reads)
constexpr int kXTileElems = 32 * kXStride;

// Eight weights of one k step: code word `w` (8 nibbles, k ascending) times
// scale `s`, as bf16.  Each product has at most 6 significant bits, so the
// fp32 product is exact and so is taking its upper half as the bf16.
__device__ __forceinline__ bf16x8 dequant8(uint32_t w, float s) {
  u32x4 r;
  f32x2 v;
  v = e2m1x2<0>(w); r[0] = pack_exact_bf16x2(v.x * s, v.y * s);
  v = e2m1x2<1>(w); r[1] = pack_exact_bf16x2(v.x * s, v.y * s);
  v = e2m1x2<2>(w); r[2] = pack_exact_bf16x2(v.x * s, v.y * s);
  v = e2m1x2<3>(w); r[3] = pack_exact_bf16x2(v.x * s, v.y * s);
  return __builtin_bit_cast(bf16x8, r);
}

struct WTile {
  u32x4 sa, sb;   // scale bytes of rows lane%32 and 32 + lane%32
  u32x4 q[8];
};

__device__ __forceinline__ void load_wtile(const uint8_t* tile, int lane, WTile& r) {
  r.sa = load16(tile + kScaleOffset + 32 * (lane & 31));
  r.sb = load16(tile + kScaleOffset + 32 * (lane & 31) + 16);
#pragma unroll
  for (int c = 0; c < 8; ++c) r.q[c] = load16(tile + c * 1024 + lane * 16);
}

// One 32-k chunk C of a tile: four MFMAs into the two tile accumulators.  The
// tile layout already holds the A operands: dword 0 = rows 0-31 step 2C,
// dword 1 = rows 32-63 step 2C, dwords 2 / 3 = the same for step 2C+1.
template <int C>
__device__ __forceinline__ void chunk_mfma(u32x4 q, u32x4 sa, u32x4 sb, bf16x8 xa, bf16x8 xb, f32x16& ta,
                                           f32x16& tb) {
  ta = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dequant8(q[0], e4m3<(2 * C) % 4>(sa[C / 2])), xa, ta, 0, 0, 0);
  tb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dequant8(q[1], e4m3<(2 * C) % 4>(sb[C / 2])), xa, tb, 0, 0, 0);
  ta = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dequant8(q[2], e4m3<(2 * C + 1) % 4>(sa[C / 2])), xb, ta, 0, 0, 0);
  tb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dequant8(q[3], e4m3<(2 * C + 1) % 4>(sb[C / 2])), xb, tb, 0, 0, 0);
}

// Multiply the resident weight tile `w` by the activation tile in LDS (`xt`,
// 32 rows of kXStride bf16) into acc_a / acc_b.  As soon as chunk C's codes
// have been consumed, the registers take the load of chunk C of the tile at
// `next` (two tiles ahead), and after the last chunk the scale bytes follow:
// the weight stream stays two tiles deep with only two register sets.
__device__ __forceinline__ void tile_mfma_prefetch(WTile& w, const uint16_t* xt, int lane, const uint8_t* next,
                                                   f32x16& acc_a, f32x16& acc_b) {
  const uint16_t* xl = xt + (lane & 31) * kXStride + 8 * (lane >> 5);
  f32x16 ta = {}, tb = {};
#define NVFP4_CHUNK(C)                                                                                         \
  chunk_mfma<C>(w.q[C], w.sa, w.sb, __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xl + 32 * C)), \
                __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xl + 32 * C + 16)), ta, tb);        \
  if (next) w.q[C] = load16(next + C * 1024 + lane * 16);
  NVFP4_CHUNK(0) NVFP4_CHUNK(1) NVFP4_CHUNK(2) NVFP4_CHUNK(3)
  NVFP4_CHUNK(4) NVFP4_CHUNK(5) NVFP4_CHUNK(6) NVFP4_CHUNK(7)
#undef NVFP4_CHUNK
  if (next) {
    w.sa = load16(next + kScaleOffset + 32 * (lane & 31));
    w.sb = load16(next + kScaleOffset + 32 * (lane & 31) + 16);
  }
  acc_a += ta;
  acc_b += tb;
}

// Activation staging: thread t (of 256) moves row t/8, k segment (t%8)*32 .. +32
// of a 256-k tile: four 16-byte loads, zero for absent rows and k >= K.
struct XStage {
  u32x4 v[4];
};

__device__ __forceinline__ void load_xstage(const uint16_t* xrow, int64_t kb, int64_t k, XStage& s) {
  const int seg = (threadIdx.x & 7) * 32;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t kk = kb + seg + 8 * i;
    s.v[i] = (xrow != nullptr && kk < k) ? load16(xrow + kk) : u32x4{0u, 0u, 0u, 0u};
  }
}

__device__ __forceinline__ void store_xstage(uint16_t* xt, const XStage& s) {
  u32x4* dst = reinterpret_cast<u32x4*>(xt + (threadIdx.x >> 3) * kXStride + (threadIdx.x & 7) * 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = s.v[i];
}

// Workgroup-cooperative skinny product (all 256 threads must call it).
//   wtile : this wavefront's 64-row tile (its k tile 0), or nullptr if idle
//   xrow  : this thread's staging row (row threadIdx.x/8 of the 32), nullptr = zeros
//   lds_x : 2 * kXTileElems bf16 of LDS
// acc_a / acc_b receive the tile rows 0-31 / 32-63 (see acc_row) for the 32
// activation rows (lane%32), summed over k tiles [kt0, kt1).
//
// Pipeline: two weight register sets (wa, wb) hold tiles t and t+1 while
// tile t+2 streams into wa chunk by chunk as tile t is consumed; two LDS
// buffers hold the activations of tiles t and t+1, and the activations of
// t+2 wait in registers.  Every stage issues its activation loads before its
// weight loads, so storing activations to LDS never waits for weights.
// Prefetches past the range re-read the range's last tile (harmless, and it
// keeps the unrolled code free of branches).
__device__ __forceinline__ void wg_skinny(const uint8_t* wtile, int kt0, int kt1, int64_t k, const uint16_t* xrow,
                                          uint16_t* lds_x, int lane, f32x16& acc_a, f32x16& acc_b) {
  if (kt0 >= kt1) return;
  const int last = kt1 - 1;
  auto wptr = [&](int kt) -> const uint8_t* {
    return wtile ? wtile + (size_t)(kt < last ? kt : last) * kTileBytes : nullptr;
  };
  auto xk = [&](int kt) -> int64_t { return (int64_t)(kt < last ? kt : last) * kTileK; };
  uint16_t* lds0 = lds_x;
  uint16_t* lds1 = lds_x + kXTileElems;
  XStage xs;
  WTile wa, wb;
  load_xstage(xrow, xk(kt0), k, xs);
  if (wtile) load_wtile(wptr(kt0), lane, wa);
  store_xstage(lds0, xs);
  load_xstage(xrow, xk(kt0 + 1), k, xs);
  if (wtile) load_wtile(wptr(kt0 + 1), lane, wb);
  for (int kt = kt0; kt < kt1; kt += 2) {
    __syncthreads();  // lds0 holds tile kt
    if (wtile) tile_mfma_prefetch(wa, lds0, lane, kt + 2 < kt1 ? wptr(kt + 2) : nullptr, acc_a, acc_b);
    if (kt + 1 >= kt1) break;
    store_xstage(lds1, xs);  // tile kt+1; lds1 was last read before the barrier above
    load_xstage(xrow, xk(kt + 2), k, xs);
    __syncthreads();  // lds1 holds tile kt+1
    if (wtile) tile_mfma_prefetch(wb, lds1, lane, kt + 3 < kt1 ? wptr(kt + 3) : nullptr, acc_a, acc_b);
    if (kt + 2 >= kt1) break;
    store_xstage(lds0, xs);  // tile kt+2; lds0 was last read before the barrier above
    load_xstage(xrow, xk(kt + 3), k, xs);
  }
  __syncthreads();  // the LDS buffers may be reused by the caller
}

// Row (within the 64-row tile) of accumulator element i held by `lane`.
__device__ __forceinline__ int acc_row(int half, int i, int lane) {
  return 32 * half + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

}  // namespace nvfp4
