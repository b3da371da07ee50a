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
//  - per 16-byte lane load (row l of the tile, 32 consecutive k) the wavefront
//    holds a 64 x 32 weight slab; two lane-half exchanges turn it into the A
//    operands of four v_mfma_f32_32x32x16_bf16 (rows 0-31 and 32-63, two k
//    steps of 16): lane l then holds 8 consecutive k of row l%32 (or
//    32 + l%32) at k offset 8*(l/32) -- that instruction's operand layout;
//  - every weight is dequantised exactly: E2M1 -> fp32, times its E4M3 block
//    scale in fp32 (at most 6 significant bits, so exact), rounded to bf16
//    (exact, since the value fits in bf16).  The activations are the B
//    operand: lane l supplies row l%32's 8 values at the same k offset.
// Accumulation is two-level: each 256-k tile accumulates in a fresh fp32
// accumulator (16 MFMA steps), then is added to the running sum.
#pragma once

#include "device_common.h"

namespace nvfp4 {

constexpr int kXStride = kTileK + 8;  // bf16 per LDS activation row (16-byte pad: conflict-free reads)
constexpr int kXTileElems = 32 * kXStride;

// Eight weights of one k step: code word `w` (8 nibbles, k ascending) times scale `s`.
__device__ __forceinline__ bf16x8 dequant8(uint32_t w, float s) {
  u32x4 r;
  f32x2 v;
  v = e2m1x2<0>(w); r[0] = pack_bf16x2(v.x * s, v.y * s);
  v = e2m1x2<1>(w); r[1] = pack_bf16x2(v.x * s, v.y * s);
  v = e2m1x2<2>(w); r[2] = pack_bf16x2(v.x * s, v.y * s);
  v = e2m1x2<3>(w); r[3] = pack_bf16x2(v.x * s, v.y * s);
  return __builtin_bit_cast(bf16x8, r);
}

struct WTile {
  u32x4 sc;
  u32x4 q[8];
};

__device__ __forceinline__ void load_wtile(const uint8_t* t, WTile& r) {
  r.sc = load16(t + kTileCodeBytes);
#pragma unroll
  for (int c = 0; c < 8; ++c) r.q[c] = load16(t + c * 1024);
}

// One 32-k chunk C of a tile: four MFMAs into the two tile accumulators.
template <int C>
__device__ __forceinline__ void chunk_mfma(u32x4 q, const uint32_t (&sa)[4], const uint32_t (&sb)[4], bf16x8 xa,
                                           bf16x8 xb, f32x16& ta, f32x16& tb) {
  uint32_t d0 = q[0], d1 = q[1], d2 = q[2], d3 = q[3];
  // Before: lane r < 32 holds row r (k 0-7, 8-15, 16-23, 24-31), lane r+32 holds
  // row r+32.  After: d0 = rows 0-31 step 0, d1 = rows 32-63 step 0,
  // d2 = rows 0-31 step 1, d3 = rows 32-63 step 1, in MFMA operand order.
  swap_halves(d0, d1);
  swap_halves(d2, d3);
  const float s_a0 = e4m3<(2 * C) % 4>(sa[C / 2]);
  const float s_b0 = e4m3<(2 * C) % 4>(sb[C / 2]);
  const float s_a1 = e4m3<(2 * C + 1) % 4>(sa[C / 2]);
  const float s_b1 = e4m3<(2 * C + 1) % 4>(sb[C / 2]);
  ta = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dequant8(d0, s_a0), xa, ta, 0, 0, 0);
  tb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dequant8(d1, s_b0), xa, tb, 0, 0, 0);
  ta = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dequant8(d2, s_a1), xb, ta, 0, 0, 0);
  tb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dequant8(d3, s_b1), xb, tb, 0, 0, 0);
}

// Multiply one resident weight tile by the activation tile in LDS (`xt`, 32 rows
// of kXStride bf16) and add the tile's sum into acc_a / acc_b.
__device__ __forceinline__ void tile_mfma(const WTile& w, const uint16_t* xt, int lane, f32x16& acc_a,
                                          f32x16& acc_b) {
  uint32_t sa[4], sb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sa[i] = w.sc[i];
    sb[i] = w.sc[i];
    swap_halves(sa[i], sb[i]);  // sa: scales of row lane%32, sb: of row 32 + lane%32
  }
  const uint16_t* xl = xt + (lane & 31) * kXStride + 8 * (lane >> 5);
  f32x16 ta = {}, tb = {};
#define NVFP4_CHUNK(C)                                                                             \
  chunk_mfma<C>(w.q[C], sa, sb, __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xl + 32 * C)), \
                __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xl + 32 * C + 16)), ta, tb);
  NVFP4_CHUNK(0) NVFP4_CHUNK(1) NVFP4_CHUNK(2) NVFP4_CHUNK(3)
  NVFP4_CHUNK(4) NVFP4_CHUNK(5) NVFP4_CHUNK(6) NVFP4_CHUNK(7)
#undef NVFP4_CHUNK
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
__device__ __forceinline__ void wg_skinny(const uint8_t* wtile, int kt0, int kt1, int64_t k, const uint16_t* xrow,
                                          uint16_t* lds_x, int lane, f32x16& acc_a, f32x16& acc_b) {
  if (kt0 >= kt1) return;
  const uint8_t* wl = wtile ? wtile + lane * 16 : nullptr;
  WTile cur, nxt;
  XStage xs;
  if (wl) load_wtile(wl + (size_t)kt0 * kTileBytes, cur);
  load_xstage(xrow, (int64_t)kt0 * kTileK, k, xs);
  store_xstage(lds_x, xs);
  int buf = 0;
  for (int kt = kt0; kt < kt1; ++kt) {
    const bool more = kt + 1 < kt1;
    if (more) {
      if (wl) load_wtile(wl + (size_t)(kt + 1) * kTileBytes, nxt);
      load_xstage(xrow, (int64_t)(kt + 1) * kTileK, k, xs);
    }
    __syncthreads();  // LDS buffer `buf` is complete
    if (wl) tile_mfma(cur, lds_x + buf * kXTileElems, lane, acc_a, acc_b);
    if (more) {
      // Buffer buf^1 was last read in the previous iteration, which every
      // thread finished before the barrier above.
      store_xstage(lds_x + (buf ^ 1) * kXTileElems, xs);
      cur = nxt;
    }
    buf ^= 1;
  }
  __syncthreads();  // the LDS buffers may be reused by the caller
}

// Row (within the 64-row tile) of accumulator element i held by `lane`.
__device__ __forceinline__ int acc_row(int half, int i, int lane) {
  return 32 * half + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

}  // namespace nvfp4
