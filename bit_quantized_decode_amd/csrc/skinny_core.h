// The skinny-product core shared by the decode-batch GEMM and the
// mixture-of-experts expert GEMMs (gate/up, down): a workgroup of four wavefronts
// multiplies four 64-row NVFP4 tiles (one per wavefront, possibly of different
// matrices), over a common range of 256-k tiles, by the same <= 32 bf16
// activation rows, on the bf16 matrix cores.
//
// Data flow per 256-k tile:
//  - the activation tile (32 rows x 256 k, 16 KB) goes from memory straight
//    into LDS (one 16-byte load per lane per 1 KB), once per workgroup, so
//    every wavefront reads it from LDS;
//  - one 1 KB wavefront load of a tile chunk (64 rows x 32 k) is already the
//    A operands of four v_mfma_f32_32x32x16_bf16 (rows 0-31 and 32-63, two k
//    steps of 16): lane l holds 8 consecutive k of rows l%32 and 32 + l%32
//    at k offset 8*(l/32), that instruction's operand layout;
//  - every weight is dequantised exactly: E2M1 -> fp32, times its E4M3 block
//    scale in fp32 (at most 6 significant bits, so exact), and the upper
//    half of that fp32 is its bf16.  The activations are the B operand: lane
//    l supplies activation row l%32's 8 values at the same k offset.
// Accumulation is two-level: each 256-k tile accumulates in a fresh fp32
// accumulator (16 MFMA steps), then is added to the running sum.  With the
// matrix instruction's measured error of at most 4 u of its inputs'
// magnitudes (u = 2^-24), a tile costs 64 u S and each running-sum add u S.
#pragma once

#include "device_common.h"

namespace nvfp4 {

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
  r.sa = load16_stream(tile + kScaleOffset + 32 * (lane & 31));
  r.sb = load16_stream(tile + kScaleOffset + 32 * (lane & 31) + 16);
#pragma unroll
  for (int c = 0; c < 8; ++c) r.q[c] = load16_stream(tile + c * 1024 + lane * 16);
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

// ---- activation tiles in LDS --------------------------------------------
// One tile is 16 KB: activation row r (of 32) at byte 512 r, its 16-byte
// chunk c (k 8c .. 8c+7 of the 256-k tile) at physical chunk c ^ (r % 16).
// Rows are contiguous, as the LDS loads write them, and the B-operand reads
// (rows 0-15 at one logical chunk) land in sixteen distinct bank groups.
constexpr int kXTileBytes = 32 * 512;

// B operands of chunk C (k 32C .. 32C+31) for this lane: row r = lane % 32,
// logical chunks 4C + lane/32 (xa) and 4C + 2 + lane/32 (xb).  With
// c = 4C + j (j < 4) the physical chunk is 4 (C ^ (r%16)/4) + (j ^ r%4):
// `abase_a` / `abase_b` hold 512 r + 16 (j ^ r%4) for the two j, `sw` holds
// 64 ((r%16)/4).
template <int C>
__device__ __forceinline__ void load_bops(const uint8_t* buf, uint32_t abase_a, uint32_t abase_b, uint32_t sw,
                                          bf16x8& xa, bf16x8& xb) {
  const uint32_t cofs = (uint32_t)(64 * C) ^ sw;
  xa = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(buf + cofs + abase_a));
  xb = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(buf + cofs + abase_b));
}

// Staging assignment: LDS load j (0..3) of wavefront w fills activation rows
// 8w + 2j (lanes 0-31) and 8w + 2j + 1 (lanes 32-63) of a tile; lane l
// fetches the logical chunk stored at physical chunk l % 32 of its row.
__device__ __forceinline__ int stage_row(int wave, int j, int lane) { return 8 * wave + 2 * j + (lane >> 5); }

// A resident weight tile times one activation tile in LDS into fresh
// accumulators ta / tb (16 matrix steps, chunk order -- the same arithmetic
// as one step of skinny_stream).
__device__ __forceinline__ void tile_product(const WTile& w, const uint8_t* buf, int lane, f32x16& ta,
                                             f32x16& tb) {
  const int br = lane & 31, bh = lane >> 5;
  const uint32_t abase_a = 512 * br + 16 * (bh ^ (br & 3));
  const uint32_t abase_b = 512 * br + 16 * ((2 + bh) ^ (br & 3));
  const uint32_t sw = 64 * ((br & 15) >> 2);
  bf16x8 xa, xb;
#define NVFP4_TP_CHUNK(C)                          \
  load_bops<C>(buf, abase_a, abase_b, sw, xa, xb); \
  chunk_mfma<C>(w.q[C], w.sa, w.sb, xa, xb, ta, tb);
  NVFP4_TP_CHUNK(0) NVFP4_TP_CHUNK(1) NVFP4_TP_CHUNK(2) NVFP4_TP_CHUNK(3)
  NVFP4_TP_CHUNK(4) NVFP4_TP_CHUNK(5) NVFP4_TP_CHUNK(6) NVFP4_TP_CHUNK(7)
#undef NVFP4_TP_CHUNK
}

// Sixteen zero bytes: the source of activation chunks past K.
static __device__ u32x4 g_zero_chunk;

template <int I>
__device__ __forceinline__ uint8_t* pick_buf(uint8_t* b0, uint8_t* b1, uint8_t* b2, uint8_t* b3) {
  return I == 0 ? b0 : I == 1 ? b1 : I == 2 ? b2 : b3;
}

// Workgroup-cooperative skinny product (all 256 threads call it, with the
// same kt0 / ntile).
//   wrow   : this wavefront's 64-row tile at k tile 0 (tile t at wrow + t * 9216)
//   kt0, ntile : k tiles [kt0, kt0 + ntile), ntile >= 1
//   k      : the product's K (activations past K load as zeros when !KFULL)
//   rowp   : for LDS load j, the activation row stage_row(wave, j, lane)
//            (rows past the real ones may repeat any real row: their
//            outputs are not used)
//   xb0..  : D distinct LDS arrays of kXTileBytes (distinct objects, so that
//            reads of one are not ordered after loads into another)
// acc_a / acc_b receive the tile rows 0-31 / 32-63 (see acc_row) for the 32
// activation rows (lane%32), summed over the k tiles.
//
// Pipeline (D = 3 or 4 steps deep, one step per k tile): the weights of tile
// i + D stream into the registers of tile i chunk by chunk as tile i is
// consumed (D register sets); the activations of tile i + D - 1 load into
// the LDS buffer that tile i - 1 used.  Per step a wavefront issues 4
// activation loads and then 10 weight loads, and memory operations complete
// in issue order: before the barrier that ends step i it waits for its loads
// of activation tile i + 1, which leaves the 10 + 14 (D - 2) operations
// issued after them in flight -- the weights of the next D - 1 tiles are not
// waited for.  Loads past the range re-read its last tile, so every step
// issues the same operations and the counts hold.
template <int D, bool KFULL>
__device__ __forceinline__ void skinny_stream(const uint8_t* wrow, int kt0, int ntile, int64_t k,
                                              const uint16_t* const (&rowp)[4], uint8_t* xb0, uint8_t* xb1,
                                              uint8_t* xb2, uint8_t* xb3, int wave, int lane, f32x16& acc_a,
                                              f32x16& acc_b) {
  static_assert(D == 3 || D == 4, "pipeline depth");
  constexpr int kAfterX = 10 + 14 * (D - 2);
  int cofs[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) cofs[j] = 8 * ((lane & 31) ^ (stage_row(wave, j, lane) & 15));
  const int last = ntile - 1;
  auto tile_of = [&](int i) __attribute__((always_inline)) { return kt0 + (i < last ? i : last); };
  // K <= 2^30 (checked by the callers' argument validation): 32-bit k offsets.
  // Chunks at k >= K (a ragged last tile) are loaded from a zero block.
  const int k32 = (int)k;
  auto load_x = [&](int i, uint8_t* buf) __attribute__((always_inline)) {
    const int kb = tile_of(i) * kTileK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint16_t* src = rowp[j] + kb + cofs[j];
      if (!KFULL && kb + cofs[j] >= k32) src = reinterpret_cast<const uint16_t*>(&g_zero_chunk);
      load_lds16(src, buf + 512 * (8 * wave + 2 * j));
    }
  };
  const uint32_t lane_code = lane * 16, lane_scale = kScaleOffset + 32 * (lane & 31);
  auto load_w = [&](int i, WTile& w) __attribute__((always_inline)) {
    const uint8_t* t = wrow + (size_t)tile_of(i) * kTileBytes;
    w.sa = load16_stream(t + lane_scale);
    w.sb = load16_stream(t + lane_scale + 16);
#pragma unroll
    for (int c = 0; c < 8; ++c) w.q[c] = load16_stream(t + c * 1024 + lane_code);
  };
  const int br = lane & 31, bh = lane >> 5;
  const uint32_t abase_a = 512 * br + 16 * (bh ^ (br & 3));
  const uint32_t abase_b = 512 * br + 16 * ((2 + bh) ^ (br & 3));
  const uint32_t sw0 = 64 * ((br & 15) >> 2);
  auto compute = [&](WTile& w, const uint8_t* buf, int inext) __attribute__((always_inline)) {
    const uint8_t* t = wrow + (size_t)tile_of(inext) * kTileBytes;
    uint32_t sw = sw0;
    asm volatile("" : "+v"(sw));  // formed per tile: keeps the 16 chunk addresses out of registers
    f32x16 ta = {}, tb = {};
    bf16x8 xa, xb;
#define NVFP4_SK_CHUNK(C)                                 \
  load_bops<C>(buf, abase_a, abase_b, sw, xa, xb);        \
  chunk_mfma<C>(w.q[C], w.sa, w.sb, xa, xb, ta, tb);      \
  w.q[C] = load16_stream(t + C * 1024 + lane_code);
    NVFP4_SK_CHUNK(0) NVFP4_SK_CHUNK(1) NVFP4_SK_CHUNK(2) NVFP4_SK_CHUNK(3)
    NVFP4_SK_CHUNK(4) NVFP4_SK_CHUNK(5) NVFP4_SK_CHUNK(6) NVFP4_SK_CHUNK(7)
#undef NVFP4_SK_CHUNK
    w.sa = load16_stream(t + lane_scale);
    w.sb = load16_stream(t + lane_scale + 16);
    acc_a += ta;
    acc_b += tb;
  };
  // Prologue in steady-state order: W(0), then x(j), W(j + 1) for j < D - 1.
  WTile w0, w1, w2, w3;
  load_w(0, w0);
  load_x(0, xb0);
  load_w(1, w1);
  load_x(1, xb1);
  load_w(2, w2);
  if (D == 4) {
    load_x(2, xb2);
    load_w(3, w3);
  }
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt_lgkm0<kAfterX>();  // x(0)
  barrier_only();
  __builtin_amdgcn_sched_barrier(0);
#define NVFP4_SK_STEP(S, W)                                                 \
  {                                                                         \
    const int i = i0 + (S);                                                 \
    load_x(i + D - 1, pick_buf<((S) + D - 1) % D>(xb0, xb1, xb2, xb3));     \
    __builtin_amdgcn_sched_barrier(0);                                      \
    compute(W, pick_buf<(S)>(xb0, xb1, xb2, xb3), i + D);                   \
    __builtin_amdgcn_sched_barrier(0);                                      \
    wait_vmcnt_lgkm0<kAfterX>();                                            \
    barrier_only();                                                         \
    __builtin_amdgcn_sched_barrier(0);                                      \
  }
  int i0 = 0;
  if (D == 3) {
    for (; i0 + 3 <= ntile; i0 += 3) {
      NVFP4_SK_STEP(0, w0)
      NVFP4_SK_STEP(1, w1)
      NVFP4_SK_STEP(2, w2)
    }
    if (i0 < ntile) NVFP4_SK_STEP(0, w0)
    if (i0 + 1 < ntile) NVFP4_SK_STEP(1, w1)
  } else {
    for (; i0 + 4 <= ntile; i0 += 4) {
      NVFP4_SK_STEP(0, w0)
      NVFP4_SK_STEP(1, w1)
      NVFP4_SK_STEP(2, w2)
      NVFP4_SK_STEP(3, w3)
    }
    if (i0 < ntile) NVFP4_SK_STEP(0, w0)
    if (i0 + 1 < ntile) NVFP4_SK_STEP(1, w1)
    if (i0 + 2 < ntile) NVFP4_SK_STEP(2, w2)
  }
#undef NVFP4_SK_STEP
  // Loads past the range still target LDS and registers; the caller may
  // reuse the buffers once every wavefront is past this point.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// Row (within the 64-row tile) of accumulator element i held by `lane`.
__device__ __forceinline__ int acc_row(int half, int i, int lane) {
  return 32 * half + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

}  // namespace nvfp4
