// a9: NVFP4 x bf16 GEMM for many activation rows (prompt prefill).
//
// y[i][j] = s_t * sum_k W[j][k] * x[i][k]
//
// Compute-bound: each weight is dequantised exactly to bf16 (E2M1 x E4M3 in
// fp32 is exact and fits bf16) into an LDS tile once per workgroup, and bf16
// MFMA does the product with fp32 accumulation; s_t is applied after
// accumulation.  A workgroup computes a 128 (activation rows) x 128 (weight
// rows) output tile over 64-k slabs; four wavefronts each own 64 x 64 of it
// (2 x 2 v_mfma_f32_32x32x16_bf16 tiles).  The next slab's global loads are
// in flight while the current slab is multiplied.  Accumulation is two-level
// (a fresh accumulator per 1024 k, then added to the running sum) to bound
// the roundings any output sees.
#include "device_common.h"
#include "launchers.h"

namespace nvfp4 {
namespace {

constexpr int kBM = 128;            // activation rows per workgroup
constexpr int kBN = 128;            // weight rows per workgroup (two 64-row tiles)
constexpr int kBK = 64;             // k per slab
constexpr int kLdsStride = kBK + 8; // bf16 elements per LDS row (16-byte pad against bank conflicts)
constexpr int kFlushSlabs = 16;     // slabs per first-level accumulation (1024 k)

struct Stage {
  u32x4 w;        // 32 codes of one weight row
  u32x4 x[4];     // 32 bf16 of one activation row
};

__global__ __launch_bounds__(256) void prefill_kernel(const uint8_t* __restrict__ packed, int64_t n, int64_t k,
                                                      int nkt, float st, const uint16_t* __restrict__ x, int64_t m,
                                                      int64_t ldx, void* __restrict__ y, int64_t ldy, int y_bf16) {
  __shared__ __attribute__((aligned(16))) uint16_t lds_w[kBN * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t lds_x[kBM * kLdsStride];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int64_t m0 = (int64_t)blockIdx.x * kBM;
  const int rt0 = blockIdx.y * 2;  // first of the two 64-row tiles
  const int64_t n0 = (int64_t)rt0 * kTileRows;

  // Weight loader: thread -> (row tile rtl, chunk parity cp, lane): one 16-byte
  // slot of the tile layout = rows r and 32 + r (r = lane % 32) x two 8-k groups.
  const int w_rtl = tid >> 7;
  const int w_cp = (tid >> 6) & 1;
  const bool w_tile_ok = (int64_t)(rt0 + w_rtl) * kTileRows < n;
  const uint8_t* w_base = packed + (size_t)(rt0 + w_rtl) * nkt * kTileBytes;
  const int w_r = lane & 31, w_h = lane >> 5;
  // Activation loader: thread -> (row tid/2, k half tid%2): 32 bf16.
  const int x_row = tid >> 1;
  const int x_half = tid & 1;
  const bool x_ok = m0 + x_row < m;
  const uint16_t* x_base = x + (x_ok ? (m0 + x_row) : 0) * ldx + 32 * x_half;

  const int nslabs = nkt * (kTileK / kBK);
  u32x4 sa = {0u, 0u, 0u, 0u}, sb = {0u, 0u, 0u, 0u};

  auto load = [&](int slab, Stage& st_) {
    const int kt = slab >> 2, sub = slab & 3;
    const int64_t kk = (int64_t)slab * kBK + 32 * x_half;
    if (w_tile_ok) st_.w = load16(w_base + (size_t)kt * kTileBytes + (2 * sub + w_cp) * 1024 + lane * 16);
    else st_.w = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (x_ok && kk + 8 * i < k) st_.x[i] = load16(x_base + (int64_t)slab * kBK + 8 * i);
      else st_.x[i] = u32x4{0u, 0u, 0u, 0u};
    }
  };

  // Wave tile: rows (weights) wn*64.., activation rows wm*64..
  const int wm = wave >> 1, wn = wave & 1;
  f32x16 acc[2][2], tot[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) { acc[i][j] = f32x16{}; tot[i][j] = f32x16{}; }

  Stage cur;
  if (nslabs > 0) load(0, cur);
  for (int slab = 0; slab < nslabs; ++slab) {
    const int kt = slab >> 2, sub = slab & 3;
    if (sub == 0 && w_tile_ok) {
      sa = load16(w_base + (size_t)kt * kTileBytes + kScaleOffset + 32 * w_r);
      sb = load16(w_base + (size_t)kt * kTileBytes + kScaleOffset + 32 * w_r + 16);
    }
    __syncthreads();  // previous slab fully consumed
    {
      // Dequantise the slot: dword d holds row r + 32*(d&1), k steps 2c + (d>>1)
      // of this k tile (c = 2*sub + cp), 8 codes at k offset 8h.
      const int c = 2 * sub + w_cp;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t sw = (d & 1) ? sb[c >> 1] : sa[c >> 1];
        const float s = __builtin_amdgcn_cvt_f32_fp8(sw >> (8 * ((2 * c + (d >> 1)) & 3)), 0);
        f32x2 v;
        u32x4 o;
        v = e2m1x2<0>(cur.w[d]); o[0] = pack_exact_bf16x2(v.x * s, v.y * s);
        v = e2m1x2<1>(cur.w[d]); o[1] = pack_exact_bf16x2(v.x * s, v.y * s);
        v = e2m1x2<2>(cur.w[d]); o[2] = pack_exact_bf16x2(v.x * s, v.y * s);
        v = e2m1x2<3>(cur.w[d]); o[3] = pack_exact_bf16x2(v.x * s, v.y * s);
        const int lrow = w_rtl * 64 + w_r + 32 * (d & 1);
        *reinterpret_cast<u32x4*>(lds_w + lrow * kLdsStride + 32 * w_cp + 8 * w_h + 16 * (d >> 1)) = o;
      }
      u32x4* xdst = reinterpret_cast<u32x4*>(lds_x + x_row * kLdsStride + 32 * x_half);
#pragma unroll
      for (int i = 0; i < 4; ++i) xdst[i] = cur.x[i];
    }
    __syncthreads();
    if (slab + 1 < nslabs) load(slab + 1, cur);

#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int kof = ks * 16 + 8 * (lane >> 5);
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                              lds_w + (wn * 64 + i * 32 + (lane & 31)) * kLdsStride + kof));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                              lds_x + (wm * 64 + j * 32 + (lane & 31)) * kLdsStride + kof));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if ((slab + 1) % kFlushSlabs == 0 || slab + 1 == nslabs) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) { tot[i][j] += acc[i][j]; acc[i][j] = f32x16{}; }
    }
  }

  // Epilogue: element e of tile (i, j) is weight row n0 + wn*64 + i*32 + 8*(e/4) + 4*(lane/32) + e%4,
  // activation row m0 + wm*64 + j*32 + lane%32.
  const bool vec = (ldy & 3) == 0;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t row = m0 + wm * 64 + j * 32 + (lane & 31);
      if (row >= m) continue;
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int64_t col = n0 + wn * 64 + i * 32 + 8 * e4 + 4 * (lane >> 5);
        const float v0 = tot[i][j][4 * e4 + 0] * st, v1 = tot[i][j][4 * e4 + 1] * st;
        const float v2 = tot[i][j][4 * e4 + 2] * st, v3 = tot[i][j][4 * e4 + 3] * st;
        if (y_bf16) {
          uint16_t* yr = static_cast<uint16_t*>(y) + row * ldy + col;
          if (vec && col + 4 <= n) {
            *reinterpret_cast<uint2*>(yr) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
          } else {
            if (col + 0 < n) yr[0] = to_bf16(v0);
            if (col + 1 < n) yr[1] = to_bf16(v1);
            if (col + 2 < n) yr[2] = to_bf16(v2);
            if (col + 3 < n) yr[3] = to_bf16(v3);
          }
        } else {
          float* yr = static_cast<float*>(y) + row * ldy + col;
          if (vec && col + 4 <= n) {
            *reinterpret_cast<f32x4*>(yr) = f32x4{v0, v1, v2, v3};
          } else {
            if (col + 0 < n) yr[0] = v0;
            if (col + 1 < n) yr[1] = v1;
            if (col + 2 < n) yr[2] = v2;
            if (col + 3 < n) yr[3] = v3;
          }
        }
      }
    }
}

}  // namespace

size_t prefill_workspace_bytes(int64_t, const Geometry&) { return 0; }

hipError_t launch_zero_rows(void* y, int64_t m, int64_t n, int64_t ldy, bool y_bf16, hipStream_t s);

hipError_t launch_prefill(const void* packed, const Geometry& g, float st, const uint16_t* x, int64_t m, int64_t ldx,
                          void* y, int64_t ldy, bool y_bf16, void*, hipStream_t s) {
  if (m == 0 || g.n == 0) return hipSuccess;
  if (g.k == 0) return launch_zero_rows(y, m, g.n, ldy, y_bf16, s);
  dim3 grid((unsigned)((m + kBM - 1) / kBM), (unsigned)((g.nrt + 1) / 2));
  hipLaunchKernelGGL(prefill_kernel, grid, dim3(256), 0, s, static_cast<const uint8_t*>(packed), g.n, g.k,
                     (int)g.nkt, st, x, m, ldx, y, ldy, y_bf16 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace nvfp4
