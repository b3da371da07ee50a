// W4A4 prefill -- both operands in the OCP MX FP4 format (32 k elements
// per E8M0 power-of-two scale) on gfx950's scaled FP4 matrix instruction
// v_mfma_scale_f32_32x32x64_f8f6f4, the native-FP4 design point of the pages'
// prefill (imp README, "How does it work?").  An approximation of the NVFP4
// product: the weights' E4M3 scales per 16 and the bf16 activations are both
// requantised to MX blocks of 32.
//
// MX block rule (OCP MX v1.0 conversion): scale X = 2^(floor(log2 amax) - 2),
// exponent clamped to [-127, 127], byte 127 + exponent; codes = nearest E2M1
// value of v / X (exact: X is a power of two), ties to the even mantissa,
// +-6 beyond 6, sign bit = v's; an all-zero block has byte 0 and zero codes.
//
// Operand layout ("MX tiles"), the same for weights and activations: blocks of
// 32 rows x 64 k; block (rb, ks) holds 1 KB of codes at (rb * nks + ks) * 1024,
// lane l's 16 bytes at 16 l: row 32 rb + l % 32, k = 64 ks + 32 (l / 32) + j
// (j = 0..31, low nibble first) -- exactly the instruction's A / B operand for
// one lane -- and 64 scale bytes, after all codes, at (rb * nks + ks) * 64 + l.
// Rows past the matrix and k past K are zero.
//
// This file holds the conversions into that layout and the entry points; the
// product itself is the prefill's stream-K kernel with MX operands
// (prefill.hip): x is quantised into the workspace, problem by problem, and
// one launch covers up to eight products.
#include <vector>

#include "device_common.h"
#include "launchers.h"

namespace nvfp4 {
namespace {


__device__ __forceinline__ uint32_t e2m1_code(float a) {
  return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) + (uint32_t)(a >= 1.75f) +
         (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
}

// 32 values -> 16 code bytes (as four dwords) and the E8M0 byte.
__device__ __forceinline__ void mx_block(const float (&v)[32], u32x4& codes, uint32_t& scale) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  codes = u32x4{0u, 0u, 0u, 0u};
  if (amax == 0.0f) {
    scale = 0u;
    return;
  }
  int ex = ilogbf(amax) - 2;
  ex = ex < -127 ? -127 : (ex > 127 ? 127 : ex);
  scale = (uint32_t)(ex + 127);
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t c = e2m1_code(ldexpf(fabsf(v[i]), -ex)) | ((__float_as_uint(v[i]) >> 31) << 3);
    codes[i / 8] |= c << (4 * (i % 8));
  }
}

struct MxGeom {
  int64_t rows, k, nrb, nks;
  size_t scale_offset;  // bytes of the code region
};

__host__ __device__ inline MxGeom mx_geom(int64_t rows, int64_t k) {
  MxGeom g;
  g.rows = rows;
  g.k = k;
  g.nrb = (rows + 31) / 32;
  g.nks = (k + 63) / 64;
  g.scale_offset = (size_t)g.nrb * g.nks * 1024;
  return g;
}

// Where (row, 32-k block kb) goes in the MX tiles.
__device__ __forceinline__ void mx_put(uint8_t* dst, const MxGeom& g, int64_t row, int64_t kb, u32x4 codes,
                                       uint32_t scale) {
  const int64_t blk = (row / 32) * g.nks + kb / 2;
  const int lane = (int)(row % 32) + 32 * (int)(kb % 2);
  *reinterpret_cast<u32x4*>(dst + blk * 1024 + lane * 16) = codes;
  dst[g.scale_offset + blk * 64 + lane] = (uint8_t)scale;
}

// Thread t works on the element of MX tile (rb, ks) = t / 64 that lane t % 64
// of the matrix instruction holds: row 32 rb + t % 32, 32-k block 2 ks + t % 64
// / 32.  A wavefront thus writes one tile's kilobyte of codes and 64 scale
// bytes, each contiguously.
__device__ __forceinline__ void mx_element(int64_t t, int64_t nks, int64_t& row, int64_t& kb) {
  const int64_t tile = t >> 6;
  const int l = (int)(t & 63);
  row = 32 * (tile / nks) + (l & 31);
  kb = 2 * (tile % nks) + (l >> 5);
}

// Weights: canonical NVFP4 (codes [n][k/2], E4M3 scales [n][k/16]) -> MX tiles;
// one thread per (row, 32-k block) of the padded extent.
__global__ __launch_bounds__(256) void mx_pack_kernel(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales, MxGeom g,
                                                      uint8_t* __restrict__ dst) {
  const int64_t kbs = 2 * g.nks, total = g.nrb * 32 * kbs;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
    int64_t row, kb;
    mx_element(t, g.nks, row, kb);
    float v[32];
    if (row < g.rows && 32 * kb < g.k) {
      const u32x4 q = *reinterpret_cast<const u32x4*>(codes + row * (g.k / 2) + 16 * kb);
      const uint32_t s2 = *reinterpret_cast<const uint16_t*>(scales + row * (g.k / 16) + 2 * kb);
      const float sa = e4m3<0>(s2), sb = e4m3<1>(s2);
#pragma unroll
      for (int d = 0; d < 4; ++d) {  // dword d: elements 8 d .. 8 d + 7, two per byte
        const f32x2 p0 = e2m1x2<0>(q[d]), p1 = e2m1x2<1>(q[d]), p2 = e2m1x2<2>(q[d]), p3 = e2m1x2<3>(q[d]);
        const float sc = d < 2 ? sa : sb;  // the exact weight value: E2M1 times its E4M3 scale
        v[8 * d] = p0.x * sc;
        v[8 * d + 1] = p0.y * sc;
        v[8 * d + 2] = p1.x * sc;
        v[8 * d + 3] = p1.y * sc;
        v[8 * d + 4] = p2.x * sc;
        v[8 * d + 5] = p2.y * sc;
        v[8 * d + 6] = p3.x * sc;
        v[8 * d + 7] = p3.y * sc;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = 0.0f;
    }
    u32x4 out;
    uint32_t sc;
    mx_block(v, out, sc);
    mx_put(dst, g, row, kb, out, sc);
  }
}

// Activations: bf16 [m][ldx] -> MX tiles; four threads per (row, 32-k
// block), each converting 8 k (one dword of the 16 code bytes), with the
// block's largest magnitude combined across the four.
__global__ __launch_bounds__(256) void mx_quant_act_kernel(const uint16_t* __restrict__ x, int64_t ldx, MxGeom g,
                                                           uint8_t* __restrict__ dst) {
  const int64_t total = g.nrb * 32 * (2 * g.nks) * 4;  // a multiple of 4: quads are never split
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
    const int j = (int)(t & 3);
    int64_t row, kb;
    mx_element(t >> 2, g.nks, row, kb);
    float v[8];
    if (row < g.rows && 32 * kb < g.k) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(x + row * ldx + 32 * kb + 8 * j);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 4));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 4));
    uint32_t code = 0u, scale = 0u;
    if (amax != 0.0f) {
      int ex = ilogbf(amax) - 2;
      ex = ex < -127 ? -127 : (ex > 127 ? 127 : ex);
      scale = (uint32_t)(ex + 127);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        code |= (e2m1_code(ldexpf(fabsf(v[i]), -ex)) | ((__float_as_uint(v[i]) >> 31) << 3)) << (4 * i);
    }
    const int64_t blk = (row / 32) * g.nks + kb / 2;
    const int lane = (int)(row % 32) + 32 * (int)(kb % 2);
    reinterpret_cast<uint32_t*>(dst + blk * 1024 + lane * 16)[j] = code;
    if (j == 0) dst[g.scale_offset + blk * 64 + lane] = (uint8_t)scale;
  }
}

// Test hook: MX tiles -> canonical MX (codes [rows][k/2], scales [rows][k/32]).
__global__ __launch_bounds__(256) void mx_unpack_kernel(const uint8_t* __restrict__ src, MxGeom g,
                                                        uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t kbs = g.k / 32, total = g.rows * kbs;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = t / kbs, kb = t % kbs;
    const int64_t blk = (row / 32) * g.nks + kb / 2;
    const int lane = (int)(row % 32) + 32 * (int)(kb % 2);
    *reinterpret_cast<u32x4*>(codes + row * (g.k / 2) + 16 * kb) = *reinterpret_cast<const u32x4*>(src + blk * 1024 + lane * 16);
    scales[row * kbs + kb] = src[g.scale_offset + blk * 64 + lane];
  }
}

unsigned grid_of(int64_t items) {
  const int64_t wgs = (items + 255) / 256;
  return (unsigned)(wgs < 16384 ? (wgs > 0 ? wgs : 1) : 16384);
}

}  // namespace

size_t mx_packed_bytes(int64_t rows, int64_t k) {
  const MxGeom g = mx_geom(rows, k);
  return (size_t)g.nrb * g.nks * (1024 + 64);
}

hipError_t launch_mx_pack(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k, void* dst, hipStream_t s) {
  const MxGeom g = mx_geom(n, k);
  hipLaunchKernelGGL(mx_pack_kernel, dim3(grid_of(g.nrb * 32 * 2 * g.nks)), dim3(256), 0, s, codes, scales, g,
                     static_cast<uint8_t*>(dst));
  return hipGetLastError();
}

hipError_t launch_mx_unpack(const void* src, int64_t rows, int64_t k, uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const MxGeom g = mx_geom(rows, k);
  hipLaunchKernelGGL(mx_unpack_kernel, dim3(grid_of(rows * (k / 32))), dim3(256), 0, s,
                     static_cast<const uint8_t*>(src), g, codes, scales);
  return hipGetLastError();
}

hipError_t launch_mx_quant_act(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, void* dst, hipStream_t s) {
  const MxGeom g = mx_geom(m, k);
  hipLaunchKernelGGL(mx_quant_act_kernel, dim3(grid_of(g.nrb * 32 * 2 * g.nks * 4)), dim3(256), 0, s, x, ldx, g,
                     static_cast<uint8_t*>(dst));
  return hipGetLastError();
}

size_t w4a4_batch_workspace_bytes(const Problem* p, int count, int64_t m) {
  size_t need = w4a4_streamk_bytes();
  for (int i = 0; i < count; ++i)
    if (p[i].n > 0 && p[i].k > 0) need += mx_packed_bytes(m, p[i].k);
  return need;
}

size_t w4a4_workspace_bytes(int64_t m, int64_t k) { return w4a4_streamk_bytes() + mx_packed_bytes(m, k); }

hipError_t launch_w4a4_gemm_batch(const Problem* p, int count, int64_t m, bool y_bf16, void* ws, hipStream_t s) {
  if (m <= 0 || count <= 0) return hipSuccess;
  std::vector<MxProblem> q;
  q.reserve((size_t)count);
  // Workspace: the stream-K counters and partial sums, then each problem's x as MX tiles.
  uint8_t* xmx = static_cast<uint8_t*>(ws) + w4a4_streamk_bytes();
  for (int i = 0; i < count; ++i) {
    if (p[i].n <= 0) continue;
    if (p[i].k <= 0) {
      const hipError_t e = launch_zero_rows(p[i].y, m, p[i].n, p[i].ldy, y_bf16, s);
      if (e != hipSuccess) return e;
      continue;
    }
    const hipError_t e = launch_mx_quant_act(p[i].x, m, p[i].k, p[i].ldx, xmx, s);
    if (e != hipSuccess) return e;
    q.push_back(MxProblem{static_cast<const uint8_t*>(p[i].packed), p[i].n, p[i].k, p[i].st, xmx, p[i].y, p[i].ldy});
    xmx += mx_packed_bytes(m, p[i].k);
  }
  return launch_w4a4_batch(q.data(), (int)q.size(), m, y_bf16, ws, s);
}

hipError_t launch_w4a4_gemm(const void* mx_w, int64_t n, int64_t k, float st, const uint16_t* x, int64_t m,
                            int64_t ldx, void* y, int64_t ldy, bool y_bf16, void* ws, hipStream_t s) {
  const Problem p{mx_w, n, k, st, x, ldx, y, ldy};
  return launch_w4a4_gemm_batch(&p, 1, m, y_bf16, ws, s);
}

}  // namespace nvfp4
