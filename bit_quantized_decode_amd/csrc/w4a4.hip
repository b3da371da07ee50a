// f4: W4A4 prefill -- both operands in the OCP MX FP4 format (32 k elements
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
#include "device_common.h"
#include "launchers.h"

namespace nvfp4 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));

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

// Weights: canonical NVFP4 (codes [n][k/2], E4M3 scales [n][k/16]) -> MX tiles;
// one thread per (row, 32-k block) of the padded extent.
__global__ __launch_bounds__(256) void mx_pack_kernel(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales, MxGeom g,
                                                      uint8_t* __restrict__ dst) {
  const int64_t kbs = 2 * g.nks, total = g.nrb * 32 * kbs;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = t / kbs, kb = t % kbs;
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

// Activations: bf16 [m][ldx] -> MX tiles.
__global__ __launch_bounds__(256) void mx_quant_act_kernel(const uint16_t* __restrict__ x, int64_t ldx, MxGeom g,
                                                           uint8_t* __restrict__ dst) {
  const int64_t kbs = 2 * g.nks, total = g.nrb * 32 * kbs;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = t / kbs, kb = t % kbs;
    float v[32];
    if (row < g.rows && 32 * kb < g.k) {
      const u32x4* p = reinterpret_cast<const u32x4*>(x + row * ldx + 32 * kb);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 w = p[j];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[8 * j + 2 * i] = __uint_as_float(w[i] << 16);
          v[8 * j + 2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
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

// The product: a workgroup of four wavefronts computes 256 weight rows x 128
// activation rows.  Wavefront w owns weight blocks 2w and 2w + 1 (two A
// operands per 64-k step, loaded one step ahead into registers); the four
// activation blocks of a step (four B operands) are staged once per workgroup
// in LDS, double-buffered, one 16-byte load per thread; each wavefront then
// runs 2 x 4 MFMAs per step.
constexpr int kWJT = 4;        // activation blocks of 32 rows per workgroup
constexpr int kBStage = kWJT * 1024 + kWJT * 64;  // LDS bytes of one step's B operands

__device__ __forceinline__ v8i widen(u32x4 q) {
  return v8i{(int)q[0], (int)q[1], (int)q[2], (int)q[3], 0, 0, 0, 0};
}

__global__ __launch_bounds__(256, 2) void w4a4_gemm_kernel(const uint8_t* __restrict__ w, MxGeom gw,
                                                           const uint8_t* __restrict__ xm, MxGeom gx, float st,
                                                           void* __restrict__ y, int64_t ldy, int y_bf16) {
  __shared__ __attribute__((aligned(16))) uint8_t sb0[kBStage];
  __shared__ __attribute__((aligned(16))) uint8_t sb1[kBStage];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int64_t nks = gw.nks;
  // This wavefront's two weight blocks (past the end: the last block, not stored).
  int64_t wrb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t r = (int64_t)blockIdx.x * 8 + 2 * wave + i;
    wrb[i] = r < gw.nrb ? r : gw.nrb - 1;
  }
  const uint8_t* wsc = w + gw.scale_offset;
  // The B block this thread stages: codes of block tid / 64 (16 bytes at lane), and
  // for threads 0..15 a 16-byte run of the blocks' scales.
  const int sblk = tid >> 6;
  int64_t xrb = (int64_t)blockIdx.y * kWJT + sblk;
  xrb = xrb < gx.nrb ? xrb : gx.nrb - 1;
  const int64_t scb = (int64_t)blockIdx.y * kWJT + (tid >> 2);  // threads 0..15: block tid / 4, 16 scale bytes
  const int64_t scb_c = scb < gx.nrb ? scb : gx.nrb - 1;
  const uint8_t* xsc = xm + gx.scale_offset;
  auto load_b = [&](int64_t ks, u32x4& codes, u32x4& scales) __attribute__((always_inline)) {
    codes = *reinterpret_cast<const u32x4*>(xm + (xrb * nks + ks) * 1024 + lane * 16);
    if (tid < 16) scales = *reinterpret_cast<const u32x4*>(xsc + (scb_c * nks + ks) * 64 + (tid & 3) * 16);
  };
  auto store_b = [&](uint8_t* buf, u32x4 codes, u32x4 scales) __attribute__((always_inline)) {
    *reinterpret_cast<u32x4*>(buf + sblk * 1024 + lane * 16) = codes;
    if (tid < 16) *reinterpret_cast<u32x4*>(buf + kWJT * 1024 + (tid >> 2) * 64 + (tid & 3) * 16) = scales;
  };
  auto load_a = [&](int64_t ks, u32x4 (&a)[2], uint32_t (&sa)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      a[i] = *reinterpret_cast<const u32x4*>(w + (wrb[i] * nks + ks) * 1024 + lane * 16);
      sa[i] = wsc[(wrb[i] * nks + ks) * 64 + lane];
    }
  };
  f32x16 acc[2][kWJT];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < kWJT; ++j) acc[i][j] = f32x16{};
  u32x4 a[2], an[2], bc, bs = u32x4{0u, 0u, 0u, 0u};
  uint32_t sa[2], san[2];
  load_a(0, a, sa);
  load_b(0, bc, bs);
  store_b(sb0, bc, bs);
  __syncthreads();
  for (int64_t ks = 0; ks < nks; ++ks) {
    const int64_t kn = ks + 1 < nks ? ks + 1 : ks;
    load_a(kn, an, san);
    load_b(kn, bc, bs);
    const uint8_t* cur = (ks & 1) ? sb1 : sb0;
    u32x4 b[kWJT];
    uint32_t sbv[kWJT];
#pragma unroll
    for (int j = 0; j < kWJT; ++j) {
      b[j] = *reinterpret_cast<const u32x4*>(cur + j * 1024 + lane * 16);
      sbv[j] = cur[kWJT * 1024 + j * 64 + lane];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const v8i av = widen(a[i]);
#pragma unroll
      for (int j = 0; j < kWJT; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, widen(b[j]), acc[i][j], 4, 4, 0, (int)sa[i], 0,
                                                                    (int)sbv[j]);
    }
    store_b((ks & 1) ? sb0 : sb1, bc, bs);  // the other buffer: read by no wavefront this step
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      a[i] = an[i];
      sa[i] = san[i];
    }
  }
  // acc[i][j] element e: weight row 32 wrb_i + 8 (e / 4) + 4 (lane / 32) + e % 4,
  // activation row 32 (4 blockIdx.y + j) + lane % 32.
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t rb = (int64_t)blockIdx.x * 8 + 2 * wave + i;
    if (rb >= gw.nrb) continue;
#pragma unroll
    for (int j = 0; j < kWJT; ++j) {
      const int64_t arow = 32 * ((int64_t)blockIdx.y * kWJT + j) + (lane & 31);
      if (arow >= gx.rows) continue;
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int64_t col = 32 * rb + 8 * e4 + 4 * (lane >> 5);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (col + c >= gw.rows) continue;
          const float v = acc[i][j][4 * e4 + c] * st;
          if (y_bf16) static_cast<uint16_t*>(y)[arow * ldy + col + c] = to_bf16(v);
          else static_cast<float*>(y)[arow * ldy + col + c] = v;
        }
      }
    }
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
  hipLaunchKernelGGL(mx_quant_act_kernel, dim3(grid_of(g.nrb * 32 * 2 * g.nks)), dim3(256), 0, s, x, ldx, g,
                     static_cast<uint8_t*>(dst));
  return hipGetLastError();
}

hipError_t launch_w4a4_gemm(const void* mx_w, int64_t n, int64_t k, float st, const uint16_t* x, int64_t m,
                            int64_t ldx, void* y, int64_t ldy, bool y_bf16, void* ws, hipStream_t s) {
  const hipError_t e = launch_mx_quant_act(x, m, k, ldx, ws, s);
  if (e != hipSuccess) return e;
  const MxGeom gw = mx_geom(n, k), gx = mx_geom(m, k);
  const dim3 grid((unsigned)((gw.nrb + 7) / 8), (unsigned)((gx.nrb + kWJT - 1) / kWJT));
  hipLaunchKernelGGL(w4a4_gemm_kernel, grid, dim3(256), 0, s, static_cast<const uint8_t*>(mx_w), gw,
                     static_cast<const uint8_t*>(ws), gx, st, y, ldy, y_bf16 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace nvfp4
