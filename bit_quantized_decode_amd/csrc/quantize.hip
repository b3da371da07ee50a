// The NVFP4 quantiser -- fp32 or bf16 weights to canonical codes [n][k/2],
// E4M3 block scales [n][k/16] and one fp32 per-tensor scale; the step before
// the repack (the imp README, "How does it work?", converts weights to NVFP4
// once and then computes on them).
//
// Encoding (the pages name the format, not its encoder):
//   s_t     = amax / 2688: the largest magnitude lands on 6 (the largest E2M1
//             value) times 448 (the largest E4M3 value); 1 for a zero matrix;
//   scale_b = E4M3(amax_b / (6 s_t)), amax_b the block's largest magnitude;
//   code    = E2M1(w / (e4m3(scale_b) s_t)), sign bit = w's sign bit;
// both roundings go to the nearest value, ties to an even mantissa, and
// saturate (448, 6); a block whose scale is 0 gets code 0 throughout.  Every
// quotient and product is an fp32 operation in the order written, so each
// integer decision is taken in fp32.
//
// Two passes over the weights, both memory-bound (2 or 4 bytes read per
// weight, then 0.5625 written): workgroup maxima of the magnitudes, then one
// thread per 16-element block, each workgroup first taking the maximum of
// those maxima (a maximum does not depend on order: deterministic).
#include "device_common.h"
#include "launchers.h"

namespace nvfp4 {
namespace {

// Block of 16 consecutive elements starting at element `off` (32 or 64
// bytes, 16-byte aligned).
template <bool BF16>
__device__ __forceinline__ void load_block(const void* w, int64_t off, float (&v)[16]) {
  if (BF16) {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(w) + off);
    const u32x4 a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(a[i] << 16);
      v[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
      v[8 + 2 * i] = __uint_as_float(b[i] << 16);
      v[8 + 2 * i + 1] = __uint_as_float(b[i] & 0xffff0000u);
    }
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(w) + off);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 t = p[j];
      v[4 * j] = t[0];
      v[4 * j + 1] = t[1];
      v[4 * j + 2] = t[2];
      v[4 * j + 3] = t[3];
    }
  }
}

__device__ __forceinline__ float block_amax(const float (&v)[16]) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
  return m;
}

// E4M3FN byte nearest to q >= 0, ties to an even mantissa, 448 (0x7E) at and
// above 448.  Below 2^-6 the values are m * 2^-9 (m = 0..8; 8 is 2^-6, byte
// 0x08); above, the fp32 mantissa is rounded to 3 bits, a carry moving to the
// next exponent.
__device__ __forceinline__ uint32_t e4m3_nearest(float q) {
  if (q >= 448.0f) return 0x7Eu;
  if (q < 0.015625f) return (uint32_t)rintf(q * 512.0f);
  const uint32_t u = __float_as_uint(q);
  const uint32_t e = (u >> 23) - 127u + 7u;  // 1 .. 15
  uint32_t m = (u >> 20) & 7u;
  const uint32_t rest = u & 0xfffffu;
  if (rest > 0x80000u || (rest == 0x80000u && (m & 1u))) ++m;
  return (e << 3) + m;  // m == 8 carries into the exponent field
}

// Exact value of a finite non-negative E4M3FN byte.
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  const uint32_t e = b >> 3, m = b & 7u;
  return e == 0u ? (float)m * 0.001953125f : ldexpf((float)(8u + m), (int)e - 10);
}

// E2M1 magnitude code (0..7) nearest to a >= 0, ties to the even code, 7 (6.0)
// above 5: the count of grid midpoints below a, each midpoint counted when a
// passes it, or reaches it when the upper neighbour is the even code.
__device__ __forceinline__ uint32_t e2m1_nearest(float a) {
  return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) + (uint32_t)(a >= 1.75f) +
         (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
}

__device__ __forceinline__ float tensor_scale_of(float amax) { return amax > 0.0f ? amax / 2688.0f : 1.0f; }

// At most one workgroup of 1024 threads per CU, each thread four blocks per
// round (8 loads in flight); each workgroup writes its maximum to its own
// word, and the quantising pass takes the maximum of those (no atomics, no
// word to clear beforehand).
constexpr int kAmaxThreads = 1024;
constexpr int kAmaxUnroll = 4;

template <bool BF16>
__global__ __launch_bounds__(kAmaxThreads) void amax_kernel(const void* __restrict__ w, int64_t n, int64_t k,
                                                            int64_t ldw, float* __restrict__ part_max) {
  __shared__ float s_max[kAmaxThreads / 64];
  const int64_t bpr = k / 16, total = n * bpr;
  const int64_t stride = (int64_t)gridDim.x * kAmaxThreads;
  float m = 0.0f;
  for (int64_t t0 = (int64_t)blockIdx.x * kAmaxThreads + threadIdx.x; t0 < total; t0 += kAmaxUnroll * stride) {
    float v[kAmaxUnroll][16];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      const int64_t t = t0 + u * stride < total ? t0 + u * stride : t0;  // past the end: re-read block t0
      const int64_t r = t / bpr, b = t - r * bpr;
      load_block<BF16>(w, r * ldw + 16 * b, v[u]);
    }
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) m = fmaxf(m, block_amax(v[u]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x < 64) {
    m = threadIdx.x < kAmaxThreads / 64 ? s_max[threadIdx.x] : 0.0f;
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if (threadIdx.x == 0) part_max[blockIdx.x] = m;
  }
}

// The matrix's largest magnitude: the maximum of the `parts` workgroup maxima.
__device__ __forceinline__ float matrix_amax(const float* __restrict__ part_max, int parts) {
  __shared__ float s_red[4];
  float m = 0.0f;
  for (int i = threadIdx.x; i < parts; i += blockDim.x) m = fmaxf(m, part_max[i]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = m;
  __syncthreads();
  return fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
}

template <bool BF16>
__global__ __launch_bounds__(256) void quantize_kernel(const void* __restrict__ w, int64_t n, int64_t k,
                                                       int64_t ldw, const float* __restrict__ part_max, int parts,
                                                       uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                       float* __restrict__ st_out) {
  const float st = tensor_scale_of(matrix_amax(part_max, parts));
  const float six_st = 6.0f * st;
  if (blockIdx.x == 0 && threadIdx.x == 0) st_out[0] = st;
  const int64_t bpr = k / 16, total = n * bpr;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = t / bpr, b = t - r * bpr;
    float v[16];
    load_block<BF16>(w, r * ldw + 16 * b, v);
    const uint32_t sb = e4m3_nearest(block_amax(v) / six_st);
    uint32_t lo = 0u, hi = 0u;
    if (sb != 0u) {
      const float d = e4m3_value(sb) * st;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t c = e2m1_nearest(fabsf(v[i] / d)) | ((__float_as_uint(v[i]) >> 31) << 3);
        if (i < 8) lo |= c << (4 * i);
        else hi |= c << (4 * (i - 8));
      }
    }
    *reinterpret_cast<uint2*>(codes + r * (k / 2) + 8 * b) = make_uint2(lo, hi);
    scales[r * bpr + b] = (uint8_t)sb;
  }
}

unsigned grid_for(int64_t blocks16, int threads, int64_t cap) {
  const int64_t wgs = (blocks16 + threads - 1) / threads;
  return (unsigned)(wgs < cap ? (wgs > 0 ? wgs : 1) : cap);
}

}  // namespace

size_t quantize_workspace_bytes() { return 256 * sizeof(float); }

hipError_t launch_quantize(const void* w, bool bf16, int64_t n, int64_t k, int64_t ldw, uint8_t* codes,
                           uint8_t* scales, float* tensor_scale, void* ws, hipStream_t s) {
  float* part_max = static_cast<float*>(ws);  // one word per amax workgroup (at most 256)
  const int64_t blocks16 = n * (k / 16);
  const unsigned ga = grid_for(blocks16, kAmaxThreads, 256), gq = grid_for(blocks16, 256, 8192);
  if (bf16) {
    hipLaunchKernelGGL(amax_kernel<true>, dim3(ga), dim3(kAmaxThreads), 0, s, w, n, k, ldw, part_max);
    hipLaunchKernelGGL(quantize_kernel<true>, dim3(gq), dim3(256), 0, s, w, n, k, ldw, part_max, (int)ga, codes,
                       scales, tensor_scale);
  } else {
    hipLaunchKernelGGL(amax_kernel<false>, dim3(ga), dim3(kAmaxThreads), 0, s, w, n, k, ldw, part_max);
    hipLaunchKernelGGL(quantize_kernel<false>, dim3(gq), dim3(256), 0, s, w, n, k, ldw, part_max, (int)ga, codes,
                       scales, tensor_scale);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
