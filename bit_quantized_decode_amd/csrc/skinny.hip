// a3: NVFP4 x bf16 GEMM for up to 32 activation rows (a decode batch).
//
// y[i][j] = s_t * sum_k W[j][k] * x[i][k],   i < m <= 32.
//
// At 32 rows the product needs ~64 flop per weight byte -- more than the fp32
// vector units can deliver at HBM speed, so the weights are dequantised in
// registers to bf16 and fed to the matrix cores (skinny_core.h), while the
// kernel stays bound by the weight stream.  A workgroup of four wavefronts
// owns four 64-row tiles (one each) and a k range, sharing each activation
// tile through LDS; the k dimension is split across workgroups, whose partial
// sums meet in the workspace and are added in a fixed order by the last
// workgroup of the row group to arrive.
#include "device_common.h"
#include "launchers.h"
#include "skinny_core.h"

namespace nvfp4 {
namespace {

constexpr int kWaves = 4;

__host__ __device__ __forceinline__ int part_begin(int p, int nkt, int parts) {
  return (int)(((int64_t)p * nkt) / parts);
}

// Store 4 consecutive outputs (row .. row+3) of activation row `tok`.
__device__ __forceinline__ void store4(void* y, int y_bf16, int64_t ldy, int64_t tok, int64_t row, int64_t n,
                                       bool vec, float v0, float v1, float v2, float v3) {
  if (y_bf16) {
    uint16_t* yr = static_cast<uint16_t*>(y) + tok * ldy + row;
    if (vec && row + 4 <= n) {
      *reinterpret_cast<uint2*>(yr) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
    } else {
      if (row + 0 < n) yr[0] = to_bf16(v0);
      if (row + 1 < n) yr[1] = to_bf16(v1);
      if (row + 2 < n) yr[2] = to_bf16(v2);
      if (row + 3 < n) yr[3] = to_bf16(v3);
    }
  } else {
    float* yr = static_cast<float*>(y) + tok * ldy + row;
    if (vec && row + 4 <= n) {
      *reinterpret_cast<f32x4*>(yr) = f32x4{v0, v1, v2, v3};
    } else {
      if (row + 0 < n) yr[0] = v0;
      if (row + 1 < n) yr[1] = v1;
      if (row + 2 < n) yr[2] = v2;
      if (row + 3 < n) yr[3] = v3;
    }
  }
}

// Workgroup (row group rg, k part grp): four 64-row tiles 4*rg .. 4*rg+3, one
// per wavefront, over k tiles [part_begin(grp), part_begin(grp + 1)).
__global__ __launch_bounds__(256) void skinny_kernel(const uint8_t* __restrict__ packed, int64_t n, int64_t k,
                                                     int nkt, int nrt, int groups, float st,
                                                     const uint16_t* __restrict__ x, int64_t m, int64_t ldx,
                                                     void* __restrict__ y, int64_t ldy, int y_bf16,
                                                     unsigned* __restrict__ counters, float* __restrict__ partial,
                                                     int64_t np_tiles) {
  __shared__ __attribute__((aligned(16))) uint16_t lds_x[2 * kXTileElems];
  const int rg = blockIdx.x / groups;
  const int grp = blockIdx.x % groups;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int rt = rg * kWaves + wave;
  const int kt0 = part_begin(grp, nkt, groups), kt1 = part_begin(grp + 1, nkt, groups);
  const int stage_row = threadIdx.x >> 3;
  const uint16_t* xrow = stage_row < m ? x + stage_row * ldx : nullptr;
  f32x16 acc_a = {}, acc_b = {};
  wg_skinny(rt < nrt ? packed + (size_t)rt * nkt * kTileBytes : nullptr, kt0, kt1, k, xrow, lds_x, lane, acc_a,
            acc_b);

  const int tok = lane & 31;
  const bool vec = (ldy & 3) == 0;
  if (groups == 1) {
    if (rt >= nrt || tok >= m) return;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x16& a = h ? acc_b : acc_a;
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int64_t row = (int64_t)rt * kTileRows + acc_row(h, 4 * e4, lane);
        store4(y, y_bf16, ldy, tok, row, n, vec, a[4 * e4] * st, a[4 * e4 + 1] * st, a[4 * e4 + 2] * st,
               a[4 * e4 + 3] * st);
      }
    }
    return;
  }
  // Split k: partial[grp][rt][i][lane] = accumulator element i of this lane
  // (i < 16: acc_a, else acc_b) -- each element is one contiguous 256-byte run,
  // so the write-through stores go out as full lines.
  float* mine = partial + (((size_t)grp * np_tiles + rt) * 32) * 64 + lane;
  if (rt < nrt) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      store_coherent(mine + (size_t)i * 64, acc_a[i]);
      store_coherent(mine + (size_t)(16 + i) * 64, acc_b[i]);
    }
  }
  if (!arrive_last(counters + rg, (unsigned)groups)) return;
  // Last to arrive: each wavefront adds up its own tile's partials over the
  // groups in index order, two groups per round trip, and stores as above.
  if (rt >= nrt || tok >= m) return;
  f32x16 sa = {}, sb = {};
  const size_t gstride = (size_t)np_tiles * 32 * 64;
  const float* base = partial + ((size_t)rt * 32) * 64 + lane;
  for (int g0 = 0; g0 < groups; g0 += 2) {
    const int g1 = g0 + 1 < groups ? g0 + 1 : g0;
    float v0[32], v1[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      v0[i] = load_coherent(base + g0 * gstride + (size_t)i * 64);
      v1[i] = load_coherent(base + g1 * gstride + (size_t)i * 64);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sa[i] += v0[i];
      sb[i] += v0[16 + i];
    }
    if (g0 + 1 < groups) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sa[i] += v1[i];
        sb[i] += v1[16 + i];
      }
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const f32x16& a = h ? sb : sa;
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const int64_t row = (int64_t)rt * kTileRows + acc_row(h, 4 * e4, lane);
      store4(y, y_bf16, ldy, tok, row, n, vec, a[4 * e4] * st, a[4 * e4 + 1] * st, a[4 * e4 + 2] * st,
             a[4 * e4 + 3] * st);
    }
  }
}

__global__ void zero_rows_kernel(void* __restrict__ y, int64_t m, int64_t n, int64_t ldy, int y_bf16) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= m * n) return;
  int64_t r = i / n, c = i % n;
  if (y_bf16) static_cast<uint16_t*>(y)[r * ldy + c] = 0;
  else static_cast<float*>(y)[r * ldy + c] = 0.0f;
}

}  // namespace

// Row groups of 256 rows; k is split across `groups` workgroups so that about
// `target` workgroups stream at once, each keeping at least two k tiles.
SplitPlan skinny_plan(const Geometry& g) {
  const int64_t target = 384;
  const int64_t nrg = (g.nrt + kWaves - 1) / kWaves;
  int64_t groups = (target + nrg - 1) / nrg;
  int64_t max_groups = g.nkt / 2;
  if (max_groups < 1) max_groups = 1;
  if (groups > max_groups) groups = max_groups;
  if (groups > 8) groups = 8;
  if (groups < 1) groups = 1;
  return SplitPlan{(int)groups, (int)groups};
}

size_t skinny_workspace_bytes(const Geometry& g) {
  SplitPlan p = skinny_plan(g);
  if (p.groups <= 1) return 0;
  const size_t nrg = (size_t)(g.nrt + kWaves - 1) / kWaves;
  return kCounterBytes + (size_t)p.groups * nrg * kWaves * 32 * 64 * 4;
}

hipError_t launch_zero_rows(void* y, int64_t m, int64_t n, int64_t ldy, bool y_bf16, hipStream_t s) {
  int64_t total = m * n;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_rows_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, y, m, n, ldy,
                     y_bf16 ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_skinny(const void* packed, const Geometry& g, float st, const uint16_t* x, int64_t m, int64_t ldx,
                         void* y, int64_t ldy, bool y_bf16, void* ws, hipStream_t s) {
  if (m == 0 || g.n == 0) return hipSuccess;
  if (g.k == 0) return launch_zero_rows(y, m, g.n, ldy, y_bf16, s);
  SplitPlan p = skinny_plan(g);
  const int64_t nrg = (g.nrt + kWaves - 1) / kWaves;
  unsigned* counters = static_cast<unsigned*>(ws);
  float* partial = ws ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kCounterBytes) : nullptr;
  hipLaunchKernelGGL(skinny_kernel, dim3((unsigned)(nrg * p.groups)), dim3(256), 0, s,
                     static_cast<const uint8_t*>(packed), g.n, g.k, (int)g.nkt, (int)g.nrt, p.groups, st, x, m, ldx,
                     y, ldy, y_bf16 ? 1 : 0, counters, partial, nrg * kWaves);
  return hipGetLastError();
}

}  // namespace nvfp4
