// a2: NVFP4 GEMV, one bf16 activation vector -> fp32 outputs.
//
// y[j] = s_t * sum_k e2m1(c[j][k]) * e4m3(sigma[j][k/16]) * x[k]
//
// The memory-bound decode product (the Ignis README's decode round is weight
// streaming at the card's bandwidth).  Mapping on gfx950:
//  - a wavefront owns one 64-row tile and a range of its 256-k tiles; lane l
//    owns row l, so every lane reads the same activations: x comes in through
//    scalar loads (wave-uniform) and never occupies vector registers or LDS;
//  - each 16-byte code load (32 weights) is converted two codes per
//    instruction to fp32 and multiplied into fp32 with x by FMA (products
//    exact); the E4M3 scale multiplies each 16-weight block partial, once;
//  - four wavefronts of a workgroup split the row tile's k range and meet in
//    LDS; several workgroups per row tile meet through the workspace, summed
//    in a fixed order by whichever arrives last (no float atomics).
// Rounding: every fp32 result passes through at most 16 (block) + 1 (scale)
// + 16 (tile) + (k tiles per wave) + 3 (wave merge) + (workgroups per row
// tile) + 1 (s_t) roundings; the plans below keep that under 100, i.e. an
// error below 100 * 2^-24 * sum|w x| = 6e-6 * sum|w x|.
#include "device_common.h"
#include "launchers.h"

namespace nvfp4 {
namespace {

constexpr int kGemvWaves = 4;

// 8 weights (code word `q`, 8 nibbles, k ascending) against 4 x pairs.
__device__ __forceinline__ float dot8(uint32_t q, uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3, float p) {
  f32x2 w;
  w = e2m1x2<0>(q); p = fmaf(w.x, bf16_lo(x0), p); p = fmaf(w.y, bf16_hi(x0), p);
  w = e2m1x2<1>(q); p = fmaf(w.x, bf16_lo(x1), p); p = fmaf(w.y, bf16_hi(x1), p);
  w = e2m1x2<2>(q); p = fmaf(w.x, bf16_lo(x2), p); p = fmaf(w.y, bf16_hi(x2), p);
  w = e2m1x2<3>(q); p = fmaf(w.x, bf16_lo(x3), p); p = fmaf(w.y, bf16_hi(x3), p);
  return p;
}

// One 32-k chunk (two scale blocks) of one row: returns acc + s0*p0 + s1*p1.
// `xc` points at the chunk's 16 x pairs in LDS (the same address in every lane).
template <int C>
__device__ __forceinline__ float chunk(u32x4 q, const uint32_t* xc, u32x4 sc, float acc) {
  const u32x4 xa = *reinterpret_cast<const u32x4*>(xc);
  const u32x4 xb = *reinterpret_cast<const u32x4*>(xc + 4);
  const u32x4 xc2 = *reinterpret_cast<const u32x4*>(xc + 8);
  const u32x4 xd = *reinterpret_cast<const u32x4*>(xc + 12);
  float p0 = dot8(q[0], xa[0], xa[1], xa[2], xa[3], 0.0f);
  p0 = dot8(q[1], xb[0], xb[1], xb[2], xb[3], p0);
  float p1 = dot8(q[2], xc2[0], xc2[1], xc2[2], xc2[3], 0.0f);
  p1 = dot8(q[3], xd[0], xd[1], xd[2], xd[3], p1);
  const float s0 = e4m3<(2 * C) % 4>(sc[C / 2]);
  const float s1 = e4m3<(2 * C + 1) % 4>(sc[C / 2]);
  acc = fmaf(p0, s0, acc);
  return fmaf(p1, s1, acc);
}

struct TileRegs {
  u32x4 sc;
  u32x4 q[8];
};

__device__ __forceinline__ void load_tile(const uint8_t* t, TileRegs& r) {
  r.sc = load16(t + kTileCodeBytes);
#pragma unroll
  for (int c = 0; c < 8; ++c) r.q[c] = load16(t + c * 1024);
}

// k tiles [kt(p), kt(p+1)) of part p when nkt tiles are cut into `parts` parts.
__host__ __device__ __forceinline__ int part_begin(int p, int nkt, int parts) {
  return (int)(((int64_t)p * nkt) / parts);
}

__global__ __launch_bounds__(256) void gemv_kernel(const uint8_t* __restrict__ packed, int64_t n, int64_t k,
                                                   int nkt, int groups, float st,
                                                   const uint32_t* __restrict__ x2, float* __restrict__ y,
                                                   unsigned* __restrict__ counters, float* __restrict__ partial,
                                                   int64_t np) {
  extern __shared__ u32x4 xs4[];  // this workgroup's k range of x, as bf16 pairs, zero past K
  const uint32_t* xs = reinterpret_cast<const uint32_t*>(xs4);
  const int rt = blockIdx.x / groups;
  const int grp = blockIdx.x % groups;
  // The wave index is uniform across the wavefront; saying so keeps the loop
  // bounds in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int parts = groups * kGemvWaves;
  const int wg_kt0 = part_begin(grp * kGemvWaves, nkt, parts);
  const int wg_kt1 = part_begin(grp * kGemvWaves + kGemvWaves, nkt, parts);
  const int kt0 = part_begin(grp * kGemvWaves + wave, nkt, parts);
  const int kt1 = part_begin(grp * kGemvWaves + wave + 1, nkt, parts);

  // Stage x for the workgroup's k range in LDS (16 bytes = 8 k per thread per step).
  {
    const int64_t k_base = (int64_t)wg_kt0 * kTileK;
    const int n16 = (wg_kt1 - wg_kt0) * (kTileK / 8);
    const u32x4* xg = reinterpret_cast<const u32x4*>(x2);
    for (int i = threadIdx.x; i < n16; i += 256) {
      const int64_t kk = k_base + 8 * (int64_t)i;
      xs4[i] = kk < k ? xg[kk >> 3] : u32x4{0u, 0u, 0u, 0u};
    }
  }

  const uint8_t* base = packed + (size_t)rt * nkt * kTileBytes + lane * 16;
  float acc = 0.0f;
  TileRegs cur, nxt;
  if (kt0 < kt1) load_tile(base + (size_t)kt0 * kTileBytes, cur);
  __syncthreads();
  for (int kt = kt0; kt < kt1; ++kt) {
    if (kt + 1 < kt1) load_tile(base + (size_t)(kt + 1) * kTileBytes, nxt);
    const uint32_t* xt = xs + (kt - wg_kt0) * (kTileK / 2);
    float a = 0.0f;
    a = chunk<0>(cur.q[0], xt + 0, cur.sc, a);
    a = chunk<1>(cur.q[1], xt + 16, cur.sc, a);
    a = chunk<2>(cur.q[2], xt + 32, cur.sc, a);
    a = chunk<3>(cur.q[3], xt + 48, cur.sc, a);
    a = chunk<4>(cur.q[4], xt + 64, cur.sc, a);
    a = chunk<5>(cur.q[5], xt + 80, cur.sc, a);
    a = chunk<6>(cur.q[6], xt + 96, cur.sc, a);
    a = chunk<7>(cur.q[7], xt + 112, cur.sc, a);
    acc += a;
    cur = nxt;
  }

  __shared__ float red[kGemvWaves][64];
  red[wave][lane] = acc;
  __syncthreads();
  const int64_t row = (int64_t)rt * kTileRows + lane;
  if (groups == 1) {
    if (wave == 0 && row < n) y[row] = (((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane]) * st;
    return;
  }
  if (wave == 0)
    store_coherent(partial + (size_t)grp * np + row, ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane]);
  if (arrive_last(counters + rt, (unsigned)groups)) {
    if (wave == 0 && row < n) {
      float s = 0.0f;
      for (int g2 = 0; g2 < groups; ++g2) s += load_coherent(partial + (size_t)g2 * np + row);
      y[row] = s * st;
    }
  }
}

__global__ void zero_f32_kernel(float* __restrict__ y, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = 0.0f;
}

}  // namespace

SplitPlan gemv_plan(const Geometry& g) {
  // Enough workgroups that all 256 CUs stream, each wave keeping >= 1 k tile.
  const int64_t target = 512;
  int64_t groups = (target + g.nrt - 1) / g.nrt;
  int64_t max_groups = g.nkt / kGemvWaves;
  if (max_groups < 1) max_groups = 1;
  if (groups > max_groups) groups = max_groups;
  if (groups > 16) groups = 16;
  // At most 64 k tiles (32 KB of x) per workgroup in LDS.
  const int64_t min_groups = (g.nkt + 63) / 64;
  if (groups < min_groups) groups = min_groups;
  if (groups < 1) groups = 1;
  return SplitPlan{(int)groups, (int)groups * kGemvWaves};
}

// Largest k range (in tiles) any workgroup stages.
static int max_wg_tiles(const Geometry& g, const SplitPlan& p) {
  int m = 0;
  for (int grp = 0; grp < p.groups; ++grp) {
    int t = part_begin(grp * kGemvWaves + kGemvWaves, (int)g.nkt, p.parts) - part_begin(grp * kGemvWaves, (int)g.nkt, p.parts);
    if (t > m) m = t;
  }
  return m;
}

size_t gemv_workspace_bytes(const Geometry& g) {
  SplitPlan p = gemv_plan(g);
  if (p.groups <= 1) return 0;
  return kCounterBytes + (size_t)p.groups * (size_t)g.nrt * 64 * 4;
}

hipError_t launch_gemv(const void* packed, const Geometry& g, float st, const uint16_t* x, float* y, void* ws,
                       hipStream_t s) {
  if (g.n == 0) return hipSuccess;
  if (g.k == 0) {
    hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)((g.n + 255) / 256)), dim3(256), 0, s, y, g.n);
    return hipGetLastError();
  }
  SplitPlan p = gemv_plan(g);
  unsigned* counters = static_cast<unsigned*>(ws);
  float* partial = ws ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kCounterBytes) : nullptr;
  const size_t smem = (size_t)max_wg_tiles(g, p) * (kTileK / 2) * 4;
  hipLaunchKernelGGL(gemv_kernel, dim3((unsigned)(g.nrt * p.groups)), dim3(256), smem, s,
                     static_cast<const uint8_t*>(packed), g.n, g.k, (int)g.nkt, p.groups, st,
                     reinterpret_cast<const uint32_t*>(x), y, counters, partial, g.nrt * 64);
  return hipGetLastError();
}

}  // namespace nvfp4
