// NVFP4 x bf16 GEMM for up to 32 activation rows (a decode batch).
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

// A batch of up to kMaxBatch skinny products sharing m and the output type;
// workgroups [wg_begin[p], wg_begin[p+1]) belong to problem p.  Within a
// problem, workgroup (row group rg, k part grp) owns the four 64-row tiles
// 4*rg .. 4*rg+3, one per wavefront, over k tiles [part_begin(grp),
// part_begin(grp + 1)).
struct SkinnyBatch {
  int count;
  int wg_begin[kMaxBatch + 1];
  const uint8_t* packed[kMaxBatch];
  const uint16_t* x[kMaxBatch];
  void* y[kMaxBatch];
  int64_t ldx[kMaxBatch];
  int64_t ldy[kMaxBatch];
  int64_t n[kMaxBatch];
  int64_t k[kMaxBatch];
  int nkt[kMaxBatch];
  int nrt[kMaxBatch];
  int groups[kMaxBatch];
  float st[kMaxBatch];
  int counter_base[kMaxBatch];
  int64_t partial_base[kMaxBatch];  // floats
};

template <bool KFULL>
__global__ __launch_bounds__(256, 2) void skinny_kernel(const SkinnyBatch b, int64_t m, int y_bf16,
                                                        unsigned* __restrict__ counters,
                                                        float* __restrict__ partial_all) {
  __shared__ __attribute__((aligned(16))) uint8_t xb0[kXTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t xb1[kXTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t xb2[kXTileBytes];
  int p = 0;
  while (p + 1 < b.count && (int)blockIdx.x >= b.wg_begin[p + 1]) ++p;
  const int groups = b.groups[p], nkt = b.nkt[p], nrt = b.nrt[p];
  const int64_t n = b.n[p], k = b.k[p], ldx = b.ldx[p], ldy = b.ldy[p];
  const float st = b.st[p];
  void* __restrict__ y = b.y[p];
  const int local = (int)blockIdx.x - b.wg_begin[p];
  const int rg = local / groups;
  const int grp = local % groups;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int rt = rg * kWaves + wave;
  const int kt0 = part_begin(grp, nkt, groups), kt1 = part_begin(grp + 1, nkt, groups);
  // Activation rows past m repeat row m - 1; a wavefront past the last row
  // tile streams the last one (neither result is stored).
  const uint16_t* rowp[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = stage_row(wave, j, lane);
    rowp[j] = b.x[p] + (int64_t)(r < m ? r : m - 1) * ldx;
  }
  const uint8_t* wrow = b.packed[p] + (size_t)(rt < nrt ? rt : nrt - 1) * nkt * kTileBytes;
  f32x16 acc_a = {}, acc_b = {};
  skinny_stream<3, KFULL>(wrow, kt0, kt1 - kt0, k, rowp, xb0, xb1, xb2, xb2, wave, lane, acc_a, acc_b);

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
  const int np_tiles = ((nrt + kWaves - 1) / kWaves) * kWaves;
  float* partial = partial_all + b.partial_base[p];
  float* mine = partial + (((size_t)grp * np_tiles + rt) * 32) * 64 + lane;
  if (rt < nrt) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      store_coherent(mine + (size_t)i * 64, acc_a[i]);
      store_coherent(mine + (size_t)(16 + i) * 64, acc_b[i]);
    }
  }
  if (!arrive_last(counters + b.counter_base[p] + rg, (unsigned)groups)) return;
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

// K parts per problem for a batch: aim at about 2048 wavefronts over the whole
// batch (two per SIMD), i.e. `tpw` k tiles per wavefront, with at most 12 parts
// per row group (bounding the last workgroup's reduction) and none empty --
// but at least one part per 64 k tiles, so that no wavefront's running sum
// chains more than 64 tile sums (the accumulation bound).
int skinny_groups(const Geometry& g, int64_t batch_units) {
  int64_t tpw = (batch_units + 2047) / 2048;
  if (tpw < 2) tpw = 2;
  int64_t groups = (g.nkt + tpw - 1) / tpw;
  if (groups > 12) groups = 12;
  if (groups < (g.nkt + 63) / 64) groups = (g.nkt + 63) / 64;
  if (groups > g.nkt) groups = g.nkt;
  if (groups < 1) groups = 1;
  return (int)groups;
}

int64_t batch_units(const Problem* p, int count) {
  int64_t u = 0;
  for (int i = 0; i < count; ++i) {
    const Geometry g = geometry(p[i].n, p[i].k);
    u += ((g.nrt + kWaves - 1) / kWaves) * kWaves * g.nkt;
  }
  return u;
}

size_t partial_floats(const Geometry& g, int groups) {
  if (groups <= 1) return 0;
  const int64_t nrg = (g.nrt + kWaves - 1) / kWaves;
  return (size_t)groups * nrg * kWaves * 32 * 64;
}

}  // namespace

SplitPlan skinny_plan(const Geometry& g) {
  Problem pr{nullptr, g.n, g.k, 1.0f, nullptr, 0, nullptr, 0};
  const int groups = skinny_groups(g, batch_units(&pr, 1));
  return SplitPlan{groups, groups};
}

size_t skinny_workspace_bytes(const Geometry& g) {
  const size_t f = partial_floats(g, skinny_plan(g).groups);
  return f ? kCounterBytes + f * 4 : 0;
}

size_t skinny_batch_workspace_bytes(const Problem* p, int count) {
  size_t worst = 0;
  for (int b0 = 0; b0 < count; b0 += kMaxBatch) {
    const int cnt = count - b0 < kMaxBatch ? count - b0 : kMaxBatch;
    const int64_t units = batch_units(p + b0, cnt);
    size_t f = 0;
    for (int i = b0; i < b0 + cnt; ++i) {
      const Geometry g = geometry(p[i].n, p[i].k);
      if (g.n > 0 && g.k > 0) f += partial_floats(g, skinny_groups(g, units));
    }
    if (f > worst) worst = f;
  }
  return worst ? kCounterBytes + worst * 4 : 0;
}

hipError_t launch_zero_rows(void* y, int64_t m, int64_t n, int64_t ldy, bool y_bf16, hipStream_t s) {
  int64_t total = m * n;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_rows_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, y, m, n, ldy,
                     y_bf16 ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_skinny_batch(const Problem* p, int count, int64_t m, bool y_bf16, void* ws, hipStream_t s) {
  if (m == 0) return hipSuccess;
  for (int b0 = 0; b0 < count; b0 += kMaxBatch) {
    const int cnt = count - b0 < kMaxBatch ? count - b0 : kMaxBatch;
    const int64_t units = batch_units(p + b0, cnt);
    SkinnyBatch b = {};
    int wgs = 0, counters = 0;
    int64_t pbase = 0;
    for (int i = b0; i < b0 + cnt; ++i) {
      const Geometry g = geometry(p[i].n, p[i].k);
      if (g.n == 0) continue;
      if (g.k == 0) {
        hipError_t e = launch_zero_rows(p[i].y, m, g.n, p[i].ldy, y_bf16, s);
        if (e != hipSuccess) return e;
        continue;
      }
      const int groups = skinny_groups(g, units);
      const int64_t nrg = (g.nrt + kWaves - 1) / kWaves;
      const int j = b.count++;
      b.wg_begin[j] = wgs;
      b.packed[j] = static_cast<const uint8_t*>(p[i].packed);
      b.x[j] = p[i].x;
      b.y[j] = p[i].y;
      b.ldx[j] = p[i].ldx;
      b.ldy[j] = p[i].ldy;
      b.n[j] = g.n;
      b.k[j] = g.k;
      b.nkt[j] = (int)g.nkt;
      b.nrt[j] = (int)g.nrt;
      b.groups[j] = groups;
      b.st[j] = p[i].st;
      b.counter_base[j] = counters;
      b.partial_base[j] = pbase;
      wgs += (int)(nrg * groups);
      if (groups > 1) {
        counters += (int)nrg;
        pbase += (int64_t)partial_floats(g, groups);
      }
    }
    if (b.count == 0) continue;
    b.wg_begin[b.count] = wgs;
    unsigned* cnt_ptr = static_cast<unsigned*>(ws);
    float* partial = ws ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kCounterBytes) : nullptr;
    bool kfull = true;
    for (int j = 0; j < b.count; ++j) kfull = kfull && (b.k[j] % kTileK) == 0;
    if (kfull)
      skinny_kernel<true><<<dim3((unsigned)wgs), dim3(256), 0, s>>>(b, m, y_bf16 ? 1 : 0, cnt_ptr, partial);
    else
      skinny_kernel<false><<<dim3((unsigned)wgs), dim3(256), 0, s>>>(b, m, y_bf16 ? 1 : 0, cnt_ptr, partial);
  }
  return hipGetLastError();
}

hipError_t launch_skinny(const void* packed, const Geometry& g, float st, const uint16_t* x, int64_t m, int64_t ldx,
                         void* y, int64_t ldy, bool y_bf16, void* ws, hipStream_t s) {
  Problem pr{packed, g.n, g.k, st, x, ldx, y, ldy};
  return launch_skinny_batch(&pr, 1, m, y_bf16, ws, s);
}

}  // namespace nvfp4
