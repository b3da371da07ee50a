// NVFP4 GEMV: one bf16 activation vector -> fp32 outputs.
//
// y[j] = s_t * sum_k e2m1(c[j][k]) * e4m3(sigma[j][k/16]) * x[k]
//
// The memory-bound decode product (the Ignis README's decode round is weight
// streaming at the card's bandwidth).  Mapping on gfx950:
//  - one wavefront per (64-row tile, 256-k tile), issuing all ten of its
//    16-byte loads per lane at once; the grid holds every tile of the matrix,
//    so the whole weight stream is requested from the start; the loads are
//    non-temporal (each weight is read once: measured, the layer runs ~6 %
//    faster than with ordinary loads);
//  - in the tile layout lane l carries rows l%32 and 32 + l%32 at k half
//    l/32 of every 16-k step, so it needs only 16 of each chunk's 32
//    activations; a workgroup is four wavefronts on four consecutive k tiles
//    of one row tile and stages those 1024 activations in LDS once;
//  - codes become bf16 two per instruction (exact: E2M1 values fit bf16) and
//    meet the bf16 activations in v_dot2_f32_bf16 (products exact in fp32);
//    the E4M3 scale multiplies each 8-weight half-block partial once;
//  - the two k halves meet with one lane-half exchange, the four wavefronts
//    in LDS, and the workgroups of one row tile through the workspace, summed
//    in a fixed order by whichever arrives last (no floating-point atomics).
// Error (first order, u = 2^-24, S = sum|w x|): a half-block partial is a
// chain of 4 dot2, each measured to err by at most 3 u of its inputs'
// magnitudes (12 u S); the scale enters by one fma per half-block, 16 of
// them per lane and tile (16 u S); then the k-half merge (1), the wavefront
// merge (3), one add per workgroup of the row tile (K / 1024) and s_t (1):
// at most (33 + K / 1024) u S, i.e. 65 u S = 3.9e-6 S for K <= 32768, the
// longest k the products accept.
#include <mutex>

#include "device_common.h"
#include "launchers.h"

// Scratch of nvfp4_gemv_batched_noalloc (callers that cannot allocate): the
// split-K counters and partial sums of one batched GEMV call, in a device
// array of the library itself.  Each device holds its own copy for the life of
// the process.  Host code reaches it only through the address that
// hipGetSymbolAddress returns on that device (static_scratch below); the
// array's name is not a device address on the host.
static __device__ __align__(256) uint8_t scratch[nvfp4::kStaticScratchBytes];

namespace nvfp4 {
namespace {

constexpr int kGemvWaves = 4;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int SEL>
__device__ __forceinline__ bf16x2 e2m1x2_bf16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL);
}

__device__ __forceinline__ float dot2(bf16x2 w, uint32_t x, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(w, __builtin_bit_cast(bf16x2, x), acc, false);
}

// 8 weights (code word `q`, 8 nibbles, k ascending) against 4 bf16 x pairs.
__device__ __forceinline__ float dot8(uint32_t q, u32x4 x) {
  float p = dot2(e2m1x2_bf16<0>(q), x[0], 0.0f);
  p = dot2(e2m1x2_bf16<1>(q), x[1], p);
  p = dot2(e2m1x2_bf16<2>(q), x[2], p);
  return dot2(e2m1x2_bf16<3>(q), x[3], p);
}

// Chunk C (k steps 2C, 2C+1) of this lane's two rows.  xa / xb: the lane's
// 8 activations of the two steps; sa / sb: the rows' 16 scale bytes.
template <int C>
__device__ __forceinline__ void chunk(u32x4 q, u32x4 xa, u32x4 xb, u32x4 sa, u32x4 sb, float& acc_a,
                                      float& acc_b) {
  acc_a = fmaf(dot8(q[0], xa), e4m3<(2 * C) % 4>(sa[C / 2]), acc_a);
  acc_b = fmaf(dot8(q[1], xa), e4m3<(2 * C) % 4>(sb[C / 2]), acc_b);
  acc_a = fmaf(dot8(q[2], xb), e4m3<(2 * C + 1) % 4>(sa[C / 2]), acc_a);
  acc_b = fmaf(dot8(q[3], xb), e4m3<(2 * C + 1) % 4>(sb[C / 2]), acc_b);
}

// A batch of up to kMaxBatch GEMVs in one launch; workgroups [wg_begin[p],
// wg_begin[p+1]) belong to problem p.
struct GemvBatch {
  int count;
  int wg_begin[kMaxBatch + 1];
  const uint8_t* packed[kMaxBatch];
  const u32x4* x[kMaxBatch];
  float* y[kMaxBatch];
  int64_t n[kMaxBatch];
  int64_t k[kMaxBatch];
  int nkt[kMaxBatch];
  int groups[kMaxBatch];
  float st[kMaxBatch];
  int counter_base[kMaxBatch];
  int64_t partial_base[kMaxBatch];
};

__global__ __launch_bounds__(256) void gemv_kernel(const GemvBatch b, unsigned* __restrict__ counters,
                                                   float* __restrict__ partial_all) {
  __shared__ u32x4 xs[2 * kGemvWaves * kTileK / 8];  // 4 k tiles of x as bf16 pairs, zero past K (+ an unread half)
  __shared__ float red[kGemvWaves][64];
  int p = 0;
  while (p + 1 < b.count && (int)blockIdx.x >= b.wg_begin[p + 1]) ++p;
  const uint8_t* __restrict__ packed = b.packed[p];
  const u32x4* __restrict__ x16 = b.x[p];
  const int64_t n = b.n[p], k = b.k[p];
  const int nkt = b.nkt[p], groups = b.groups[p];
  const int local = (int)blockIdx.x - b.wg_begin[p];
  const int rt = local / groups;
  const int grp = local % groups;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int kt = grp * kGemvWaves + wave;
  const bool has_tile = kt < nkt;

  // The workgroup's 1024 activations (128 x 16 bytes) load first, so that
  // they reach the LDS (and the barrier) while the weights are still on the
  // way, and each chunk's arithmetic starts as its weights land.  Every
  // thread loads and stores (the last 128 repeat the first 128's loads into
  // an unread half of the buffer), and wavefronts past the last k tile load
  // that tile and drop it: no load or store sits under a branch, so the load
  // stays first and every wait counts exactly the loads it needs.
  const int64_t kk = (int64_t)grp * kGemvWaves * kTileK + 8 * (int64_t)(threadIdx.x & 127);
  const u32x4 xv = x16[(kk < k ? kk : 0) >> 3];
  u32x4 q[8], sa, sb;
  {
    const uint8_t* t = packed + ((size_t)rt * nkt + (has_tile ? kt : nkt - 1)) * kTileBytes;
    sa = load16_stream(t + kScaleOffset + 32 * (lane & 31));
    sb = load16_stream(t + kScaleOffset + 32 * (lane & 31) + 16);
#pragma unroll
    for (int c = 0; c < 8; ++c) q[c] = load16_stream(t + c * 1024 + lane * 16);
  }
  xs[threadIdx.x] = kk < k ? xv : u32x4{0u, 0u, 0u, 0u};
  wait_vmcnt_lgkm0<63>();  // this thread's LDS store is done (the weight loads are not waited for)
  barrier_only();

  float acc_a = 0.0f, acc_b = 0.0f;
  if (has_tile) {
    // Activations of chunk c for this lane: k = 32c + 8h (step 2c) and 32c + 16 + 8h (step 2c+1).
    const u32x4* xt = xs + wave * (kTileK / 8) + (lane >> 5);
#define NVFP4_GEMV_CHUNK(C) chunk<C>(q[C], xt[4 * C], xt[4 * C + 2], sa, sb, acc_a, acc_b);
    NVFP4_GEMV_CHUNK(0) NVFP4_GEMV_CHUNK(1) NVFP4_GEMV_CHUNK(2) NVFP4_GEMV_CHUNK(3)
    NVFP4_GEMV_CHUNK(4) NVFP4_GEMV_CHUNK(5) NVFP4_GEMV_CHUNK(6) NVFP4_GEMV_CHUNK(7)
#undef NVFP4_GEMV_CHUNK
  }
  // Merge the k halves: afterwards lane l < 32 holds row l's two halves in
  // (acc_a, acc_b) and lane l >= 32 holds row l's (row 32 + l%32).
  uint32_t ua = __float_as_uint(acc_a), ub = __float_as_uint(acc_b);
  swap_halves(ua, ub);
  red[wave][lane] = __uint_as_float(ua) + __uint_as_float(ub);
  __syncthreads();
  const int64_t row = (int64_t)rt * kTileRows + lane;
  const float st = b.st[p];
  float* __restrict__ y = b.y[p];
  if (groups == 1) {
    if (wave == 0 && row < n) y[row] = (((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane]) * st;
    return;
  }
  const int64_t np = (int64_t)((n + 63) / 64) * 64;
  float* partial = partial_all + b.partial_base[p];
  if (wave == 0)
    store_coherent(partial + (size_t)grp * np + row, ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane]);
  if (arrive_last(counters + b.counter_base[p] + rt, (unsigned)groups)) {
    if (wave == 0 && row < n) y[row] = sum_coherent(partial + row, (size_t)np, groups) * st;
  }
}

// ---- one or two activation rows (m <= kGemvRowsMax) through the GEMV --------
// The same tile mapping and reductions as above, for M activation rows: each
// weight pair is converted once and meets every row's activations in that
// row's own dot2 chain, in the order the single-row kernel uses, so row i's
// outputs are bit-identical to a GEMV of row i.  The VALU work grows by one
// dot2 per weight pair and row: at two rows it still hides under the weight
// stream (the 27B-class layer: 41 us, against 53 us on the matrix-core
// path); at three it no longer does (55 us, the same as that path).
struct GemvRowsBatch {
  int count;
  int y_bf16;
  int wg_begin[kMaxBatch + 1];
  const uint8_t* packed[kMaxBatch];
  const uint16_t* x[kMaxBatch];
  void* y[kMaxBatch];
  int64_t ldx[kMaxBatch];
  int64_t ldy[kMaxBatch];
  int64_t n[kMaxBatch];
  int64_t k[kMaxBatch];
  int nkt[kMaxBatch];
  int groups[kMaxBatch];
  float st[kMaxBatch];
  int counter_base[kMaxBatch];
  int64_t partial_base[kMaxBatch];
};

template <int C, int M>
__device__ __forceinline__ void chunk_rows(u32x4 q, const u32x4 (&xs)[2][kGemvWaves * kTileK / 8], int xi, u32x4 sa,
                                           u32x4 sb, float (&acc_a)[M], float (&acc_b)[M]) {
  bf16x2 w[4][4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    w[d][0] = e2m1x2_bf16<0>(q[d]);
    w[d][1] = e2m1x2_bf16<1>(q[d]);
    w[d][2] = e2m1x2_bf16<2>(q[d]);
    w[d][3] = e2m1x2_bf16<3>(q[d]);
  }
  const float s_a0 = e4m3<(2 * C) % 4>(sa[C / 2]), s_b0 = e4m3<(2 * C) % 4>(sb[C / 2]);
  const float s_a1 = e4m3<(2 * C + 1) % 4>(sa[C / 2]), s_b1 = e4m3<(2 * C + 1) % 4>(sb[C / 2]);
#pragma unroll
  for (int r = 0; r < M; ++r) {
    const u32x4 xa = xs[r][xi + 4 * C], xb = xs[r][xi + 4 * C + 2];
    auto d8 = [&](int d, u32x4 x) __attribute__((always_inline)) {
      float p = dot2(w[d][0], x[0], 0.0f);
      p = dot2(w[d][1], x[1], p);
      p = dot2(w[d][2], x[2], p);
      return dot2(w[d][3], x[3], p);
    };
    acc_a[r] = fmaf(d8(0, xa), s_a0, acc_a[r]);
    acc_b[r] = fmaf(d8(1, xa), s_b0, acc_b[r]);
    acc_a[r] = fmaf(d8(2, xb), s_a1, acc_a[r]);
    acc_b[r] = fmaf(d8(3, xb), s_b1, acc_b[r]);
  }
}

template <int M>
__global__ __launch_bounds__(256) void gemv_rows_kernel(const GemvRowsBatch b, unsigned* __restrict__ counters,
                                                        float* __restrict__ partial_all) {
  // M rows' 4 k tiles of x, zero past K (and, for M = 1, an unread half)
  __shared__ u32x4 xs[2][kGemvWaves * kTileK / 8];
  __shared__ float red[M][kGemvWaves][64];
  int p = 0;
  while (p + 1 < b.count && (int)blockIdx.x >= b.wg_begin[p + 1]) ++p;
  const uint8_t* __restrict__ packed = b.packed[p];
  const uint16_t* __restrict__ x = b.x[p];
  const int64_t n = b.n[p], k = b.k[p], ldx = b.ldx[p];
  const int nkt = b.nkt[p], groups = b.groups[p];
  const int local = (int)blockIdx.x - b.wg_begin[p];
  const int rt = local / groups;
  const int grp = local % groups;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int kt = grp * kGemvWaves + wave;
  const bool has_tile = kt < nkt;

  // As in gemv_kernel: the activations load first and no load or store sits
  // under a branch.  Thread t loads chunk t % 128 of row (t / 128) % M.
  const int xr = M == 1 ? 0 : (int)(threadIdx.x >> 7), xc = (int)threadIdx.x & 127;
  const int64_t kk = (int64_t)grp * kGemvWaves * kTileK + 8 * (int64_t)xc;
  const u32x4 xv = *reinterpret_cast<const u32x4*>(x + xr * ldx + (kk < k ? kk : 0));
  u32x4 q[8], sa, sb;
  {
    const uint8_t* t = packed + ((size_t)rt * nkt + (has_tile ? kt : nkt - 1)) * kTileBytes;
    sa = load16_stream(t + kScaleOffset + 32 * (lane & 31));
    sb = load16_stream(t + kScaleOffset + 32 * (lane & 31) + 16);
#pragma unroll
    for (int c = 0; c < 8; ++c) q[c] = load16_stream(t + c * 1024 + lane * 16);
  }
  xs[threadIdx.x >> 7][xc] = kk < k ? xv : u32x4{0u, 0u, 0u, 0u};
  wait_vmcnt_lgkm0<63>();  // this thread's LDS store is done (the weight loads are not waited for)
  barrier_only();

  float acc_a[M], acc_b[M];
#pragma unroll
  for (int r = 0; r < M; ++r) acc_a[r] = acc_b[r] = 0.0f;
  if (has_tile) {
    const int xi = wave * (kTileK / 8) + (lane >> 5);
#define NVFP4_GEMV_ROWS_CHUNK(C) chunk_rows<C, M>(q[C], xs, xi, sa, sb, acc_a, acc_b);
    NVFP4_GEMV_ROWS_CHUNK(0) NVFP4_GEMV_ROWS_CHUNK(1) NVFP4_GEMV_ROWS_CHUNK(2) NVFP4_GEMV_ROWS_CHUNK(3)
    NVFP4_GEMV_ROWS_CHUNK(4) NVFP4_GEMV_ROWS_CHUNK(5) NVFP4_GEMV_ROWS_CHUNK(6) NVFP4_GEMV_ROWS_CHUNK(7)
#undef NVFP4_GEMV_ROWS_CHUNK
  }
#pragma unroll
  for (int r = 0; r < M; ++r) {
    uint32_t ua = __float_as_uint(acc_a[r]), ub = __float_as_uint(acc_b[r]);
    swap_halves(ua, ub);
    red[r][wave][lane] = __uint_as_float(ua) + __uint_as_float(ub);
  }
  __syncthreads();
  const int64_t row = (int64_t)rt * kTileRows + lane;
  const float st = b.st[p];
  void* __restrict__ y = b.y[p];
  const int64_t ldy = b.ldy[p];
  auto put = [&](int r, float v) __attribute__((always_inline)) {
    if (b.y_bf16) static_cast<uint16_t*>(y)[r * ldy + row] = to_bf16(v);
    else static_cast<float*>(y)[r * ldy + row] = v;
  };
  if (groups == 1) {
    if (wave == 0 && row < n)
#pragma unroll
      for (int r = 0; r < M; ++r) put(r, (((red[r][0][lane] + red[r][1][lane]) + red[r][2][lane]) + red[r][3][lane]) * st);
    return;
  }
  // Partials: [group][row][np], so row r's groups are M * np apart.
  const int64_t np = (int64_t)((n + 63) / 64) * 64;
  float* partial = partial_all + b.partial_base[p];
  if (wave == 0)
#pragma unroll
    for (int r = 0; r < M; ++r)
      store_coherent(partial + ((size_t)grp * M + r) * np + row,
                     ((red[r][0][lane] + red[r][1][lane]) + red[r][2][lane]) + red[r][3][lane]);
  if (arrive_last(counters + b.counter_base[p] + rt, (unsigned)groups)) {
    if (wave == 0 && row < n)
#pragma unroll
      for (int r = 0; r < M; ++r) put(r, sum_coherent(partial + (size_t)r * np + row, (size_t)M * np, groups) * st);
  }
}

__global__ void zero_f32_kernel(float* __restrict__ y, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = 0.0f;
}

}  // namespace

// One wavefront per 256-k tile, four per workgroup: ceil(K / 1024) workgroups per row tile.
SplitPlan gemv_plan(const Geometry& g) {
  int64_t groups = (g.nkt + kGemvWaves - 1) / kGemvWaves;
  if (groups < 1) groups = 1;
  return SplitPlan{(int)groups, (int)groups * kGemvWaves};
}

size_t gemv_workspace_bytes(const Geometry& g) {
  SplitPlan p = gemv_plan(g);
  if (p.groups <= 1) return 0;
  return kCounterBytes + (size_t)p.groups * (size_t)g.nrt * 64 * 4;
}

size_t gemv_batch_workspace_bytes(const Problem* p, int count) {
  // Each launch of up to kMaxBatch problems lays out its partials from offset 0.
  size_t worst = 0;
  for (int b0 = 0; b0 < count; b0 += kMaxBatch) {
    size_t part = 0;
    for (int i = b0; i < count && i < b0 + kMaxBatch; ++i) {
      const Geometry g = geometry(p[i].n, p[i].k);
      const SplitPlan pl = gemv_plan(g);
      if (pl.groups > 1 && g.n > 0 && g.k > 0) part += (size_t)pl.groups * (size_t)g.nrt * 64 * 4;
    }
    if (part > worst) worst = part;
  }
  return worst ? kCounterBytes + worst : 0;
}

hipError_t launch_gemv_batch(const Problem* p, int count, void* ws, hipStream_t s) {
  for (int b0 = 0; b0 < count; b0 += kMaxBatch) {
    GemvBatch b = {};
    int wgs = 0, counters = 0;
    int64_t pbase = 0;
    for (int i = b0; i < count && i < b0 + kMaxBatch; ++i) {
      const Geometry g = geometry(p[i].n, p[i].k);
      if (g.n == 0) continue;
      if (g.k == 0) {
        hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)((g.n + 255) / 256)), dim3(256), 0, s,
                           static_cast<float*>(p[i].y), g.n);
        continue;
      }
      const SplitPlan pl = gemv_plan(g);
      const int j = b.count++;
      b.wg_begin[j] = wgs;
      b.packed[j] = static_cast<const uint8_t*>(p[i].packed);
      b.x[j] = reinterpret_cast<const u32x4*>(p[i].x);
      b.y[j] = static_cast<float*>(p[i].y);
      b.n[j] = g.n;
      b.k[j] = g.k;
      b.nkt[j] = (int)g.nkt;
      b.groups[j] = pl.groups;
      b.st[j] = p[i].st;
      b.counter_base[j] = counters;
      b.partial_base[j] = pbase;
      wgs += (int)(g.nrt * pl.groups);
      if (pl.groups > 1) {
        counters += (int)g.nrt;
        pbase += (int64_t)pl.groups * g.nrt * 64;
      }
    }
    if (b.count == 0) continue;
    b.wg_begin[b.count] = wgs;
    unsigned* cnt = static_cast<unsigned*>(ws);
    float* partial = ws ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kCounterBytes) : nullptr;
    hipLaunchKernelGGL(gemv_kernel, dim3((unsigned)wgs), dim3(256), 0, s, b, cnt, partial);
  }
  return hipGetLastError();
}

size_t gemv_rows_batch_workspace_bytes(const Problem* p, int count, int64_t m) {
  return gemv_batch_workspace_bytes(p, count) == 0 ? 0 : kCounterBytes + (gemv_batch_workspace_bytes(p, count) - kCounterBytes) * (size_t)m;
}

hipError_t launch_gemv_rows_batch(const Problem* p, int count, int64_t m, bool y_bf16, void* ws, hipStream_t s) {
  for (int b0 = 0; b0 < count; b0 += kMaxBatch) {
    GemvRowsBatch b = {};
    b.y_bf16 = y_bf16 ? 1 : 0;
    int wgs = 0, counters = 0;
    int64_t pbase = 0;
    for (int i = b0; i < count && i < b0 + kMaxBatch; ++i) {
      const Geometry g = geometry(p[i].n, p[i].k);
      if (g.n == 0) continue;
      if (g.k == 0) {
        hipError_t e = launch_zero_rows(p[i].y, m, g.n, p[i].ldy, y_bf16, s);
        if (e != hipSuccess) return e;
        continue;
      }
      const SplitPlan pl = gemv_plan(g);
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
      b.groups[j] = pl.groups;
      b.st[j] = p[i].st;
      b.counter_base[j] = counters;
      b.partial_base[j] = pbase;
      wgs += (int)(g.nrt * pl.groups);
      if (pl.groups > 1) {
        counters += (int)g.nrt;
        pbase += (int64_t)pl.groups * g.nrt * 64 * m;
      }
    }
    if (b.count == 0) continue;
    b.wg_begin[b.count] = wgs;
    unsigned* cnt = static_cast<unsigned*>(ws);
    float* partial = ws ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kCounterBytes) : nullptr;
    static_assert(kGemvRowsMax == 2, "row counts instantiated below");
    if (m == 1)
      hipLaunchKernelGGL(gemv_rows_kernel<1>, dim3((unsigned)wgs), dim3(256), 0, s, b, cnt, partial);
    else
      hipLaunchKernelGGL(gemv_rows_kernel<2>, dim3((unsigned)wgs), dim3(256), 0, s, b, cnt, partial);
  }
  return hipGetLastError();
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];
}  // namespace

hipError_t static_scratch(hipStream_t s, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    // The counters must start at zero (every call leaves them so); the array
    // is zero when the code object loads, and this fill, ordered before the
    // first call's launch, makes that explicit.
    e = launch_fill_zero(p, kCounterBytes, s);
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

hipError_t launch_gemv(const void* packed, const Geometry& g, float st, const uint16_t* x, float* y, void* ws,
                       hipStream_t s) {
  Problem pr{packed, g.n, g.k, st, x, 0, y, 0};
  return launch_gemv_batch(&pr, 1, ws, s);
}

}  // namespace nvfp4
