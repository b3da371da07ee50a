// a9: NVFP4 x bf16 GEMM for many activation rows (prompt prefill).
//
// y[i][j] = s_t * sum_k W[j][k] * x[i][k]
//
// Compute-bound.  Every weight is dequantised exactly to bf16 (E2M1 x E4M3
// in fp32 has at most 6 significant bits, so the fp32 product is exact and
// its upper half is its bf16) and bf16 MFMA (v_mfma_f32_32x32x16_bf16) forms
// the products with fp32 accumulation; s_t is applied after accumulation.
//
// Workgroup tile: BM = 32*JT activation rows x 256 weight rows.  Each of the
// four wavefronts owns one 64-row packed weight tile and dequantises it
// straight into MFMA A operands: the packed layout already puts a lane's
// eight codes of a k step where the A operand wants them, so weights never
// pass through LDS and no weight is dequantised twice in a workgroup.  The
// activation tile (BM rows x 64 k per iteration) is staged through LDS,
// double buffered, its 16-byte chunks XOR-swizzled by row so that the B
// operand reads are bank-conflict free; every wavefront reads all of it.
// Weights stream from memory four iterations ahead of use, activations two.
//
// Work decomposition (stream-K): the (output tile, 64-k iteration) pairs of
// all problems of a launch are laid end to end and cut into one equal share
// per persistent workgroup, so no compute unit idles at the end of a launch
// whatever the tile count -- the pages' split-K prefill, balanced exactly.
// A tile cut between workgroups is finished by whichever contributor arrives
// last: it adds all contributions in k order (deterministic, independent of
// arrival order) and writes the output.  No workgroup ever waits for
// another.  Consecutive shares run on the same XCD, so an XCD's workgroups
// walk neighbouring tiles and share their activation rows in its L2.
#include "skinny_core.h"
#include "launchers.h"

namespace nvfp4 {
namespace {

constexpr int kBN = 256;        // weight rows per workgroup tile: four packed row tiles
constexpr int kBK = 64;         // k per iteration
constexpr int kPreWgs = 256;    // persistent workgroups (the compute units of an MI355X)
constexpr int kMinShare = 8;    // iterations per workgroup below which fewer workgroups are used
constexpr int kMaxPre = 8;      // problems per launch

struct PrefillBatch {
  int count;
  int mtiles;                       // activation-row tiles
  int wgs;                          // workgroups (shares)
  int y_bf16;
  int64_t m;                        // activation rows
  int64_t total;                    // iterations over all problems
  int64_t iter_begin[kMaxPre + 1];  // first global iteration of each problem
  int tile_base[kMaxPre];           // first global tile (counter slot) of each problem
  int iters[kMaxPre];               // iterations per tile
  int nkt[kMaxPre];
  int nrt[kMaxPre];
  const uint8_t* packed[kMaxPre];
  const uint16_t* x[kMaxPre];
  void* y[kMaxPre];
  int64_t n[kMaxPre], k[kMaxPre], ldx[kMaxPre], ldy[kMaxPre];
  float st[kMaxPre];
};

// Share w covers global iterations [share_begin(w), share_begin(w + 1)).
__device__ __forceinline__ int64_t share_begin(int w, int64_t total, int wgs) { return ((int64_t)w * total) / wgs; }
// The share holding global iteration g.
__device__ __forceinline__ int owner_of(int64_t g, int64_t total, int wgs) { return (int)(((g + 1) * wgs - 1) / total); }

// LDS byte offset of 16-byte chunk c (0..7) of activation row r (128 bytes a row).
__device__ __forceinline__ int swz(int r, int c) { return r * (kBK * 2) + ((c ^ (r & 7)) << 4); }

// Weights of one iteration for one lane: two 1 KB chunks of the packed tile
// (k steps 0-1 and 2-3 of the iteration) and the scale dword of rows r and
// 32 + r that covers the iteration's four 16-k blocks.
struct WStage {
  u32x4 q0, q1;
  uint32_t sa, sb;
};

// Partial sums of a cut tile: per workgroup two slots (its first and its last
// segment), each the workgroup tile in accumulator order, laid out so that
// one wavefront store writes 1 KB contiguously: float4 index u of lane l of
// wavefront v is at ((v * 8 * JT + u) * 64 + l) * 4 floats.
template <int JT>
constexpr size_t part_floats() { return (size_t)4 * 8 * JT * 64 * 4; }

// Four 16-byte stores 1 KB apart, through to memory (not held in this XCD's
// L2); the trailing nops cover the store-data read of the last store.
__device__ __forceinline__ void store4x4_coherent(float* p, f32x4 a, f32x4 b, f32x4 c, f32x4 d) {
  asm volatile(
      "global_store_dwordx4 %0, %1, off sc1\n"
      "global_store_dwordx4 %0, %2, off offset:1024 sc1\n"
      "global_store_dwordx4 %0, %3, off offset:2048 sc1\n"
      "global_store_dwordx4 %0, %4, off offset:3072 sc1\n"
      "s_nop 1"
      :
      : "v"(p), "v"(a), "v"(b), "v"(c), "v"(d)
      : "memory");
}

// Sixteen 16-byte loads 1 KB apart that bypass the non-coherent caches; the
// wait sits in the same statement, so none is in flight when it ends.
__device__ __forceinline__ void load16x4_strided_coherent(const float* p, f32x4 (&v)[16]) {
  const char* c0 = reinterpret_cast<const char*>(p);
  const char* c1 = c0 + 4096;
  const char* c2 = c0 + 8192;
  const char* c3 = c0 + 12288;
  asm volatile(
      "global_load_dwordx4 %0, %16, off sc1\n"
      "global_load_dwordx4 %1, %16, off offset:1024 sc1\n"
      "global_load_dwordx4 %2, %16, off offset:2048 sc1\n"
      "global_load_dwordx4 %3, %16, off offset:3072 sc1\n"
      "global_load_dwordx4 %4, %17, off sc1\n"
      "global_load_dwordx4 %5, %17, off offset:1024 sc1\n"
      "global_load_dwordx4 %6, %17, off offset:2048 sc1\n"
      "global_load_dwordx4 %7, %17, off offset:3072 sc1\n"
      "global_load_dwordx4 %8, %18, off sc1\n"
      "global_load_dwordx4 %9, %18, off offset:1024 sc1\n"
      "global_load_dwordx4 %10, %18, off offset:2048 sc1\n"
      "global_load_dwordx4 %11, %18, off offset:3072 sc1\n"
      "global_load_dwordx4 %12, %19, off sc1\n"
      "global_load_dwordx4 %13, %19, off offset:1024 sc1\n"
      "global_load_dwordx4 %14, %19, off offset:2048 sc1\n"
      "global_load_dwordx4 %15, %19, off offset:3072 sc1\n"
      "s_waitcnt vmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7]),
        "=&v"(v[8]), "=&v"(v[9]), "=&v"(v[10]), "=&v"(v[11]), "=&v"(v[12]), "=&v"(v[13]), "=&v"(v[14]),
        "=&v"(v[15])
      : "v"(c0), "v"(c1), "v"(c2), "v"(c3)
      : "memory");
}

// One 16-k step KS (0..3) of an iteration: A operands for weight rows r and
// 32 + r from the resident codes, B operands for the JT activation tiles
// from LDS, 2 * JT MFMAs.
template <int KS, int JT>
__device__ __forceinline__ void kstep(const uint8_t* xl, int lane, const WStage& w, f32x16 (&acc)[2][JT]) {
  constexpr int J = KS & 1;
  const u32x4 q = KS < 2 ? w.q0 : w.q1;
  const bf16x8 a0 = dequant8(q[2 * J], e4m3<KS>(w.sa));
  const bf16x8 a1 = dequant8(q[2 * J + 1], e4m3<KS>(w.sb));
  const int chunk = 2 * KS + (lane >> 5);
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) {
    const bf16x8 bx = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xl + swz(32 * jt + (lane & 31), chunk)));
    acc[0][jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bx, acc[0][jt], 0, 0, 0);
    acc[1][jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bx, acc[1][jt], 0, 0, 0);
  }
}

template <int JT>
__device__ __forceinline__ f32x4 acc4(const f32x16 (&acc)[2][JT], int u) {
  // float4 u of a lane: accumulator tile t = u / 4 (i = t / JT, jt = t % JT), elements 4 * (u % 4) ..
  const f32x16& a = acc[(u >> 2) / JT][(u >> 2) % JT];
  const int e = 4 * (u & 3);
  return f32x4{a[e], a[e + 1], a[e + 2], a[e + 3]};
}

template <int JT>
__global__ __launch_bounds__(256, 1) void prefill_kernel(const PrefillBatch b, unsigned* __restrict__ counters,
                                                         float* __restrict__ partials) {
  constexpr int kBM = 32 * JT;
  constexpr int kXBuf = kBM * kBK * 2;  // bytes of one activation buffer
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kXBuf];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;

  // Share of this workgroup.  Dispatch places workgroup b on XCD b % 8; give
  // each XCD a contiguous run of shares.
  int w = (int)blockIdx.x;
  if ((b.wgs & 7) == 0) w = (int)(blockIdx.x & 7) * (b.wgs >> 3) + (int)(blockIdx.x >> 3);
  const int64_t g_begin = share_begin(w, b.total, b.wgs);
  const int64_t g_end = share_begin(w + 1, b.total, b.wgs);

  const int xr0 = tid >> 3, xc = tid & 7;  // activation loader: rows xr0 + 32j, 16-byte chunk xc

  for (int64_t g = g_begin; g < g_end;) {
    // ---- locate the segment: problem p, tile (mt, nt), iterations [ib, ie)
    int p = 0;
    while (p + 1 < b.count && g >= b.iter_begin[p + 1]) ++p;
    const int iters = b.iters[p];
    const int64_t gl = g - b.iter_begin[p];
    const int tile = (int)(gl / iters);
    const int ib = (int)(gl - (int64_t)tile * iters);
    const int64_t tile_g0 = b.iter_begin[p] + (int64_t)tile * iters;
    const int ie = (int)(g_end - tile_g0 < iters ? g_end - tile_g0 : iters);
    const int mt = tile % b.mtiles, nt = tile / b.mtiles;
    const int64_t m0 = (int64_t)mt * kBM;
    const int64_t kdim = b.k[p];
    const int nkt = b.nkt[p];

    // Activation sources (rows past m re-read row m-1; their outputs are not written).
    const uint16_t* xsrc[JT];
#pragma unroll
    for (int j = 0; j < JT; ++j) {
      int64_t row = m0 + xr0 + 32 * j;
      row = row < b.m ? row : b.m - 1;
      xsrc[j] = b.x[p] + row * b.ldx[p] + 8 * xc;
    }
    // Weight source: this wavefront's packed row tile (clamped; rows past n are not written).
    int rt = nt * 4 + wave;
    rt = rt < b.nrt[p] ? rt : b.nrt[p] - 1;
    const uint8_t* wt = b.packed[p] + (size_t)rt * nkt * kTileBytes;
    const uint8_t* wcode = wt + lane * 16;
    const uint8_t* wscale = wt + kScaleOffset + 32 * (lane & 31);

    auto load_w = [&](int it, WStage& s) {
      const size_t t = (size_t)(it >> 2) * kTileBytes;
      const int sub = it & 3;
      s.q0 = load16(wcode + t + (2 * sub) * 1024);
      s.q1 = load16(wcode + t + (2 * sub + 1) * 1024);
      s.sa = *reinterpret_cast<const uint32_t*>(wscale + t + 4 * sub);
      s.sb = *reinterpret_cast<const uint32_t*>(wscale + t + 16 + 4 * sub);
    };
    auto load_x = [&](int it, u32x4 (&v)[JT]) {
      const bool in = (int64_t)it * kBK + 8 * xc < kdim;
#pragma unroll
      for (int j = 0; j < JT; ++j) v[j] = in ? load16(xsrc[j] + (int64_t)it * kBK) : u32x4{0u, 0u, 0u, 0u};
    };
    auto store_x = [&](int buf, const u32x4 (&v)[JT]) {
      uint8_t* xl = lds + buf * kXBuf;
#pragma unroll
      for (int j = 0; j < JT; ++j) *reinterpret_cast<u32x4*>(xl + swz(xr0 + 32 * j, xc)) = v[j];
    };

    f32x16 acc[2][JT];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < JT; ++j) acc[i][j] = f32x16{};

    // ---- pipeline.  Loads past the segment re-read its last iteration, so
    // each executed step issues the same loads in the same order.
    const int last = ie - 1;
    auto clampi = [&](int it) { return it < last ? it : last; };
    WStage w0, w1, w2, w3;
    u32x4 xa[JT], xb[JT];
    load_w(ib, w0);
    load_w(clampi(ib + 1), w1);
    load_w(clampi(ib + 2), w2);
    load_w(clampi(ib + 3), w3);
    load_x(ib, xa);
    load_x(clampi(ib + 1), xb);
    store_x(0, xa);
    __syncthreads();
    // Step S of a group of four (iteration it = i + S, LDS buffer S & 1):
    // issue the activation loads of it + 2, multiply it, stage it + 1's
    // activations into the other buffer, issue the weight loads of it + 4.
#define NVFP4_PREFILL_STEP(S, XCUR, XNEXT, WCUR)                        \
  if (i + (S) < ie) {                                                   \
    const int it = i + (S);                                             \
    load_x(clampi(it + 2), XCUR);                                       \
    {                                                                   \
      const uint8_t* xl = lds + ((S) & 1) * kXBuf;                      \
      kstep<0, JT>(xl, lane, WCUR, acc);                                \
      kstep<1, JT>(xl, lane, WCUR, acc);                                \
      kstep<2, JT>(xl, lane, WCUR, acc);                                \
      kstep<3, JT>(xl, lane, WCUR, acc);                                \
    }                                                                   \
    if (it + 1 < ie) store_x(((S) + 1) & 1, XNEXT);                     \
    load_w(clampi(it + 4), WCUR);                                       \
    __syncthreads();                                                    \
  }
    for (int i = ib; i < ie; i += 4) {
      NVFP4_PREFILL_STEP(0, xa, xb, w0)
      NVFP4_PREFILL_STEP(1, xb, xa, w1)
      NVFP4_PREFILL_STEP(2, xa, xb, w2)
      NVFP4_PREFILL_STEP(3, xb, xa, w3)
    }
#undef NVFP4_PREFILL_STEP

    // ---- output ------------------------------------------------------------
    // Accumulator element e of tile (i, jt) of this lane: weight row
    // 64 * wave + 32 * i + 8 * (e / 4) + 4 * (lane / 32) + e % 4 of the tile,
    // activation row 32 * jt + lane % 32.
    const float st = b.st[p];
    void* const y = b.y[p];
    const int64_t ldy = b.ldy[p], n = b.n[p];
    const bool vec = (ldy & 3) == 0;
    const int64_t col0 = (int64_t)nt * kBN + 64 * wave + 4 * (lane >> 5);
    auto write_y = [&](int u, f32x4 v) {
      const int t = u >> 2, i = t / JT, jt = t % JT;
      const int64_t row = m0 + 32 * jt + (lane & 31);
      if (row >= b.m) return;
      const int64_t col = col0 + 32 * i + 8 * (u & 3);
      if (col >= n) return;
      const float v0 = v[0] * st, v1 = v[1] * st, v2 = v[2] * st, v3 = v[3] * st;
      if (b.y_bf16) {
        uint16_t* yr = static_cast<uint16_t*>(y) + row * ldy + col;
        if (vec && col + 4 <= n) {
          *reinterpret_cast<uint2*>(yr) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
        } else {
          yr[0] = to_bf16(v0);
          if (col + 1 < n) yr[1] = to_bf16(v1);
          if (col + 2 < n) yr[2] = to_bf16(v2);
          if (col + 3 < n) yr[3] = to_bf16(v3);
        }
      } else {
        float* yr = static_cast<float*>(y) + row * ldy + col;
        if (vec && col + 4 <= n) {
          *reinterpret_cast<f32x4*>(yr) = f32x4{v0, v1, v2, v3};
        } else {
          yr[0] = v0;
          if (col + 1 < n) yr[1] = v1;
          if (col + 2 < n) yr[2] = v2;
          if (col + 3 < n) yr[3] = v3;
        }
      }
    };

    if (ib == 0 && ie == iters) {
#pragma unroll
      for (int u = 0; u < 8 * JT; ++u) write_y(u, acc4<JT>(acc, u));
    } else {
      // Cut tile: publish this segment's sums, then the last contributor to
      // arrive adds all contributions in k order.
      const int slot = g_begin >= tile_g0 ? 0 : 1;  // this workgroup's first or last segment
      const size_t lane_off = ((size_t)wave * 8 * JT * 64 + lane) * 4;
      float* mine = partials + ((size_t)w * 2 + slot) * part_floats<JT>() + lane_off;
#pragma unroll
      for (int u = 0; u < 8 * JT; u += 4)
        store4x4_coherent(mine + (size_t)u * 256, acc4<JT>(acc, u), acc4<JT>(acc, u + 1), acc4<JT>(acc, u + 2),
                          acc4<JT>(acc, u + 3));
      const int c_first = owner_of(tile_g0, b.total, b.wgs);
      const int c_last = owner_of(tile_g0 + iters - 1, b.total, b.wgs);
      if (arrive_last(counters + b.tile_base[p] + tile, (unsigned)(c_last - c_first + 1))) {
#pragma unroll
        for (int q = 0; q < JT / 2; ++q) {
          // float4s 16q .. 16q + 15 of this lane, summed over the contributors in order
          f32x4 s[16];
          for (int c = c_first; c <= c_last; ++c) {
            // Every contribution, this workgroup's own included, is read back
            // from its slot: the accumulators need not stay live here.
            f32x4 v[16];
            const int cslot = share_begin(c, b.total, b.wgs) >= tile_g0 ? 0 : 1;
            load16x4_strided_coherent(
                partials + ((size_t)c * 2 + cslot) * part_floats<JT>() + lane_off + (size_t)(16 * q) * 256, v);
            if (c == c_first) {
#pragma unroll
              for (int u = 0; u < 16; ++u) s[u] = v[u];
            } else {
#pragma unroll
              for (int u = 0; u < 16; ++u) s[u] += v[u];
            }
          }
#pragma unroll
          for (int u = 0; u < 16; ++u) write_y(16 * q + u, s[u]);
        }
      }
    }
    g = tile_g0 + ie;
  }
}

struct Plan {
  int jt;         // activation-row tiles of 32 per workgroup tile
  int64_t mrows;  // activation rows per launch (all of them unless the counter slots run out)
};

Plan prefill_plan(const Problem* p, int count, int64_t m) {
  Plan pl;
  pl.jt = m > 128 ? 8 : (m > 64 ? 4 : 2);
  const int64_t bm = 32 * pl.jt;
  int64_t ntiles = 0;
  for (int i = 0; i < count; ++i) ntiles += (((p[i].n + 63) / 64) + 3) / 4;
  // One counter per output tile of a launch: cut m so that a launch's tiles fit.
  const int64_t max_mt = ntiles > 0 ? kCounterSlots / ntiles : 1;
  const int64_t mt = (m + bm - 1) / bm;
  pl.mrows = (mt <= max_mt ? mt : max_mt) * bm;
  return pl;
}

size_t part_bytes(int jt) {
  return (jt == 8 ? part_floats<8>() : jt == 4 ? part_floats<4>() : part_floats<2>()) * sizeof(float);
}

}  // namespace

size_t prefill_batch_workspace_bytes(const Problem* p, int count, int64_t m) {
  if (m <= 0 || count <= 0) return 0;
  size_t need = 0;
  for (int c0 = 0; c0 < count; c0 += kMaxPre) {
    const int cn = count - c0 < kMaxPre ? count - c0 : kMaxPre;
    const Plan pl = prefill_plan(p + c0, cn, m);
    const size_t b = kCounterBytes + (size_t)2 * kPreWgs * part_bytes(pl.jt);
    if (b > need) need = b;
  }
  return need;
}

size_t prefill_workspace_bytes(int64_t m, const Geometry& g) {
  Problem pr{nullptr, g.n, g.k, 1.0f, nullptr, g.k, nullptr, g.n};
  return prefill_batch_workspace_bytes(&pr, 1, m);
}

hipError_t launch_zero_rows(void* y, int64_t m, int64_t n, int64_t ldy, bool y_bf16, hipStream_t s);

hipError_t launch_prefill_batch(const Problem* p, int count, int64_t m, bool y_bf16, void* ws, hipStream_t s) {
  if (m <= 0) return hipSuccess;
  const size_t esize = y_bf16 ? 2 : 4;
  // k == 0: the product is empty, the outputs are zero.
  for (int i = 0; i < count; ++i)
    if (p[i].n > 0 && p[i].k == 0) {
      hipError_t e = launch_zero_rows(p[i].y, m, p[i].n, p[i].ldy, y_bf16, s);
      if (e != hipSuccess) return e;
    }
  unsigned* counters = static_cast<unsigned*>(ws);
  float* partials = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kCounterBytes);
  for (int c0 = 0; c0 < count; c0 += kMaxPre) {
    const int cn = count - c0 < kMaxPre ? count - c0 : kMaxPre;
    // The problems of this launch that have work.
    Problem q[kMaxPre];
    int nq = 0;
    for (int i = c0; i < c0 + cn; ++i)
      if (p[i].n > 0 && p[i].k > 0) q[nq++] = p[i];
    if (nq == 0) continue;
    const Plan pl = prefill_plan(q, nq, m);
    const int64_t bm = 32 * pl.jt;
    for (int64_t r0 = 0; r0 < m; r0 += pl.mrows) {
      const int64_t mr = m - r0 < pl.mrows ? m - r0 : pl.mrows;
      PrefillBatch b{};
      b.count = nq;
      b.mtiles = (int)((mr + bm - 1) / bm);
      b.y_bf16 = y_bf16 ? 1 : 0;
      b.m = mr;
      int64_t it = 0;
      int tiles = 0;
      for (int j = 0; j < nq; ++j) {
        const Geometry g = geometry(q[j].n, q[j].k);
        const int ntn = (int)((g.nrt + 3) / 4);
        b.iter_begin[j] = it;
        b.tile_base[j] = tiles;
        b.iters[j] = (int)((q[j].k + kBK - 1) / kBK);
        b.nkt[j] = (int)g.nkt;
        b.nrt[j] = (int)g.nrt;
        b.packed[j] = static_cast<const uint8_t*>(q[j].packed);
        b.x[j] = q[j].x + r0 * q[j].ldx;
        b.y[j] = static_cast<uint8_t*>(q[j].y) + (size_t)r0 * q[j].ldy * esize;
        b.n[j] = q[j].n;
        b.k[j] = q[j].k;
        b.ldx[j] = q[j].ldx;
        b.ldy[j] = q[j].ldy;
        b.st[j] = q[j].st;
        tiles += ntn * b.mtiles;
        it += (int64_t)ntn * b.mtiles * b.iters[j];
      }
      b.iter_begin[nq] = it;
      b.total = it;
      int64_t wgs = it / kMinShare;
      wgs = wgs < 1 ? 1 : (wgs > kPreWgs ? kPreWgs : wgs);
      b.wgs = (int)wgs;
      switch (pl.jt) {
        case 8: hipLaunchKernelGGL(prefill_kernel<8>, dim3((unsigned)wgs), dim3(256), 0, s, b, counters, partials); break;
        case 4: hipLaunchKernelGGL(prefill_kernel<4>, dim3((unsigned)wgs), dim3(256), 0, s, b, counters, partials); break;
        default: hipLaunchKernelGGL(prefill_kernel<2>, dim3((unsigned)wgs), dim3(256), 0, s, b, counters, partials); break;
      }
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

hipError_t launch_prefill(const void* packed, const Geometry& g, float st, const uint16_t* x, int64_t m, int64_t ldx,
                          void* y, int64_t ldy, bool y_bf16, void* ws, hipStream_t s) {
  if (m == 0 || g.n == 0) return hipSuccess;
  Problem pr{packed, g.n, g.k, st, x, ldx, y, ldy};
  return launch_prefill_batch(&pr, 1, m, y_bf16, ws, s);
}

}  // namespace nvfp4
