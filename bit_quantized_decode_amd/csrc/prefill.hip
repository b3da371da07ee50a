// NVFP4 x bf16 GEMM for many activation rows (prompt prefill).
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
  int ntn[kMaxPre];                 // weight-row tiles (of 256 rows)
  const uint8_t* packed[kMaxPre];
  const uint16_t* x[kMaxPre];
  void* y[kMaxPre];
  int64_t n[kMaxPre], k[kMaxPre], ldx[kMaxPre], ldy[kMaxPre];
  float st[kMaxPre];
  // MX operands (W4A4): `packed` holds the weights' MX codes, these the rest.
  const uint8_t* wsc[kMaxPre];  // weight scale bytes
  const uint8_t* xm[kMaxPre];   // activation codes, first row block of the launch
  const uint8_t* xsc[kMaxPre];  // activation scale bytes, same block
  int64_t nrb[kMaxPre];         // weight row blocks of 32
  int64_t xnrb;                 // activation row blocks of 32 in the launch
};

// One problem's fields, as the kernel uses them.
struct ProbView {
  int64_t iter_begin;
  const uint8_t* packed;
  const uint16_t* x;
  void* y;
  int64_t n, k, ldx, ldy;
  float st;
  int tile_base, iters, nkt, nrt, ntn;
  const uint8_t *wsc, *xm, *xsc;
  int64_t nrb;
};

// Share w covers global iterations [share_begin(w), share_begin(w + 1)).
__device__ __forceinline__ int64_t share_begin(int w, int64_t total, int wgs) { return ((int64_t)w * total) / wgs; }
// The share holding global iteration g.
__device__ __forceinline__ int owner_of(int64_t g, int64_t total, int wgs) { return (int)(((g + 1) * wgs - 1) / total); }

// LDS byte offset of 16-byte chunk c (0..7) of activation row r (128 bytes a
// row).  The chunk is XOR-permuted by a row function that differs between
// any 8 consecutive rows and between the 8 rows of either parity among any 16
// consecutive rows, so that a wavefront's 16-byte reads of one chunk column
// are bank-conflict free whether the LDS serves 128 or 256 bytes a clock.
__device__ __forceinline__ int swz_key(int r) { return ((r >> 1) ^ ((r & 1) << 2)) & 7; }
__device__ __forceinline__ int swz(int r, int c) { return r * (kBK * 2) + ((c ^ swz_key(r)) << 4); }

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

// Partial-sum slot access.  Stores write through to memory (cache policy
// sc1), so that a finisher on any XCD can read them.  A finisher on the
// writers' own XCD reads through its L2 (sc0: past the L1 only); any other
// reads from memory (sc1).
struct PartBuf {
  __amdgpu_buffer_rsrc_t r;
};
__device__ __forceinline__ PartBuf part_buf(float* partials, size_t slot, size_t floats) {
  PartBuf b;
  b.r = __builtin_amdgcn_make_buffer_rsrc(partials + slot * floats, 0, (int)(floats * sizeof(float)), 0x00020000);
  return b;
}
// Byte offset = voff (per lane) + soff (uniform).
__device__ __forceinline__ void store_part(const PartBuf& b, int voff, int soff, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), b.r, voff, soff, 16);
}
template <int POLICY>  // 1: through this XCD's L2 (sc0); 16: from memory (sc1)
__device__ __forceinline__ f32x4 load_part(const PartBuf& b, int voff, int soff) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(b.r, voff, soff, POLICY));
}
template <int V>
struct Policy {
  static constexpr int value = V;
};

// The XCD this wavefront runs on (hardware register XCC_ID, bits 3:0).
__device__ __forceinline__ unsigned xcc_id() { return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 15u; }

// Per-tile XCD masks live in the upper half of the counter area.
constexpr int kMaskBase = (int)(kCounterSlots / 2);

// A operands of k step KS (0..3) of an iteration: weight rows r (a0) and
// 32 + r (a1).  Chunk KS / 2 of the iteration holds k steps 2 (KS / 2) and
// 2 (KS / 2) + 1 (dwords 0-1 and 2-3); the 16-k block of k step KS is byte KS
// of the iteration's scale dword.
struct AOps {
  bf16x8 a0, a1;
};

template <int KS>
__device__ __forceinline__ void dequant_ks(const WStage& w, AOps& o) {
  const u32x4 q = KS < 2 ? w.q0 : w.q1;
  o.a0 = dequant8(q[2 * (KS & 1)], e4m3<KS>(w.sa));
  o.a1 = dequant8(q[2 * (KS & 1) + 1], e4m3<KS>(w.sb));
}

// B operands of k step KS: the JT activation tiles' 16-k slices from LDS.
template <int KS, int JT>
__device__ __forceinline__ void load_b(const uint8_t* xl, int lane, bf16x8 (&b)[JT]) {
  const uint8_t* row = xl + (lane & 31) * (kBK * 2);
  const int c = ((2 * KS + (lane >> 5)) ^ swz_key(lane & 31)) << 4;  // swz_key(32 jt + r) == swz_key(r)
#pragma unroll
  for (int jt = 0; jt < JT; ++jt)
    b[jt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(row + jt * 32 * (kBK * 2) + c));
}

template <int JT>
__device__ __forceinline__ void mfma_ks(const AOps& a, const bf16x8 (&b)[JT], f32x16 (&acc)[2][JT]) {
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) {
    acc[0][jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.a0, b[jt], acc[0][jt], 0, 0, 0);
    acc[1][jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.a1, b[jt], acc[1][jt], 0, 0, 0);
  }
}

// Instruction interleave of one k step: each MFMA is followed by a share of
// the next k step's operand work (an LDS read, dequantisation VALU), so that
// this work issues while the matrix core runs; memory loads go wherever their
// addresses are ready.
template <int JT>
__device__ __forceinline__ void interleave_ks() {
#pragma unroll
  for (int j = 0; j < 2 * JT; ++j) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // MFMA
    if (j < JT) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // DS read
    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);                 // VALU
  }
}


// Float4 u (0 .. 8 JT - 1) of a lane's accumulators: tile t = u / 4 (half
// t / JT, activation tile t % JT), elements 4 (u % 4) .. + 3.
template <int JT>
__device__ __forceinline__ f32x4 frag4(const f32x16 (&acc)[2][JT], int u) {
  const f32x16& a = acc[(u >> 2) / JT][(u >> 2) % JT];
  const int e = 4 * (u & 3);
  return f32x4{a[e], a[e + 1], a[e + 2], a[e + 3]};
}

// Float4 u of a half (0 .. 4 JT - 1) into the wavefront's LDS buffer at the
// place stage_half puts it.
template <int JT>
__device__ __forceinline__ void stage_frag(uint8_t* buf, int lane, int u, f32x4 v) {
  const int jt = (u >> 2) % JT, e4 = u & 3;
  *reinterpret_cast<f32x4*>(buf + swz(32 * jt + (lane & 31), 2 * e4 + (lane >> 5))) = v;
}

// Add v to float4 u of a half where stage_frag / stage_half put it (this
// lane's own slot: no other lane touches it).
template <int JT>
__device__ __forceinline__ void add_frag(uint8_t* buf, int lane, int u, f32x4 v) {
  const int jt = (u >> 2) % JT, e4 = u & 3;
  f32x4* p = reinterpret_cast<f32x4*>(buf + swz(32 * jt + (lane & 31), 2 * e4 + (lane >> 5)));
  *p = *p + v;
}

// Wavefront's half H (accumulator tiles acc[H][*]) into its LDS buffer:
// activation row 32 jt + lane % 32 at byte 128 row, the 4 columns
// 8 e4 + 4 (lane / 32) of the half as 16-byte chunk 2 e4 + lane / 32.
template <int H, int JT>
__device__ __forceinline__ void stage_half(const f32x16 (&acc)[2][JT], uint8_t* buf, int lane) {
#pragma unroll
  for (int jt = 0; jt < JT; ++jt)
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const f32x16& a = acc[H][jt];
      *reinterpret_cast<f32x4*>(buf + swz(32 * jt + (lane & 31), 2 * e4 + (lane >> 5))) =
          f32x4{a[4 * e4], a[4 * e4 + 1], a[4 * e4 + 2], a[4 * e4 + 3]};
    }
}


template <int JT, bool KFULL, bool MX>
__global__ __launch_bounds__(256, 1) void prefill_kernel(const PrefillBatch b, unsigned* __restrict__ counters,
                                                         float* __restrict__ partials) {
  constexpr int kBM = 32 * JT;
  constexpr int kXBuf = kBM * kBK * 2;  // bytes of one activation buffer
  // Four activation buffers, each its own LDS object: accesses to distinct
  // objects carry distinct alias scopes, which lets the compiler see that a
  // load into one buffer does not feed reads of another (else it would wait
  // for every load in flight before each LDS read).
  __shared__ __attribute__((aligned(16))) uint8_t xb0[kXBuf];
  __shared__ __attribute__((aligned(16))) uint8_t xb1[kXBuf];
  __shared__ __attribute__((aligned(16))) uint8_t xb2[kXBuf];
  __shared__ __attribute__((aligned(16))) uint8_t xb3[kXBuf];
#define NVFP4_XBUF(I) ((I) == 0 ? xb0 : (I) == 1 ? xb1 : (I) == 2 ? xb2 : xb3)
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;

  // Share of this workgroup.  Dispatch places workgroup b on XCD b % 8; give
  // each XCD a contiguous run of shares: XCD x runs the q + (x < r) shares
  // from x q + min(x, r) on (q = wgs / 8, r = wgs % 8), a bijection for any
  // workgroup count.
  // Scalars used inside the lambdas below are copied out of the argument
  // struct: a lambda capturing the struct itself would take its address and
  // force a copy of it into scratch memory.
  const int b_wgs = b.wgs, b_count = b.count;
  const int64_t b_total = b.total, b_m = b.m;
  const bool b_ybf16 = b.y_bf16 != 0;
  const int xcd = (int)(blockIdx.x & 7), xq = b_wgs >> 3, xr = b_wgs & 7;
  const int w = xcd * xq + (xcd < xr ? xcd : xr) + (int)(blockIdx.x >> 3);
  const int64_t g_begin = share_begin(w, b_total, b_wgs);
  const int64_t g_end = share_begin(w + 1, b_total, b_wgs);

  for (int64_t g = g_begin; g < g_end;) {
    // ---- locate the segment: problem p, tile (mt, nt), iterations [ib, ie)
    // Per-problem fields are picked with static indices: indexing the
    // argument arrays at run time would copy them to scratch memory (and lose
    // the address space of the pointers in them).
    int p = 0;
#pragma unroll
    for (int i = 1; i < kMaxPre; ++i)
      if (i < b_count && g >= b.iter_begin[i]) p = i;
    ProbView pv;
#pragma unroll
    for (int i = 0; i < kMaxPre; ++i)
      if (i == p) pv = ProbView{b.iter_begin[i], b.packed[i], b.x[i], b.y[i], b.n[i], b.k[i], b.ldx[i], b.ldy[i],
                                b.st[i], b.tile_base[i], b.iters[i], b.nkt[i], b.nrt[i], b.ntn[i],
                                b.wsc[i], b.xm[i], b.xsc[i], b.nrb[i]};
    const int iters = pv.iters;
    const int64_t gl = g - pv.iter_begin;
    const int tile = (int)(gl / iters);
    const int ib = (int)(gl - (int64_t)tile * iters);
    const int64_t tile_g0 = pv.iter_begin + (int64_t)tile * iters;
    const int ie = (int)(g_end - tile_g0 < iters ? g_end - tile_g0 : iters);
    // Tiles run activation-slab-major, so the shares of one XCD mostly read one slab of activation rows.
    const int mt = tile / pv.ntn, nt = tile % pv.ntn;
    const int64_t m0 = (int64_t)mt * kBM;
    const int64_t kdim = pv.k;
    const int nkt = pv.nkt;

    f32x16 acc[2][JT];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < JT; ++j) acc[i][j] = f32x16{};
    if constexpr (MX) {
      // W4A4: both operands are MX tiles (1 KB of codes per 32 rows x 64 k, in
      // the scaled FP4 MFMA's operand order, and 64 E8M0 scale bytes), so an
      // iteration is one MFMA k step and nothing is converted.  Activation
      // blocks go straight into LDS, loaded three iterations ahead: block q's
      // codes at 1024 q; its scales, 16-byte pieces p = 4 q .. 4 q + 3, piece p
      // at 1024 (JT + p / JT) + 16 (p % JT) (wavefront v loads pieces JT v ..
      // JT v + JT - 1 with lanes 0 .. JT - 1; its other lanes repeat them into
      // the rest of its 1 KB, so that no lane is masked off).  Each
      // wavefront's two weight blocks (rows 64 rt .. 64 rt + 63) load four
      // iterations ahead into registers.  Blocks past the end re-read the last
      // one (their outputs are not written).
      static_assert(JT == 4 || JT == 8, "MX tiles: 4 or 8 activation blocks");
      constexpr int kXq = JT / 4;  // activation code blocks a wavefront loads
      const int64_t nks = pv.nkt;
      const int64_t xlast = b.xnrb - 1;
      const uint8_t* xcode[kXq];
#pragma unroll
      for (int j = 0; j < kXq; ++j) {
        int64_t xb = (int64_t)mt * JT + wave * kXq + j;
        xb = xb < xlast ? xb : xlast;
        xcode[j] = pv.xm + xb * nks * 1024 + lane * 16;
      }
      // Lanes 0 .. JT-1 of wavefront v load 16-byte piece p = JT v + lane of the JT * 64 scale bytes.
      const int piece = wave * JT + (lane & (JT - 1));
      int64_t xbs = (int64_t)mt * JT + piece / 4;
      xbs = xbs < xlast ? xbs : xlast;
      const uint8_t* xscale = pv.xsc + xbs * nks * 64 + 16 * (piece & 3);
      auto dma_mx = [&](int it, uint8_t* xbuf) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < kXq; ++j) load_lds16(xcode[j] + (size_t)it * 1024, xbuf + (wave * kXq + j) * 1024);
        load_lds16(xscale + (size_t)it * 64, xbuf + (JT + wave) * 1024);
      };
      int rt = nt * 4 + wave;
      rt = rt < pv.nrt ? rt : pv.nrt - 1;
      const uint8_t* wcode[2];
      const uint8_t* wscale[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        int64_t rb = 2 * (int64_t)rt + h;
        rb = rb < pv.nrb ? rb : pv.nrb - 1;
        wcode[h] = pv.packed + rb * nks * 1024 + lane * 16;
        wscale[h] = pv.wsc + rb * nks * 64 + lane;
      }
      // Scale bytes stay 8-bit in the ring: widened where an MFMA takes them
      // (after that iteration's wait), not where the loop carries them.
      struct MxA {
        u32x4 a0, a1;
        uint8_t s0, s1;
      };
      auto load_a = [&](int it, MxA& o) __attribute__((always_inline)) {
        o.a0 = load16(wcode[0] + (size_t)it * 1024);
        o.a1 = load16(wcode[1] + (size_t)it * 1024);
        o.s0 = wscale[0][(size_t)it * 64];
        o.s1 = wscale[1][(size_t)it * 64];
      };
      // Before the barrier that ends iteration it, the activations of it + 1
      // (loaded during it - 2) must have landed; after them 4 + D + 4 + D + 4
      // memory instructions have been issued (D = kXq + 1 a load of activations).
      constexpr int kVmAfter = 12 + 2 * (kXq + 1);
      const int last = ie - 1;
      auto clampi = [&](int it) __attribute__((always_inline)) { return it < last ? it : last; };
      MxA w0, w1, w2, w3;
      // Prologue in the steady state's issue order: the first iteration waits
      // only for its own operands, not for the whole pipeline fill.
      load_a(ib, w0);
      dma_mx(ib, NVFP4_XBUF(0));
      load_a(clampi(ib + 1), w1);
      dma_mx(clampi(ib + 1), NVFP4_XBUF(1));
      load_a(clampi(ib + 2), w2);
      dma_mx(clampi(ib + 2), NVFP4_XBUF(2));
      load_a(clampi(ib + 3), w3);
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<kVmAfter>();
      barrier_only();
      __builtin_amdgcn_sched_barrier(0);
#define NVFP4_MX_STEP(S, WC)                                                                                  \
  {                                                                                                           \
    const int it = i + (S);                                                                                   \
    const uint8_t* xcur = NVFP4_XBUF(S);                                                                      \
    u32x4 bq[JT];                                                                                             \
    uint32_t bs[JT];                                                                                          \
    _Pragma("unroll") for (int q = 0; q < JT; ++q) {                                                          \
      bq[q] = *reinterpret_cast<const u32x4*>(xcur + q * 1024 + lane * 16);                                   \
      bs[q] = xcur[(JT + 4 * q / JT) * 1024 + (4 * q % JT) * 16 + lane];                                      \
    }                                                                                                         \
    dma_mx(clampi(it + 3), NVFP4_XBUF(((S) + 3) & 3));                                                        \
    const v8i a0 = v8i{(int)WC.a0[0], (int)WC.a0[1], (int)WC.a0[2], (int)WC.a0[3], 0, 0, 0, 0};               \
    const v8i a1 = v8i{(int)WC.a1[0], (int)WC.a1[1], (int)WC.a1[2], (int)WC.a1[3], 0, 0, 0, 0};               \
    _Pragma("unroll") for (int q = 0; q < JT; ++q) {                                                          \
      const v8i bv = v8i{(int)bq[q][0], (int)bq[q][1], (int)bq[q][2], (int)bq[q][3], 0, 0, 0, 0};             \
      acc[0][q] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, bv, acc[0][q], 4, 4, 0, (int)WC.s0, 0,  \
                                                                  (int)bs[q]);                                \
      acc[1][q] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, bv, acc[1][q], 4, 4, 0, (int)WC.s1, 0,  \
                                                                  (int)bs[q]);                                \
    }                                                                                                         \
    /* the products stay ahead of the barrier: nothing may sink them past it */                             \
    _Pragma("unroll") for (int q = 0; q < JT; ++q) asm volatile("" ::"a"(acc[0][q]), "a"(acc[1][q]));         \
    load_a(clampi(it + 4), WC);                                                                               \
    wait_vmcnt_lgkm0<kVmAfter>();                                                                             \
    barrier_only();                                                                                           \
    __builtin_amdgcn_sched_barrier(0);                                                                        \
  }
      int i = ib;
      for (; i + 4 <= ie; i += 4) {
        NVFP4_MX_STEP(0, w0)
        NVFP4_MX_STEP(1, w1)
        NVFP4_MX_STEP(2, w2)
        NVFP4_MX_STEP(3, w3)
      }
      if (i < ie) NVFP4_MX_STEP(0, w0)
      if (i + 1 < ie) NVFP4_MX_STEP(1, w1)
      if (i + 2 < ie) NVFP4_MX_STEP(2, w2)
#undef NVFP4_MX_STEP
    } else {
      // Activations go from memory straight into LDS: load j of this wavefront
      // fills the 1 KB block q = wave * JT + j of a buffer, lane l landing at
      // byte 16 l -- row 8 q + l / 8, physical chunk l % 8 -- so lane l fetches
      // the logical chunk that the swizzle puts there.  Rows past m re-read row
      // m - 1 (their outputs are not written).
      const uint16_t* xrow[JT];
      int c8[JT];  // k offset (elements) of this lane's chunk within an iteration
#pragma unroll
      for (int j = 0; j < JT; ++j) {
        const int row = 8 * (wave * JT + j) + (lane >> 3);
        c8[j] = 8 * ((lane & 7) ^ swz_key(row));
        int64_t r = m0 + row;
        r = r < b_m ? r : b_m - 1;
        xrow[j] = pv.x + r * pv.ldx;
      }
      auto dma_x = [&](int it, uint8_t* xbuf) __attribute__((always_inline)) {
        uint8_t* dst = xbuf + wave * JT * 1024;
#pragma unroll
        for (int j = 0; j < JT; ++j) {
          int64_t kk = (int64_t)it * kBK + c8[j];
          if (!KFULL) kk = kk < kdim ? kk : kdim - 8;  // in bounds; zeroed once landed
          load_lds16(xrow[j] + kk, dst + j * 1024);
        }
      };
      // Iteration it's chunks at k >= K must read as zeros (K % 64 != 0 only):
      // each lane clears the chunks it loaded, after they have landed.
      auto zero_tail = [&](int it, uint8_t* xbuf) __attribute__((always_inline)) {
        if (KFULL || it != iters - 1) return;
#pragma unroll
        for (int j = 0; j < JT; ++j)
          if ((int64_t)it * kBK + c8[j] >= kdim)
            *reinterpret_cast<u32x4*>(xbuf + (wave * JT + j) * 1024 + lane * 16) = u32x4{0u, 0u, 0u, 0u};
      };

      // Weight source: this wavefront's packed row tile (clamped; rows past n are not written).
      int rt = nt * 4 + wave;
      rt = rt < pv.nrt ? rt : pv.nrt - 1;
      // Addresses: a wavefront-uniform base (scalar registers) plus a fixed
      // 32-bit per-lane offset, so no per-step vector address arithmetic.
      const uint8_t* wt = pv.packed + (size_t)rt * nkt * kTileBytes;
      const uint32_t lane_code = lane * 16;
      const uint32_t lane_scale = kScaleOffset + 32 * (lane & 31);
      auto load_w = [&](int it, WStage& s) __attribute__((always_inline)) {
        const uint8_t* tb = wt + (size_t)(it >> 2) * kTileBytes;
        const uint8_t* cb = tb + (it & 3) * 2048;
        const uint8_t* sb = tb + 4 * (it & 3);
        s.q0 = load16(cb + lane_code);
        s.q1 = load16(cb + 1024 + lane_code);
        s.sa = *reinterpret_cast<const uint32_t*>(sb + lane_scale);
        s.sb = *reinterpret_cast<const uint32_t*>(sb + 16 + lane_scale);
      };


      // ---- pipeline.  Four LDS activation buffers: iteration it lives in
      // buffer (it - ib) % 4, loaded three iterations ahead; weights are loaded
      // four iterations ahead; each k step's operands are read from LDS and
      // dequantised during the previous k step's MFMAs.  Loads past the segment
      // re-read its last iteration, so every step issues the same memory
      // instructions in the same order -- per step JT activation loads (k step
      // 0) and four weight loads (k step 2) -- and the main loop has no branches.
      // Before k step 3 of step it the activations of it + 1 (loaded at k step
      // 0 of step it - 2) must have landed; after them 4 + JT + 4 + JT + 4
      // memory instructions have been issued.
      constexpr int kVmAfterX = 12 + 2 * JT;
      const int last = ie - 1;
      auto clampi = [&](int it) __attribute__((always_inline)) { return it < last ? it : last; };
      WStage w0, w1, w2, w3;
      // Prologue in the steady state's issue order (weights of it, then its
      // activations), so that the first iteration waits only for its own
      // operands -- after them 4 + JT + 4 + JT + 4 memory instructions are
      // issued, as before every later iteration -- instead of the whole
      // pipeline fill.  Each later step clears the tail of the activations it
      // waits for (zero_tail), so only the first buffer's is cleared here.
      load_w(ib, w0);
      dma_x(ib, NVFP4_XBUF(0));
      load_w(clampi(ib + 1), w1);
      dma_x(clampi(ib + 1), NVFP4_XBUF(1));
      load_w(clampi(ib + 2), w2);
      dma_x(clampi(ib + 2), NVFP4_XBUF(2));
      load_w(clampi(ib + 3), w3);
      __builtin_amdgcn_sched_barrier(0);  // no operand work is hoisted above the wait (it would wait for every load)
      wait_vmcnt<kVmAfterX>();
      zero_tail(ib, NVFP4_XBUF(0));
      barrier_only();
      __builtin_amdgcn_sched_barrier(0);
      AOps ac, an;
      bf16x8 bc[JT], bn[JT];
      load_b<0, JT>(NVFP4_XBUF(0), lane, bc);
      dequant_ks<0>(w0, ac);
      // Step S of a group of four: iteration it = i + S in buffer S.  On entry
      // ac / bc hold k step 0's operands; on exit, iteration it + 1's.  Before
      // k step 3 every wavefront waits for its loads of it + 1's activations
      // (which also covers the weights of it + 1) and for its own LDS reads,
      // then the workgroup barrier publishes buffer it + 1, so that k step 3
      // can read it + 1's first B operands while its MFMAs run.
#define NVFP4_PREFILL_STEP(S, WC, WN)                                   \
    {                                                                     \
      const int it = i + (S);                                             \
      const uint8_t* xcur = NVFP4_XBUF(S);                                \
      load_b<1, JT>(xcur, lane, bn);                                      \
      dma_x(clampi(it + 3), NVFP4_XBUF(((S) + 3) & 3));                   \
      dequant_ks<1>(WC, an);                                              \
      mfma_ks<JT>(ac, bc, acc);                                           \
      interleave_ks<JT>();                                                \
      __builtin_amdgcn_sched_barrier(0);                                  \
      load_b<2, JT>(xcur, lane, bc);                                      \
      dequant_ks<2>(WC, ac);                                              \
      mfma_ks<JT>(an, bn, acc);                                           \
      interleave_ks<JT>();                                                \
      __builtin_amdgcn_sched_barrier(0);                                  \
      load_b<3, JT>(xcur, lane, bn);                                      \
      dequant_ks<3>(WC, an);                                              \
      load_w(clampi(it + 4), WC);                                         \
      mfma_ks<JT>(ac, bc, acc);                                           \
      interleave_ks<JT>();                                                \
      __builtin_amdgcn_sched_barrier(0);                                  \
      wait_vmcnt_lgkm0<kVmAfterX>();                                      \
      zero_tail(it + 1, NVFP4_XBUF(((S) + 1) & 3));                       \
      barrier_only();                                                     \
      __builtin_amdgcn_sched_barrier(0);                                  \
      load_b<0, JT>(NVFP4_XBUF(((S) + 1) & 3), lane, bc);                 \
      dequant_ks<0>(WN, ac);                                              \
      mfma_ks<JT>(an, bn, acc);                                           \
      interleave_ks<JT>();                                                \
      __builtin_amdgcn_sched_barrier(0);                                  \
    }
      int i = ib;
      for (; i + 4 <= ie; i += 4) {
        NVFP4_PREFILL_STEP(0, w0, w1)
        NVFP4_PREFILL_STEP(1, w1, w2)
        NVFP4_PREFILL_STEP(2, w2, w3)
        NVFP4_PREFILL_STEP(3, w3, w0)
      }
      if (i < ie) NVFP4_PREFILL_STEP(0, w0, w1)
      if (i + 1 < ie) NVFP4_PREFILL_STEP(1, w1, w2)
      if (i + 2 < ie) NVFP4_PREFILL_STEP(2, w2, w3)
#undef NVFP4_PREFILL_STEP
    }

    // ---- output ------------------------------------------------------------
    // Accumulator element e of tile (i, jt) of this lane: weight row
    // 64 * wave + 32 * i + 8 * (e / 4) + 4 * (lane / 32) + e % 4 of the tile,
    // activation row 32 * jt + lane % 32.  The tile leaves the registers
    // through LDS one half (i) at a time: wavefront v writes its columns
    // [64 v + 32 i, +32) of all BM activation rows into activation buffer v
    // (row r at byte 128 r, 16-byte column chunk c at the swizzled slot), and
    // then all threads move whole 16-byte chunks -- coalesced output rows, or
    // partial sums in chunk order (half i, buffer v, row r, chunk c at
    // ((i * 4 + v) * BM + r) * 8 + c).
    wait_vmcnt<0>();  // activation loads past the segment still target the buffers
    __syncthreads();
    const float st = pv.st;
    void* const y = pv.y;
    const int64_t ldy = pv.ldy, n = pv.n;
    const bool vec = (ldy & 3) == 0;
    uint8_t* const mybuf = wave == 0 ? NVFP4_XBUF(0) : wave == 1 ? NVFP4_XBUF(1) : wave == 2 ? NVFP4_XBUF(2) : NVFP4_XBUF(3);
    // 4 output columns (chunk c of buffer v, half h) of activation row r, scaled by s_t.
    auto store_y = [&](int h, int v, int r, int c, f32x4 val) __attribute__((always_inline)) {
      const int64_t row = m0 + r;
      const int64_t col = (int64_t)nt * kBN + 64 * v + 32 * h + 4 * c;
      if (row >= b_m || col >= n) return;
      const float v0 = val[0] * st, v1 = val[1] * st, v2 = val[2] * st, v3 = val[3] * st;
      if (b_ybf16) {
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
    // Thread tid moves chunks q = v * JT + j of a half: buffer v, local chunk
    // e = tid + 256 j, i.e. activation row tid / 8 + 32 j, column chunk tid % 8.
    // When the whole tile lies inside y (and rows are 16-byte aligned) the
    // stores need no checks: one per-thread base pointer, a scalar row stride.
    const bool y_full = vec && m0 + kBM <= b_m && (int64_t)nt * kBN + kBN <= n;
    const int64_t esize = b_ybf16 ? 2 : 4;
    uint8_t* const ythr =
        static_cast<uint8_t*>(y) + ((m0 + (tid >> 3)) * ldy + (int64_t)nt * kBN + 4 * (tid & 7)) * esize;
    const int64_t yrow32 = 32 * ldy * esize;
    auto store_fast = [&](int h, int v, int j, f32x4 val) __attribute__((always_inline)) {
      uint8_t* yr = ythr + j * yrow32 + (64 * v + 32 * h) * esize;
      if (b_ybf16)
        *reinterpret_cast<uint2*>(yr) = make_uint2(pack_bf16x2(val[0] * st, val[1] * st), pack_bf16x2(val[2] * st, val[3] * st));
      else
        *reinterpret_cast<f32x4*>(yr) = f32x4{val[0] * st, val[1] * st, val[2] * st, val[3] * st};
    };
    auto buf_of = [&](int v) __attribute__((always_inline)) -> uint8_t* {
      return v == 0 ? NVFP4_XBUF(0) : v == 1 ? NVFP4_XBUF(1) : v == 2 ? NVFP4_XBUF(2) : NVFP4_XBUF(3);
    };
    auto write_half = [&](int h) __attribute__((always_inline)) {
      if (y_full) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int j = 0; j < JT; ++j) {
            const int e = tid + 256 * j;
            store_fast(h, v, j, *reinterpret_cast<const f32x4*>(NVFP4_XBUF(v) + swz(e >> 3, e & 7)));
          }
        return;
      }
#pragma unroll 1
      for (int q = 0; q < 4 * JT; ++q) {
        const int v = q / JT, e = tid + 256 * (q % JT);
        store_y(h, v, e >> 3, e & 7, *reinterpret_cast<const f32x4*>(buf_of(v) + swz(e >> 3, e & 7)));
      }
    };

    if (ib == 0 && ie == iters) {
      stage_half<0, JT>(acc, mybuf, lane);
      __syncthreads();
      write_half(0);
      __syncthreads();
      stage_half<1, JT>(acc, mybuf, lane);
      __syncthreads();
      write_half(1);
    } else {
      // Cut tile.  Normally each contributor publishes its segment's sums
      // straight from the accumulators (written through to memory, in
      // accumulator order: float4 u of lane l of wavefront v at
      // ((v * 8 JT + u) * 64 + l) * 16 bytes), notes its XCD in the tile's
      // mask, and the last contributor to arrive adds all contributions in k
      // order.  The head segment (the tile's first iterations, which ends this
      // workgroup's share) usually finishes after all the others: if at that
      // point every other contributor has arrived, the head finishes the tile
      // itself, keeping the first half of its sums in LDS (staged as the
      // output is) instead of writing them out and reading them back.
      const int gtile = pv.tile_base + tile;
      const unsigned xcc = xcc_id();
      const int c_first = owner_of(tile_g0, b_total, b_wgs);
      const int c_last = owner_of(tile_g0 + iters - 1, b_total, b_wgs);
      const int slot = g_begin >= tile_g0 ? 0 : 1;  // this workgroup's first or last segment
      const PartBuf mine = part_buf(partials, (size_t)w * 2 + slot, part_floats<JT>());
      const int frag_off = (wave * 8 * JT * 64 + lane) * 16;
      __shared__ unsigned s_others_in;
      bool head_finishes = false;
      if (ib == 0) {
        if (threadIdx.x == 0)
          s_others_in = __hip_atomic_load(counters + gtile, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                        (unsigned)(c_last - c_first);
        __syncthreads();
        head_finishes = s_others_in != 0u;
      }
      bool finisher;
      if (head_finishes) {
        stage_half<0, JT>(acc, mybuf, lane);  // the buffers are free: the main loop ended with a barrier
#pragma unroll
        for (int u = 4 * JT; u < 8 * JT; ++u) store_part(mine, frag_off, u * 1024, frag4<JT>(acc, u));
        if (threadIdx.x == 0) __hip_atomic_store(counters + gtile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);  // the second half's sums have landed before they are read back
        finisher = true;
      } else {
#pragma unroll
        for (int u = 0; u < 8 * JT; ++u) store_part(mine, frag_off, u * 1024, frag4<JT>(acc, u));
        if (threadIdx.x == 0)
          __hip_atomic_fetch_or(counters + kMaskBase + gtile, 1u << xcc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        finisher = arrive_last(counters + gtile, (unsigned)(c_last - c_first + 1));
      }
      if (finisher) {
        // Every contributor that published ran on this XCD: their sums are in
        // this XCD's L2 and are read from there; else from memory.
        const unsigned mask = __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(counters + kMaskBase + gtile, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        __syncthreads();
        if (threadIdx.x == 0)
          __hip_atomic_store(counters + kMaskBase + gtile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool local = mask == (1u << xcc);
        auto slot_of = [&](int c) __attribute__((always_inline)) {
          return part_buf(partials, (size_t)c * 2 + (share_begin(c, b_total, b_wgs) >= tile_g0 ? 0 : 1),
                          part_floats<JT>());
        };
        // Each wavefront sums its own fragments (16 float4 at a time) and
        // stages them like its accumulators; the workgroup then writes the
        // half out coalesced.
        // Sums are ((p_first + p_next) + ...) in contributor (k) order; every
        // contribution is read from its slot (the accumulators are dead once
        // published) except the head's first half when the head finishes,
        // which is staged already and has the others added in place; with two
        // contributions both slots' fragments are loaded together.
        auto finish_half = [&](auto hc, auto policy) __attribute__((always_inline)) {
          constexpr int H = decltype(hc)::value;
          constexpr int POL = decltype(policy)::value;
          // A half holds 4 JT float4s per lane, taken G at a time.
          constexpr int G = 4 * JT < 16 ? 4 * JT : 16;
          if (H == 0 && head_finishes) {
#pragma unroll
            for (int q = 0; q < 4 * JT / G; ++q) {
              for (int c = c_first + 1; c <= c_last; ++c) {
                const PartBuf src = slot_of(c);
                f32x4 v[G];
#pragma unroll
                for (int t = 0; t < G; ++t) v[t] = load_part<POL>(src, frag_off, (G * q + t) * 1024);
#pragma unroll
                for (int t = 0; t < G; ++t) add_frag<JT>(mybuf, lane, G * q + t, v[t]);
              }
            }
            __syncthreads();
            write_half(H);
            return;
          }
          __syncthreads();  // the buffers are free
#pragma unroll
          for (int q = 0; q < 4 * JT / G; ++q) {  // float4s u = 4 JT H + G q + [0, G)
            constexpr int U0 = 4 * JT * H;
            f32x4 sum[G];
            if (c_last - c_first == 1) {
              const PartBuf s0 = slot_of(c_first), s1 = slot_of(c_last);
              f32x4 v0[G], v1[G];
#pragma unroll
              for (int t = 0; t < G; ++t) {
                v0[t] = load_part<POL>(s0, frag_off, (U0 + G * q + t) * 1024);
                v1[t] = load_part<POL>(s1, frag_off, (U0 + G * q + t) * 1024);
              }
#pragma unroll
              for (int t = 0; t < G; ++t) sum[t] = v0[t] + v1[t];
            } else {
              for (int c = c_first; c <= c_last; ++c) {
                const PartBuf src = slot_of(c);
                f32x4 v[G];
#pragma unroll
                for (int t = 0; t < G; ++t) v[t] = load_part<POL>(src, frag_off, (U0 + G * q + t) * 1024);
#pragma unroll
                for (int t = 0; t < G; ++t) sum[t] = c == c_first ? v[t] : sum[t] + v[t];
              }
            }
#pragma unroll
            for (int t = 0; t < G; ++t) stage_frag<JT>(mybuf, lane, G * q + t, sum[t]);
          }
          __syncthreads();
          write_half(H);
        };
        if (local) {
          finish_half(Policy<0>(), Policy<1>());
          finish_half(Policy<1>(), Policy<1>());
        } else {
          finish_half(Policy<0>(), Policy<16>());
          finish_half(Policy<1>(), Policy<16>());
        }
      }
    }
    __syncthreads();  // the buffers are refilled by the next segment
    g = tile_g0 + ie;
  }
#undef NVFP4_XBUF
}

template <int JT, bool KFULL, bool MX = false>
void launch_one(const PrefillBatch& b, unsigned wgs, unsigned* counters, float* partials, hipStream_t s) {
  prefill_kernel<JT, KFULL, MX><<<dim3(wgs), dim3(256), 0, s>>>(b, counters, partials);
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
  // One counter and one XCD mask per output tile of a launch: cut m so that a launch's tiles fit.
  // (Launches hold at most 8 problems of at most kCounterSlots row tiles of
  // 64 in all, so ntiles <= kCounterSlots / 4 and max_mt >= 2.)
  int64_t max_mt = ntiles > 0 ? (kCounterSlots / 2) / ntiles : 1;
  if (max_mt < 1) max_mt = 1;
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
        b.ntn[j] = ntn;
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
      bool kfull = true;  // every problem's k a multiple of the iteration depth
      for (int j = 0; j < nq; ++j) kfull = kfull && (q[j].k % kBK) == 0;
      const unsigned nwg = (unsigned)wgs;
      if (pl.jt == 8) {
        if (kfull) launch_one<8, true>(b, nwg, counters, partials, s);
        else launch_one<8, false>(b, nwg, counters, partials, s);
      } else if (pl.jt == 4) {
        if (kfull) launch_one<4, true>(b, nwg, counters, partials, s);
        else launch_one<4, false>(b, nwg, counters, partials, s);
      } else {
        if (kfull) launch_one<2, true>(b, nwg, counters, partials, s);
        else launch_one<2, false>(b, nwg, counters, partials, s);
      }
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

// Workgroup count for an MX launch.  Its iterations are cheap next to the
// fix-up of a tile cut between workgroups (measured: one cut costs about as
// much as 40 iterations), so fewer, longer shares can win when their
// boundaries fall on tile boundaries -- e.g. 204 shares of 160 iterations over
// gate, up and down at 512 tokens cut no gate or up tile (~10 % faster than 256
// shares, which cut nearly every tile).  Candidates: 256, and every count in
// [192, 256] whose share is a whole number of one problem's tiles; each is
// scored as its share length plus 32 iterations per cut boundary per workgroup.
int64_t mx_share_count(const PrefillBatch& b, int nq) {
  constexpr int64_t kCutCost = 32, kLow = 192;
  const int64_t total = b.total;
  auto cuts = [&](int64_t wgs) {
    int64_t n = 0;
    for (int64_t w = 1; w < wgs; ++w) {
      const int64_t g = w * total / wgs;
      int p = 0;
      for (int i = 1; i < nq; ++i)
        if (g >= b.iter_begin[i]) p = i;
      if ((g - b.iter_begin[p]) % b.iters[p] != 0) ++n;
    }
    return n;
  };
  auto score = [&](int64_t wgs) { return (total + wgs - 1) / wgs + (2 * kCutCost * cuts(wgs)) / wgs; };
  int64_t best = kPreWgs, best_score = score(kPreWgs);
  for (int i = 0; i < nq; ++i)
    for (int64_t j = 1; j <= 64; ++j) {
      const int64_t len = j * b.iters[i];
      if (total % len != 0) continue;
      const int64_t wgs = total / len;
      if (wgs < kLow || wgs >= kPreWgs) continue;
      const int64_t sc = score(wgs);
      if (sc < best_score) best = wgs, best_score = sc;
    }
  return best;
}

size_t w4a4_streamk_bytes() { return kCounterBytes + (size_t)2 * kPreWgs * part_bytes(8); }

hipError_t launch_w4a4_batch(const MxProblem* p, int count, int64_t m, bool y_bf16, void* ws, hipStream_t s) {
  if (m <= 0) return hipSuccess;
  const size_t esize = y_bf16 ? 2 : 4;
  const int jt = m > 128 ? 8 : 4;
  const int64_t bm = 32 * jt, xnrb_all = (m + 31) / 32;
  unsigned* counters = static_cast<unsigned*>(ws);
  float* partials = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kCounterBytes);
  for (int c0 = 0; c0 < count; c0 += kMaxPre) {
    const int cn = count - c0 < kMaxPre ? count - c0 : kMaxPre;
    MxProblem q[kMaxPre];
    int nq = 0;
    for (int i = c0; i < c0 + cn; ++i)
      if (p[i].n > 0 && p[i].k > 0) q[nq++] = p[i];
    if (nq == 0) continue;
    // One counter and one XCD mask per output tile of a launch: cut m so that
    // a launch's tiles fit (a launch holds at most kCounterSlots row tiles of
    // 64, so at most kCounterSlots / 4 weight-row tiles and max_mt >= 2).
    int64_t ntiles = 0;
    for (int j = 0; j < nq; ++j) ntiles += ((q[j].n + 63) / 64 + 3) / 4;
    int64_t max_mt = (kCounterSlots / 2) / ntiles;
    if (max_mt < 1) max_mt = 1;
    const int64_t mt_all = (m + bm - 1) / bm;
    const int64_t mrows = (mt_all <= max_mt ? mt_all : max_mt) * bm;
    for (int64_t r0 = 0; r0 < m; r0 += mrows) {
      const int64_t mr = m - r0 < mrows ? m - r0 : mrows;
      PrefillBatch b{};
      b.count = nq;
      b.mtiles = (int)((mr + bm - 1) / bm);
      b.y_bf16 = y_bf16 ? 1 : 0;
      b.m = mr;
      b.xnrb = (mr + 31) / 32;
      int64_t it = 0;
      int tiles = 0;
      for (int j = 0; j < nq; ++j) {
        const int64_t nrb = (q[j].n + 31) / 32, nks = (q[j].k + 63) / 64;
        const int nrt = (int)((nrb + 1) / 2), ntn = (nrt + 3) / 4;
        b.iter_begin[j] = it;
        b.tile_base[j] = tiles;
        b.iters[j] = (int)nks;
        b.nkt[j] = (int)nks;
        b.nrt[j] = nrt;
        b.ntn[j] = ntn;
        b.packed[j] = q[j].w;
        b.wsc[j] = q[j].w + (size_t)nrb * nks * 1024;
        b.xm[j] = q[j].x + (size_t)(r0 / 32) * nks * 1024;
        b.xsc[j] = q[j].x + (size_t)xnrb_all * nks * 1024 + (size_t)(r0 / 32) * nks * 64;
        b.nrb[j] = nrb;
        b.y[j] = static_cast<uint8_t*>(q[j].y) + (size_t)r0 * q[j].ldy * esize;
        b.n[j] = q[j].n;
        b.k[j] = q[j].k;
        b.ldy[j] = q[j].ldy;
        b.st[j] = q[j].st;
        tiles += ntn * b.mtiles;
        it += (int64_t)ntn * b.mtiles * nks;
      }
      b.iter_begin[nq] = it;
      b.total = it;
      int64_t wgs = it / kMinShare;
      wgs = wgs < 1 ? 1 : (wgs > kPreWgs ? kPreWgs : wgs);
      if (wgs == kPreWgs) wgs = mx_share_count(b, nq);
      b.wgs = (int)wgs;
      if (jt == 8) launch_one<8, true, true>(b, (unsigned)wgs, counters, partials, s);
      else launch_one<4, true, true>(b, (unsigned)wgs, counters, partials, s);
      const hipError_t e = hipGetLastError();
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
