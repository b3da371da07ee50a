// The top-k routed mixture-of-experts layer on NVFP4 experts.
//
// Each token is routed to `top_k` of `experts` experts and only the routed
// experts' weights are read (CHImp-Alpha-v1.0 model card, "How it fits on one
// GPU": 10 of 512 experts per token).  Launches on the caller's stream:
//   1. route    one wavefront per token: top_k rounds of a wavefront-wide
//               (logit desc, id asc) maximum, then the softmax over the
//               selected logits (fp32);
//   2. group    one workgroup: expert histogram, exclusive scan, the stable
//               counting sort of the flat (t*top_k + j) indices by expert, and
//               the work list of the expert GEMMs: each active expert's rows
//               in chunks of 32 with their token indices -- integer only, so
//               bit-exact and independent of scheduling;
//   3. gate/up  per (chunk, 64-row tile): the expert's gate and up tiles over
//               k slots, activation rows gathered by the chunk's token list,
//               then h = bf16(silu(s_g Wg x) * (s_u Wu x));
//   4. down     per (chunk, four 64-row tiles): d = s_d Wd h (fp32);
//   5. scatter  y[t] = sum_j g[t][j] * d[pos(t, j)], j ascending.
// The expert GEMMs run on persistent grids (at most two workgroups per CU,
// what fits at once) that walk the work list; its actual length is read on
// the device.  A chunk's record holds everything a GEMM workgroup needs, so
// its weight loads wait on one load only.
// A small batch (tokens * top_k <= 1024 routed rows over at most 1024
// experts, the decode case) skips launch 2: every gate/up workgroup groups
// the routed rows itself in its LDS before its first item -- a few
// microseconds of integer work in parallel on every CU instead of a
// dependent one-workgroup launch -- and workgroup 0 writes the grouping
// outputs and the work-list headers that launches 4 and 5 read.  The result
// is the same stable grouping, bit for bit.
#include <atomic>

#include "device_common.h"
#include "launchers.h"
#include "skinny_core.h"

namespace nvfp4 {
namespace {

constexpr int kMaxExperts = 2048;
constexpr int kMaxTopK = 64;
constexpr int kChunkRows = 32;               // activation rows per expert-GEMM workgroup
constexpr int kChunkInts = 4 + kChunkRows;   // one work-list record
// Batches the gate/up workgroups group in their own LDS.
constexpr int kLocalFlat = 1024;
constexpr int kLocalExperts = 1024;
constexpr int kLocalChunks = kLocalExperts + kLocalFlat / kChunkRows;  // bound on the work-list length

// Routing key of one logit: larger logit first, then the smaller expert id
// (-0 counts as +0); unsigned 64-bit order = (logit desc, id asc).
__device__ __forceinline__ uint64_t route_key(float v, int id) {
  uint32_t b = v == 0.0f ? 0u : __float_as_uint(v);
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)b << 32) | (uint32_t)~id;
}
__device__ __forceinline__ float key_logit(uint64_t k) {
  const uint32_t b = (uint32_t)(k >> 32);
  return __uint_as_float((b & 0x80000000u) ? (b & 0x7fffffffu) : ~b);
}

// Wavefront-wide maximum of a 32-bit value, in every lane: shifts within
// each row of 16 leave the row maximum in its lane 15, two row broadcasts
// gather it in lane 63, which is then read out.  (DPP lane moves; a lane
// without a source keeps its own value.)
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t max_step(uint32_t v) {
  const uint32_t o = __builtin_amdgcn_update_dpp(v, v, CTRL, ROWS, 0xf, false);
  return o > v ? o : v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max_step<0x111, 0xf>(v);  // row_shr:1
  v = max_step<0x112, 0xf>(v);  // row_shr:2
  v = max_step<0x114, 0xf>(v);  // row_shr:4
  v = max_step<0x118, 0xf>(v);  // row_shr:8
  v = max_step<0x142, 0xa>(v);  // row_bcast:15 into rows 1, 3
  v = max_step<0x143, 0xc>(v);  // row_bcast:31 into rows 2, 3
  return __builtin_amdgcn_readlane(v, 63);
}

// The maximum 64-bit key of the wavefront: the maximum upper half first;
// only if several lanes hold it (tied logits) the lower halves decide.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) {
  const uint32_t hi = (uint32_t)(k >> 32), lo = (uint32_t)k;
  const uint32_t mh = wave_max_u32(hi);
  const uint64_t tied = __ballot(hi == mh);
  uint32_t ml;
  if ((tied & (tied - 1)) == 0) ml = __builtin_amdgcn_readlane(lo, __builtin_ctzll(tied));  // one lane
  else ml = wave_max_u32(hi == mh ? lo : 0u);
  return ((uint64_t)mh << 32) | ml;
}

// Route one token (one wavefront): top_k rounds of the wavefront-wide
// (logit desc, id asc) maximum, then the softmax over the selected logits
// (fp32, exponentials relative to the largest, summed in selection order).
// Lane l holds the logits of experts l + 64 i (i < NPL); each lane keeps its
// best remaining key, and only the round's winner recomputes its own.
template <int NPL>
__device__ __forceinline__ void route_token(const float* __restrict__ lt, int experts, int top_k, int lane,
                                            float* s_val /* [top_k], this wavefront's */, int32_t* ids_out,
                                            float* g_out) {
  // All loads first (addresses clamped into the row), then the keys: a
  // load under a branch would be waited for on its own.
  float v[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = lt[e < experts ? e : experts - 1];
  }
  uint64_t key[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < experts ? route_key(v[i], e) : 0ull;
  }
  auto local_best = [&]() __attribute__((always_inline)) {
    uint64_t b = key[0];
#pragma unroll
    for (int i = 1; i < NPL; ++i) b = key[i] > b ? key[i] : b;
    return b;
  };
  uint64_t best = local_best();
  int win_id = 0;
  for (int r = 0; r < top_k; ++r) {
    const uint64_t wk = wave_max_key(best);
    const int id = (int)~(uint32_t)wk;
    if (lane == 0) s_val[r] = key_logit(wk);
    if (lane == r) win_id = id;
    if (lane == (id & 63)) {
#pragma unroll
      for (int i = 0; i < NPL; ++i)
        if (i == (id >> 6)) key[i] = 0ull;
      best = local_best();
    }
  }
  // Lanes j < top_k: exponential of selection j; lane 0 adds them in order.
  // (LDS operations of one wavefront are performed in order.)
  const float l0 = s_val[0];
  float ex = 0.0f;
  if (lane < top_k) {
    ex = expf(s_val[lane] - l0);
    s_val[lane] = ex;
  }
  __builtin_amdgcn_wave_barrier();
  // Lane 0 adds them in order, sixteen LDS reads per round issued together.
  float sum = 0.0f;
  if (lane == 0)
    for (int j0 = 0; j0 < top_k; j0 += 16) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = s_val[j0 + u < top_k ? j0 + u : top_k - 1];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (j0 + u < top_k) sum += v[u];
    }
  sum = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(sum), 0));
  if (lane < top_k) {
    ids_out[lane] = win_id;
    g_out[lane] = ex / sum;
  }
}

// One token per 64-thread workgroup: a small batch spreads over many CUs.
template <int NPL>
__global__ __launch_bounds__(64) void route_kernel(const float* __restrict__ logits, int64_t tokens, int experts,
                                                   int top_k, int32_t* __restrict__ ids, float* __restrict__ g) {
  __shared__ float s_val[kMaxTopK];
  const int64_t t = blockIdx.x;
  route_token<NPL>(logits + t * experts, experts, top_k, threadIdx.x, s_val, ids + t * top_k, g + t * top_k);
}

// Inclusive sum over the lanes of a wavefront (DPP: shifts within each row
// of 16, then row broadcasts; a lane without a source adds 0).
template <int CTRL, int ROWS>
__device__ __forceinline__ int scan_step(int v) {
  return v + __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xf, false);
}
__device__ __forceinline__ int wave_inclusive_sum(int v) {
  v = scan_step<0x111, 0xf>(v);  // row_shr:1
  v = scan_step<0x112, 0xf>(v);  // row_shr:2
  v = scan_step<0x114, 0xf>(v);  // row_shr:4
  v = scan_step<0x118, 0xf>(v);  // row_shr:8
  v = scan_step<0x142, 0xa>(v);  // row_bcast:15 into rows 1, 3
  v = scan_step<0x143, 0xc>(v);  // row_bcast:31 into rows 2, 3
  return v;
}

// Exclusive scan of `in[0..n)` (n <= 2048) by a 1024-thread workgroup
// (thread t owns elements 2t, 2t+1); returns the total.  `in` and `out` may
// be the same array.
__device__ int block_exclusive_scan(const int* in, int* out, int n, int* s_tmp /* [32] */) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int a0 = 2 * tid < n ? in[2 * tid] : 0;
  const int a1 = 2 * tid + 1 < n ? in[2 * tid + 1] : 0;
  const int incl = wave_inclusive_sum(a0 + a1);
  if (lane == 63) s_tmp[wave] = incl;
  __syncthreads();
  if (tid < 64) {
    const int t = lane < 16 ? s_tmp[lane] : 0;
    const int ti = wave_inclusive_sum(t);
    if (lane < 16) s_tmp[16 + lane] = ti - t;  // exclusive prefix of the wavefront totals
    if (lane == 15) s_tmp[32] = ti;
  }
  __syncthreads();
  const int excl = s_tmp[16 + wave] + incl - (a0 + a1);
  if (2 * tid < n) out[2 * tid] = excl;
  if (2 * tid + 1 < n) out[2 * tid + 1] = excl + a0;
  const int total = s_tmp[32];
  __syncthreads();
  return total;
}

// Grouping by one 1024-thread workgroup (ids: global or LDS).
__device__ __forceinline__ void group_body(const int32_t* ids, int total, int experts, int top_k,
                                           int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                           int32_t* __restrict__ perm, int32_t* __restrict__ pos,
                                           int32_t* __restrict__ chunks, int32_t* __restrict__ n_chunks) {
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_off[kMaxExperts];
  __shared__ int s_run[kMaxExperts];
  __shared__ int s_chb[kMaxExperts];
  __shared__ int s_last[kMaxExperts];  // token of each expert's last row
  __shared__ int s_tmp[64];
  const int tid = threadIdx.x;
  for (int e = tid; e < experts; e += 1024) { s_cnt[e] = 0; s_run[e] = 0; }
  __syncthreads();
  for (int f = tid; f < total; f += 1024) atomicAdd(&s_cnt[ids[f]], 1);
  __syncthreads();
  const int all = block_exclusive_scan(s_cnt, s_off, experts, s_tmp);
  for (int e = tid; e < experts; e += 1024) {
    counts[e] = s_cnt[e];
    offsets[e] = s_off[e];
    s_chb[e] = (s_cnt[e] + kChunkRows - 1) / kChunkRows;
  }
  if (tid == 0) offsets[experts] = all;
  __syncthreads();
  // Work list of the expert GEMMs: each expert's rows in chunks of 32, in
  // expert order; record j = {expert, first row slot, rows, 0, the token of
  // each of its 32 rows (the last one repeated past the end)}.
  const int nch = block_exclusive_scan(s_chb, s_chb, experts, s_tmp);
  if (tid == 0) *n_chunks = nch;
  // Stable counting sort, 1024 flat indices at a time; each row's token goes
  // straight into its chunk record.  Within a wavefront a row's rank among
  // equal experts comes from lane masks (one round per distinct expert);
  // the wavefronts then take their rows in order.
  const int wave = tid >> 6, lane = tid & 63;
  const uint64_t lanes_below = (1ull << lane) - 1ull;
  for (int base = 0; base < total; base += 1024) {
    const int f = base + tid;
    const int e = f < total ? ids[f] : -1;
    uint64_t todo = __ballot(e >= 0);
    int rank_w = 0, cnt_w = 0;
    while (todo) {
      const int le = __builtin_amdgcn_readlane(e, __builtin_ctzll(todo));
      const uint64_t m = __ballot(e == le);
      if (e == le) {
        rank_w = __builtin_popcountll(m & lanes_below);
        cnt_w = __builtin_popcountll(m);
      }
      todo &= ~m;
    }
    const int nw = (total - base + 63) / 64 < 16 ? (total - base + 63) / 64 : 16;
    for (int w = 0; w < nw; ++w) {
      if (wave == w && e >= 0) {
        const int r = s_run[e] + rank_w;  // row within the expert
        const int p = s_off[e] + r;
        perm[p] = f;
        pos[f] = p;
        chunks[(size_t)(s_chb[e] + r / kChunkRows) * kChunkInts + 4 + r % kChunkRows] = f / top_k;
        if (r == s_cnt[e] - 1) s_last[e] = f / top_k;
      }
      __syncthreads();
      if (wave == w && e >= 0 && rank_w == 0) s_run[e] += cnt_w;
      __syncthreads();
    }
  }
  // Headers, and the unused rows of each expert's last chunk.
  for (int e = tid; e < experts; e += 1024) {
    const int cnt = s_cnt[e];
    for (int c = 0; c * kChunkRows < cnt; ++c) {
      int32_t* r = chunks + (size_t)(s_chb[e] + c) * kChunkInts;
      const int rows = cnt - c * kChunkRows < kChunkRows ? cnt - c * kChunkRows : kChunkRows;
      r[0] = e;
      r[1] = s_off[e] + c * kChunkRows;
      r[2] = rows;
      r[3] = 0;
      if (rows < kChunkRows) {
        const int tok = s_last[e];
        for (int q = rows; q < kChunkRows; ++q) r[4 + q] = tok;
      }
    }
  }
}

__global__ __launch_bounds__(1024) void group_kernel(const int32_t* __restrict__ ids, int total, int experts,
                                                     int top_k, int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                     int32_t* __restrict__ pos, int32_t* __restrict__ chunks,
                                                     int32_t* __restrict__ n_chunks) {
  group_body(ids, total, experts, top_k, counts, offsets, perm, pos, chunks, n_chunks);
}

// ---- grouping inside the expert-GEMM workgroups (small batches) ----------
// What a gate/up workgroup keeps of the grouping for its items: the expert
// offsets, the stable permutation, and per work-list chunk its expert and
// its index among that expert's chunks.
struct LocalGroups {
  int off[kLocalExperts + 1];
  int perm[kLocalFlat];
  uint32_t chunk[kLocalChunks];  // expert << 16 | chunk index within the expert
  int nch;
};

// Two exclusive scans at once over n <= 1024 entries by a 512-thread
// workgroup (thread t owns entries 2t, 2t+1): out_a of in_a, and out_b of
// the 32-row chunk counts ceil(in_a / 32).  out_a[n] and out_b[n] receive the
// totals.  s_red: 32 ints of scratch.
__device__ __forceinline__ void scan_counts_512(const int* in_a, int* out_a, int* out_b, int n, int* s_red) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int a0 = 2 * tid < n ? in_a[2 * tid] : 0;
  const int a1 = 2 * tid + 1 < n ? in_a[2 * tid + 1] : 0;
  const int b0 = (a0 + kChunkRows - 1) / kChunkRows, b1 = (a1 + kChunkRows - 1) / kChunkRows;
  const int ia = wave_inclusive_sum(a0 + a1), ib = wave_inclusive_sum(b0 + b1);
  if (lane == 63) {
    s_red[wave] = ia;
    s_red[8 + wave] = ib;
  }
  __syncthreads();
  if (tid < 64) {
    // Lanes 0-7 scan the eight wavefront totals of a, lanes 16-23 those of b.
    const int v = (lane & 15) < 8 && lane < 32 ? s_red[(lane >> 4) * 8 + (lane & 7)] : 0;
    const int inc = wave_inclusive_sum(v);  // rows of 16: lanes 16-31 continue lanes 0-15's sum
    const int tot_a = __builtin_amdgcn_readlane(inc, 15);
    const int base = lane >= 16 && lane < 32 ? tot_a : 0;
    if (lane < 8) s_red[16 + lane] = inc - v;
    if (lane >= 16 && lane < 24) s_red[24 + (lane & 7)] = inc - base - v;
    if (lane == 7) s_red[32] = inc;
    if (lane == 23) s_red[33] = inc - base;
  }
  __syncthreads();
  const int ea = s_red[16 + wave] + ia - (a0 + a1), eb = s_red[24 + wave] + ib - (b0 + b1);
  if (2 * tid < n) {
    out_a[2 * tid] = ea;
    out_b[2 * tid] = eb;
  }
  if (2 * tid + 1 < n) {
    out_a[2 * tid + 1] = ea + a0;
    out_b[2 * tid + 1] = eb + b0;
  }
  if (tid == 0) {
    out_a[n] = s_red[32];
    out_b[n] = s_red[33];
  }
  __syncthreads();
}

// The stable grouping of `flat` routed rows (flat <= kLocalFlat, experts <=
// kLocalExperts) by a 512-thread workgroup, into `lg`.  `tmp` is scratch of at
// least (2 kLocalFlat + 3 kLocalExperts + 65) ints.  Each row is placed in
// its expert's segment by an LDS atomic (any order), then ranked by the
// number of that segment's rows with a smaller flat index, so the
// permutation is the stable sort by expert whatever the atomics' order.
// With `write` the grouping outputs and the work-list headers (expert, first
// row slot, rows) also go to memory.
__device__ void group_local(const int32_t* __restrict__ ids, int flat, int experts, int* tmp, LocalGroups& lg,
                            bool write, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                            int32_t* __restrict__ perm, int32_t* __restrict__ pos, int32_t* __restrict__ chunks,
                            int32_t* __restrict__ n_chunks) {
  int* s_ids = tmp;                     // [kLocalFlat]
  int* s_unord = s_ids + kLocalFlat;    // [kLocalFlat] rows placed by atomics
  int* s_cnt = s_unord + kLocalFlat;    // [kLocalExperts]
  int* s_run = s_cnt + kLocalExperts;   // [kLocalExperts]
  int* s_chb = s_run + kLocalExperts;   // [kLocalExperts + 1] first chunk of each expert
  int* s_red = s_chb + kLocalExperts + 1;
  const int tid = threadIdx.x;
  for (int f = tid; f < flat; f += 512) s_ids[f] = ids[f];
  for (int e = tid; e < experts; e += 512) s_cnt[e] = s_run[e] = 0;
  __syncthreads();
  for (int f = tid; f < flat; f += 512) atomicAdd(&s_cnt[s_ids[f]], 1);
  __syncthreads();
  scan_counts_512(s_cnt, lg.off, s_chb, experts, s_red);
  for (int f = tid; f < flat; f += 512) {
    const int e = s_ids[f];
    s_unord[lg.off[e] + atomicAdd(&s_run[e], 1)] = f;
  }
  __syncthreads();
  for (int f = tid; f < flat; f += 512) {
    const int e = s_ids[f], b = lg.off[e], n = s_cnt[e];
    int r = 0;
    for (int q0 = 0; q0 < n; q0 += 8) {  // eight LDS reads per round, issued together
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = s_unord[b + (q0 + u < n ? q0 + u : n - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u) r += (q0 + u < n && v[u] < f) ? 1 : 0;
    }
    lg.perm[b + r] = f;
  }
  for (int e = tid; e < experts; e += 512)
    for (int c = 0, c0 = s_chb[e]; c0 + c < s_chb[e + 1]; ++c) lg.chunk[c0 + c] = ((uint32_t)e << 16) | (uint32_t)c;
  if (tid == 0) lg.nch = s_chb[experts];
  __syncthreads();
  if (write) {
    for (int e = tid; e < experts; e += 512) {
      counts[e] = s_cnt[e];
      offsets[e] = lg.off[e];
    }
    if (tid == 0) {
      offsets[experts] = flat;
      *n_chunks = lg.nch;
    }
    for (int p = tid; p < flat; p += 512) {
      perm[p] = lg.perm[p];
      pos[lg.perm[p]] = p;
    }
    for (int j = tid; j < lg.nch; j += 512) {
      const int e = (int)(lg.chunk[j] >> 16), c = (int)(lg.chunk[j] & 0xffffu);
      const int p0 = lg.off[e] + c * kChunkRows;
      const int rows = lg.off[e] + s_cnt[e] - p0 < kChunkRows ? lg.off[e] + s_cnt[e] - p0 : kChunkRows;
      int32_t* r = chunks + (size_t)j * kChunkInts;
      r[0] = e;
      r[1] = p0;
      r[2] = rows;
      r[3] = 0;
    }
  }
  __syncthreads();  // the scratch is free again
}

// ---- expert GEMMs --------------------------------------------------------
// One workgroup of 8 wavefronts per (work-list chunk, output rows); each
// wavefront multiplies one 64-row weight tile by one 256-k activation tile
// per round.  Each round stages
// the chunk's activation tiles of the k slots in LDS once for all eight
// (activations past K load as zeros).  The products of the k slots then meet
// in LDS and are added in slot order.  This spreads a small expert batch
// over the whole chip -- two workgroups per CU, four wavefronts per SIMD,
// which the dequantisation needs to keep a SIMD busy.
constexpr int kExpertWaves = 8;
constexpr int kExpertLds = 64 * 1024;  // 4 activation tiles, later 8 wavefronts' partial sums
static_assert(kExpertWaves * 64 == 512, "group_local and scan_counts_512 assume 512 threads");

// This wavefront's share of staging k tiles t0 .. t0 + KS - 1 of a chunk:
// activation rows 4 w .. 4 w + 3 of each (row 4 w + 2 j + lane / 32 from
// `xrow[j]`), swizzled as skinny_core.h lays tiles out.
template <int KS>
__device__ __forceinline__ void stage_k_tiles(const uint16_t* const (&xrow)[2], int t0, int k, int wave, int lane,
                                              uint8_t* lds) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int srow = 4 * wave + 2 * j + (lane >> 5);
    const int cofs = 8 * ((lane & 31) ^ (srow & 15));
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      const int kk = (t0 + t) * kTileK + cofs;
      const uint16_t* src = kk < k ? xrow[j] + kk : reinterpret_cast<const uint16_t*>(&g_zero_chunk);
      load_lds16(src, lds + t * kXTileBytes + (4 * wave + 2 * j) * 512);
    }
  }
}

// Rounds over the k tiles: wavefront slot `slot` of KS takes tiles slot,
// slot + KS, ...; its 64-row tile at `wrow` (null: no rows, stages only).
// The running sums acc_a / acc_b continue one matrix chain across rounds.
// (A round's weights load with its activations: holding the next round's
// weights as well would not fit four wavefronts per SIMD.)
template <int KS>
__device__ __forceinline__ void expert_rounds(const uint8_t* wrow, int nkt, int k, int slot,
                                              const uint16_t* const (&xrow)[2], int wave, int lane, uint8_t* lds,
                                              f32x16& acc_a, f32x16& acc_b) {
  for (int g0 = 0; g0 < nkt; g0 += KS) {
    const int kt = g0 + slot;
    const bool mine = wrow && kt < nkt;
    WTile w;
    if (mine) load_wtile(wrow + (size_t)kt * kTileBytes, lane, w);
    stage_k_tiles<KS>(xrow, g0, k, wave, lane, lds);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (mine) tile_product(w, lds + slot * kXTileBytes, lane, acc_a, acc_b);
    __syncthreads();  // the tiles are consumed before they are overwritten
  }
}

__device__ __forceinline__ void store_partials(float* red, int wave, int lane, const f32x16& acc_a,
                                               const f32x16& acc_b) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    red[(32 * wave + i) * 64 + lane] = acc_a[i];
    red[(32 * wave + 16 + i) * 64 + lane] = acc_b[i];
  }
}

// Gate/up.  Workgroup (chunk, row tile rt): wavefronts 0-3 take the gate
// matrix's tile rt at k slots 0-3, wavefronts 4-7 the up matrix's; then
// h = bf16(silu(s_g Wg x) * (s_u Wu x)) for the tile's 64 rows.
// LOCAL: the workgroup first groups the routed rows (`ids`) itself; the work
// list then lives in its LDS, and workgroup 0 writes the grouping outputs.
struct LocalArgs {
  const int32_t* ids;
  int flat, experts, top_k;
  int32_t *counts, *offsets, *perm, *pos;
};

template <bool LOCAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void gate_up_kernel(
    const uint16_t* __restrict__ x, int32_t* __restrict__ chunks, int32_t* __restrict__ n_chunks,
    int max_chunks, int hidden, int inter, const uint8_t* __restrict__ w_gate, const uint8_t* __restrict__ w_up,
    size_t stride_gate, size_t stride_up, const int32_t* __restrict__ slot_table,
    const float* __restrict__ scale_gate, const float* __restrict__ scale_up, uint16_t* __restrict__ h,
    float* __restrict__ dbg_gate, float* __restrict__ dbg_up, const LocalArgs la) {
  constexpr int KS = 4;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kExpertLds];
  __shared__ LocalGroups lg;  // LOCAL only (otherwise unused, and not allocated)
  const int nrt = (inter + 63) / 64;
  const int nkt = (hidden + 255) / 256;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int slot = wave % KS;
  int nch;
  if constexpr (LOCAL) {
    group_local(la.ids, la.flat, la.experts, reinterpret_cast<int*>(lds), lg, blockIdx.x == 0, la.counts,
                la.offsets, la.perm, la.pos, chunks, n_chunks);
    nch = lg.nch;
  } else {
    nch = *n_chunks;
  }
  for (int64_t item = blockIdx.x;; item += gridDim.x) {
    const int64_t jq = item / nrt;
    const int jc = jq < max_chunks ? (int)jq : max_chunks;  // max_chunks: past the list
    const int rt = (int)(item % nrt);
    int e, p0, rows;
    const uint16_t* xrow[2];
    if constexpr (LOCAL) {
      if (jc >= nch) break;
      const uint32_t ci = lg.chunk[jc];
      e = (int)(ci >> 16);
      p0 = lg.off[e] + (int)(ci & 0xffffu) * kChunkRows;
      rows = lg.off[e + 1] - p0 < kChunkRows ? lg.off[e + 1] - p0 : kChunkRows;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = 4 * wave + 2 * j + (lane >> 5);
        xrow[j] = x + (int64_t)(lg.perm[p0 + (r < rows ? r : rows - 1)] / la.top_k) * hidden;
      }
    } else {
      // The record's loads do not wait for the count: its index is clamped
      // into the list's allocation.
      const int32_t* rec = chunks + (size_t)(jc < max_chunks ? jc : max_chunks - 1) * kChunkInts;
      e = rec[0];
      p0 = rec[1];
      rows = rec[2];
      if (jc >= nch) break;
#pragma unroll
      for (int j = 0; j < 2; ++j) xrow[j] = x + (int64_t)rec[4 + 4 * wave + 2 * j + (lane >> 5)] * hidden;
    }
    const int es = slot_table ? slot_table[e] : e;  // where expert e's matrices sit in the pools
    const uint8_t* wrow =
        (wave >= KS ? w_up + es * stride_up : w_gate + es * stride_gate) + (size_t)rt * nkt * kTileBytes;
    f32x16 acc_a = {}, acc_b = {};
    expert_rounds<KS>(wrow, nkt, hidden, slot, xrow, wave, lane, lds, acc_a, acc_b);
    float* red = reinterpret_cast<float*>(lds);
    store_partials(red, wave, lane, acc_a, acc_b);
    __syncthreads();
    // Thread t: accumulator elements i0 + 8 q (i0 = t / 64) of lane t % 64,
    // gate and up.  (t is opaque here, so that the addresses derived from it
    // are formed per item instead of being kept, spilled, across the rounds.)
    int t = (int)threadIdx.x;
    asm volatile("" : "+v"(t));
    const int l = t & 63, i0 = t >> 6;
    const int slots = nkt < KS ? nkt : KS;
    const float sg = scale_gate[e], su = scale_up[e];
    const int tok = l & 31;
    if (tok < rows) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = i0 + 8 * q;
        float g = 0.0f, u = 0.0f;
#pragma unroll
        for (int sl = 0; sl < KS; ++sl) {  // all slots' reads issued together (clamped), added in slot order
          const int sc = sl < slots ? sl : slots - 1;
          const float gs = red[(32 * sc + i) * 64 + l], us = red[(32 * (KS + sc) + i) * 64 + l];
          if (sl < slots) {
            g += gs;
            u += us;
          }
        }
        const int row = rt * 64 + acc_row(i >> 4, i & 15, l);
        if (row < inter) {
          const int64_t at = (int64_t)(p0 + tok) * inter + row;
          const float gv = g * sg, uv = u * su;
          h[at] = to_bf16((gv / (1.0f + expf(-gv))) * uv);
          if (dbg_gate) dbg_gate[at] = gv;
          if (dbg_up) dbg_up[at] = uv;
        }
      }
    }
    __syncthreads();  // the sums are read before the next item stages into the LDS
  }
}

// Down.  Workgroup (chunk, row tiles 4 q .. 4 q + 3): wavefront w takes
// row tile 4 q + w / 2 at k slot w % 2; d = s_d Wd h (fp32) for those rows.
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void down_kernel(
    const uint16_t* __restrict__ hin, const int32_t* __restrict__ chunks, const int32_t* __restrict__ n_chunks,
    int max_chunks, int hidden, int inter, const uint8_t* __restrict__ w_down, size_t stride_down,
    const int32_t* __restrict__ slot_table, const float* __restrict__ scale_down, float* __restrict__ d) {
  constexpr int KS = 2;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kExpertLds];
  const int nrt = (hidden + 63) / 64;
  const int ngrp = (nrt + 3) / 4;
  const int nkt = (inter + 255) / 256;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int slot = wave % KS;
  const int nch = *n_chunks;
  for (int64_t item = blockIdx.x;; item += gridDim.x) {
    const int64_t jq = item / ngrp;
    const int jc = jq < max_chunks ? (int)jq : max_chunks;  // max_chunks: past the list
    const int grp = (int)(item % ngrp);
    const int32_t* rec = chunks + (size_t)(jc < max_chunks ? jc : max_chunks - 1) * kChunkInts;
    const int e = rec[0], p0 = rec[1], rows = rec[2];
    if (jc >= nch) break;
    const int rt = 4 * grp + wave / KS;
    const bool has_rows = rt < nrt;
    const int es = slot_table ? slot_table[e] : e;
    const uint8_t* wrow = has_rows ? w_down + es * stride_down + (size_t)rt * nkt * kTileBytes : nullptr;
    // The chunk's rows of h are contiguous (the last repeated past the end).
    const uint16_t* xrow[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int srow = 4 * wave + 2 * j + (lane >> 5);
      xrow[j] = hin + (int64_t)(p0 + (srow < rows ? srow : rows - 1)) * inter;
    }
    f32x16 acc_a = {}, acc_b = {};
    expert_rounds<KS>(wrow, nkt, inter, slot, xrow, wave, lane, lds, acc_a, acc_b);
    float* red = reinterpret_cast<float*>(lds);
    store_partials(red, wave, lane, acc_a, acc_b);
    __syncthreads();
    // The slot-0 wavefront of each row tile adds its tile's slots in order.
    const int tok = lane & 31;
    if (slot == 0 && has_rows && tok < rows) {
      const int slots = nkt < KS ? nkt : KS;
      const float sd = scale_down[e];
      float* drow = d + (int64_t)(p0 + tok) * hidden;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          float v[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int i = 16 * hh + 4 * e4 + c;
            float acc = 0.0f;
#pragma unroll
            for (int sl = 0; sl < KS; ++sl) {  // reads issued together (clamped), added in slot order
              const float v = red[(32 * (wave + (sl < slots ? sl : slots - 1)) + i) * 64 + lane];
              if (sl < slots) acc += v;
            }
            v[c] = acc * sd;
          }
          const int row = rt * 64 + acc_row(hh, 4 * e4, lane);
          if (row + 4 <= hidden) {
            *reinterpret_cast<f32x4*>(drow + row) = f32x4{v[0], v[1], v[2], v[3]};
          } else {
            for (int c = 0; c < 4; ++c)
              if (row + c < hidden) drow[row + c] = v[c];
          }
        }
      }
    }
    __syncthreads();  // the sums are read before the next item stages into the LDS
  }
}

__global__ __launch_bounds__(256) void scatter_kernel(const float* __restrict__ d, const float* __restrict__ g,
                                                      const int32_t* __restrict__ pos, int64_t tokens, int top_k,
                                                      int hidden, void* __restrict__ y, int y_bf16) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= tokens * hidden) return;
  const int64_t t = i / hidden;
  const int o = (int)(i % hidden);
  // Sixteen selections per round: their positions and weights load together,
  // then their d values together, so a round costs two memory round trips
  // whatever top_k is (a plain loop waits twice per selection).  The sum is
  // still taken in j order; padding entries re-read the last selection and
  // are not added.
  float acc = 0.0f;
  for (int j0 = 0; j0 < top_k; j0 += 16) {
    int pj[16];
    float gj[16], dj[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int64_t f = t * top_k + (j0 + u < top_k ? j0 + u : top_k - 1);
      pj[u] = pos[f];
      gj[u] = g[f];
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) dj[u] = d[(int64_t)pj[u] * hidden + o];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (j0 + u < top_k) acc = fmaf(gj[u], dj[u], acc);
  }
  if (y_bf16) static_cast<uint16_t*>(y)[i] = to_bf16(acc);
  else static_cast<float*>(y)[i] = acc;
}

// Copies of whole expert matrices from pinned host memory into device cache
// slots, read by the GPU over PCIe: one launch for all of a call's copies, so
// that many 16-byte reads are in flight at once (a DMA transfer per matrix
// pays a set-up cost per copy).  Entry j copies words16[j] 16-byte words.
constexpr int kCopiesPerLaunch = 96;
constexpr int kCopyWordsPerBlock = 256 * 8;  // 32 KB per workgroup
struct CopyList {
  int count;
  int blocks_per_entry;
  const u32x4* src[kCopiesPerLaunch];
  u32x4* dst[kCopiesPerLaunch];
  int64_t words16[kCopiesPerLaunch];
};

__global__ __launch_bounds__(256) void expert_copy_kernel(const CopyList l) {
  const int entry = blockIdx.x / l.blocks_per_entry;
  const int64_t w0 = (int64_t)(blockIdx.x % l.blocks_per_entry) * kCopyWordsPerBlock;
  int j = 0;
#pragma unroll
  for (int i = 1; i < kCopiesPerLaunch; ++i)
    if (i == entry) j = i;  // static indices into the argument arrays
  const u32x4* src = nullptr;
  u32x4* dst = nullptr;
  int64_t n = 0;
#pragma unroll
  for (int i = 0; i < kCopiesPerLaunch; ++i)
    if (i == j) {
      src = l.src[i];
      dst = l.dst[i];
      n = l.words16[i];
    }
  u32x4 v[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int64_t w = w0 + u * 256 + threadIdx.x;
    if (w < n) v[u] = src[w];
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int64_t w = w0 + u * 256 + threadIdx.x;
    if (w < n) dst[w] = v[u];
  }
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Compute units of the current device (queried once per device).
int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Upper bound on the work-list length: every active expert (at most
// min(experts, tokens * top_k)) has one partial chunk, plus the full ones.
int64_t max_chunks(int64_t tokens, int64_t experts, int64_t top_k) {
  const int64_t flat = tokens * top_k;
  return (experts < flat ? experts : flat) + flat / kChunkRows;
}

struct MoeWs {
  int32_t* pos;
  uint16_t* h;
  float* d;
  int32_t* chunks;
  int32_t* n_chunks;
};

MoeWs carve(void* ws, int64_t tokens, int64_t experts, int64_t top_k, int64_t hidden, int64_t inter, size_t* total) {
  uint8_t* p = static_cast<uint8_t*>(ws);
  size_t off = 0;
  // (ws == nullptr: only the total is wanted; no pointer arithmetic on it.)
  auto at = [&](size_t o) { return p ? p + o : nullptr; };
  MoeWs w;
  const int64_t f = tokens * top_k;
  w.pos = reinterpret_cast<int32_t*>(at(off)); off = align256(off + (size_t)f * 4);
  w.h = reinterpret_cast<uint16_t*>(at(off)); off = align256(off + (size_t)f * inter * 2);
  w.d = reinterpret_cast<float*>(at(off)); off = align256(off + (size_t)f * hidden * 4);
  w.chunks = reinterpret_cast<int32_t*>(at(off)); off = align256(off + (size_t)max_chunks(tokens, experts, top_k) * kChunkInts * 4);
  w.n_chunks = reinterpret_cast<int32_t*>(at(off)); off = align256(off + 16);
  if (total) *total = off;
  return w;
}

}  // namespace

int64_t moe_max_experts() { return kMaxExperts; }

hipError_t launch_expert_copies(const void* const* src, void* const* dst, const size_t* bytes, int count,
                                hipStream_t s) {
  for (int c0 = 0; c0 < count; c0 += kCopiesPerLaunch) {
    CopyList l = {};
    l.count = count - c0 < kCopiesPerLaunch ? count - c0 : kCopiesPerLaunch;
    int64_t most = 0;
    for (int i = 0; i < l.count; ++i) {
      l.src[i] = static_cast<const u32x4*>(src[c0 + i]);
      l.dst[i] = static_cast<u32x4*>(dst[c0 + i]);
      l.words16[i] = (int64_t)(bytes[c0 + i] / 16);
      if (l.words16[i] > most) most = l.words16[i];
    }
    l.blocks_per_entry = (int)((most + kCopyWordsPerBlock - 1) / kCopyWordsPerBlock);
    if (l.blocks_per_entry == 0) continue;
    hipLaunchKernelGGL(expert_copy_kernel, dim3((unsigned)(l.count * l.blocks_per_entry)), dim3(256), 0, s, l);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

size_t moe_workspace_bytes(int64_t tokens, int64_t experts, int64_t top_k, int64_t hidden, int64_t inter) {
  size_t total = 0;
  carve(nullptr, tokens, experts, top_k, hidden, inter, &total);
  return total;
}

namespace {
// Whether the gate/up workgroups group the batch themselves.
bool local_grouping(const MoeLaunch& a) {
  return a.slot_table == nullptr && a.tokens * a.top_k <= kLocalFlat && a.experts <= kLocalExperts;
}

// Expert GEMMs and scatter; with `local`, gate/up also groups the routed rows.
hipError_t launch_experts(const MoeLaunch& a, bool local, hipStream_t s) {
  if (a.tokens == 0) return hipSuccess;
  MoeWs w = carve(a.ws, a.tokens, a.experts, a.top_k, a.hidden, a.inter, nullptr);
  const int64_t flat = a.tokens * a.top_k;
  hipError_t err = hipSuccess;
  // The expert GEMMs run on persistent grids of at most two workgroups per
  // CU (what fits at once), which walk the work list's items (chunk, output
  // rows) with a stride; the list's actual length is read on the device.
  const int64_t mch = max_chunks(a.tokens, a.experts, a.top_k);
  const int64_t resident = 2 * (int64_t)cu_count();
  const int64_t nrt_i = (a.inter + 63) / 64;
  const int64_t gu_items = mch * nrt_i;
  const dim3 gu_grid((unsigned)(gu_items < resident ? gu_items : resident));
  const LocalArgs la{a.ids, (int)flat, (int)a.experts, (int)a.top_k, a.counts, a.offsets, a.perm, w.pos};
  if (local)
    hipLaunchKernelGGL(gate_up_kernel<true>, gu_grid, dim3(64 * kExpertWaves), 0, s, a.x, w.chunks, w.n_chunks,
                       (int)mch, (int)a.hidden, (int)a.inter, a.w_gate, a.w_up, a.stride_gate, a.stride_up,
                       a.slot_table, a.scale_gate, a.scale_up, w.h, a.dbg_gate, a.dbg_up, la);
  else
    hipLaunchKernelGGL(gate_up_kernel<false>, gu_grid, dim3(64 * kExpertWaves), 0, s, a.x, w.chunks, w.n_chunks,
                       (int)mch, (int)a.hidden, (int)a.inter, a.w_gate, a.w_up, a.stride_gate, a.stride_up,
                       a.slot_table, a.scale_gate, a.scale_up, w.h, a.dbg_gate, a.dbg_up, la);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int64_t grp_h = ((a.hidden + 63) / 64 + 3) / 4;
  const int64_t dn_items = mch * grp_h;
  float* d = a.dbg_down ? a.dbg_down : w.d;
  hipLaunchKernelGGL(down_kernel, dim3((unsigned)(dn_items < resident ? dn_items : resident)),
                     dim3(64 * kExpertWaves), 0, s, w.h, w.chunks, w.n_chunks, (int)mch, (int)a.hidden,
                     (int)a.inter, a.w_down, a.stride_down, a.slot_table, a.scale_down, d);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int64_t outs = a.tokens * a.hidden;
  hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)((outs + 255) / 256)), dim3(256), 0, s, d, a.g, w.pos, a.tokens,
                     (int)a.top_k, (int)a.hidden, a.y, a.y_bf16 ? 1 : 0);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (a.dbg_h) {
    err = hipMemcpyAsync(a.dbg_h, w.h, (size_t)flat * a.inter * 2, hipMemcpyDeviceToDevice, s);
  }
  return err;
}

hipError_t launch_route(const MoeLaunch& a, hipStream_t s) {
#define NVFP4_R(NPL)                                                                                        \
  hipLaunchKernelGGL(route_kernel<NPL>, dim3((unsigned)a.tokens), dim3(64), 0, s, a.logits, a.tokens, (int)a.experts, \
                     (int)a.top_k, a.ids, a.g)
  if (a.experts <= 512) NVFP4_R(8);
  else if (a.experts <= 1024) NVFP4_R(16);
  else NVFP4_R(32);
#undef NVFP4_R
  return hipGetLastError();
}
}  // namespace

hipError_t launch_moe_routing(const MoeLaunch& a, hipStream_t s) {
  if (a.tokens == 0) return hipSuccess;
  MoeWs w = carve(a.ws, a.tokens, a.experts, a.top_k, a.hidden, a.inter, nullptr);
  const int64_t flat = a.tokens * a.top_k;
  hipError_t err = launch_route(a, s);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(group_kernel, dim3(1), dim3(1024), 0, s, a.ids, (int)flat, (int)a.experts, (int)a.top_k,
                     a.counts, a.offsets, a.perm, w.pos, w.chunks, w.n_chunks);
  return hipGetLastError();
}

hipError_t launch_moe_experts(const MoeLaunch& a, hipStream_t s) { return launch_experts(a, false, s); }

hipError_t launch_moe(const MoeLaunch& a, hipStream_t s) {
  if (a.tokens == 0) return hipSuccess;
  if (local_grouping(a)) {
    const hipError_t err = launch_route(a, s);
    return err != hipSuccess ? err : launch_experts(a, true, s);
  }
  const hipError_t err = launch_moe_routing(a, s);
  return err != hipSuccess ? err : launch_experts(a, false, s);
}

}  // namespace nvfp4
