// a4-a8: the top-k routed mixture-of-experts layer on NVFP4 experts.
//
// Each token is routed to `top_k` of `experts` experts and only the routed
// experts' weights are read (CHImp-Alpha-v1.0 model card, "How it fits on one
// GPU": 10 of 512 experts per token).  Five launches on the caller's stream:
//   1. route    one wavefront per token: top_k rounds of a wavefront-wide
//               (logit desc, id asc) argmax, then the softmax over the
//               selected logits (fp32);
//   2. group    one workgroup: expert histogram, exclusive scan, the stable
//               counting sort of the flat (t*top_k + j) indices by expert, and
//               the ascending list of active experts -- integer only, so
//               bit-exact and independent of scheduling;
//   3. gate/up  per (active expert, pair of 64-row tiles): the skinny core on
//               the expert's gate and up tiles, activation rows gathered
//               through perm, then h = bf16(silu(s_g Wg x) * (s_u Wu x));
//   4. down     per (active expert, four 64-row tiles): d = s_d Wd h (fp32);
//   5. scatter  y[t] = sum_j g[t][j] * d[pos(t, j)], j ascending.
// Launch grids cover the worst case (min(experts, tokens*top_k) active
// experts); workgroups past the active count return at once.
#include "device_common.h"
#include "launchers.h"
#include "skinny_core.h"

namespace nvfp4 {
namespace {

constexpr int kMaxExperts = 2048;
constexpr int kMaxTopK = 64;

__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  if (ai < 0) return false;
  if (bi < 0) return true;
  return av > bv || (av == bv && ai < bi);
}

template <int NPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int64_t tokens, int experts,
                                                    int top_k, int32_t* __restrict__ ids, float* __restrict__ g) {
  __shared__ float s_val[4][kMaxTopK];
  __shared__ int s_id[4][kMaxTopK];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= tokens) return;
  const float* lt = logits + t * experts;
  float v[NPL];
  uint32_t avail = 0;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < experts ? lt[e] : 0.0f;
    if (e < experts) avail |= 1u << i;
  }
  for (int r = 0; r < top_k; ++r) {
    float bv = 0.0f;
    int bi = -1;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = lane + 64 * i;
      if (((avail >> i) & 1u) && better(v[i], e, bv, bi)) { bv = v[i]; bi = e; }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if (bi >= 0 && lane == (bi & 63)) avail &= ~(1u << (bi >> 6));
    if (lane == 0) { s_val[wave][r] = bv; s_id[wave][r] = bi; }
  }
  // Lane 0 wrote s_val / s_id and lane 0 reads them: no barrier needed.
  if (lane == 0) {
    const float l0 = s_val[wave][0];
    float sum = 0.0f;
    for (int j = 0; j < top_k; ++j) sum += expf(s_val[wave][j] - l0);
    for (int j = 0; j < top_k; ++j) {
      ids[t * top_k + j] = s_id[wave][j];
      g[t * top_k + j] = expf(s_val[wave][j] - l0) / sum;
    }
  }
}

// Exclusive scan of `in[0..n)` (n <= 2048) by a 1024-thread workgroup; returns the total.
__device__ int block_exclusive_scan(const int* in, int* out, int n, int* s_tmp /* [1024] */) {
  const int tid = threadIdx.x;
  const int a0 = 2 * tid < n ? in[2 * tid] : 0;
  const int a1 = 2 * tid + 1 < n ? in[2 * tid + 1] : 0;
  s_tmp[tid] = a0 + a1;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = tid >= off ? s_tmp[tid - off] : 0;
    __syncthreads();
    s_tmp[tid] += v;
    __syncthreads();
  }
  const int incl = s_tmp[tid];
  const int excl = incl - (a0 + a1);
  if (2 * tid < n) out[2 * tid] = excl;
  if (2 * tid + 1 < n) out[2 * tid + 1] = excl + a0;
  const int total = s_tmp[1023];
  __syncthreads();
  return total;
}

__global__ __launch_bounds__(1024) void group_kernel(const int32_t* __restrict__ ids, int total, int experts,
                                                     int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ perm, int32_t* __restrict__ pos,
                                                     int32_t* __restrict__ active, int32_t* __restrict__ n_active) {
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_off[kMaxExperts];
  __shared__ int s_run[kMaxExperts];
  __shared__ int s_tmp[1024];
  __shared__ int s_chunk[1024];
  const int tid = threadIdx.x;
  for (int e = tid; e < experts; e += 1024) { s_cnt[e] = 0; s_run[e] = 0; }
  __syncthreads();
  for (int f = tid; f < total; f += 1024) atomicAdd(&s_cnt[ids[f]], 1);
  __syncthreads();
  const int all = block_exclusive_scan(s_cnt, s_off, experts, s_tmp);
  for (int e = tid; e < experts; e += 1024) {
    counts[e] = s_cnt[e];
    offsets[e] = s_off[e];
  }
  if (tid == 0) offsets[experts] = all;
  // Active experts, ascending: scan of (count > 0).
  for (int e = tid; e < experts; e += 1024) s_run[e] = s_cnt[e] > 0 ? 1 : 0;
  __syncthreads();
  const int na = block_exclusive_scan(s_run, s_run, experts, s_tmp);
  for (int e = tid; e < experts; e += 1024)
    if (s_cnt[e] > 0) active[s_run[e]] = e;
  if (tid == 0) *n_active = na;
  __syncthreads();
  for (int e = tid; e < experts; e += 1024) s_run[e] = 0;
  __syncthreads();
  // Stable counting sort, 1024 flat indices at a time.
  for (int base = 0; base < total; base += 1024) {
    const int f = base + tid;
    const int e = f < total ? ids[f] : -1;
    s_chunk[tid] = e;
    __syncthreads();
    if (e >= 0) {
      int rank = 0;
      for (int j = 0; j < tid; ++j) rank += s_chunk[j] == e ? 1 : 0;
      const int p = s_off[e] + s_run[e] + rank;
      perm[p] = f;
      pos[f] = p;
    }
    __syncthreads();
    if (e >= 0) atomicAdd(&s_run[e], 1);
    __syncthreads();
  }
}

// a6: per workgroup (active expert a, row pair j): waves 0/1 take gate row
// tiles 2j, 2j+1 and waves 2/3 the same up row tiles, all over the whole
// hidden dimension with one shared activation tile per k tile; the up results
// go through LDS to the gate waves, which form h = bf16(silu(G) * U).
template <bool KFULL>
__global__ __launch_bounds__(256, 1) void gate_up_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ perm, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ active, const int32_t* __restrict__ n_active, int top_k, int hidden, int inter,
    const uint8_t* __restrict__ w_gate, const uint8_t* __restrict__ w_up, size_t stride_gate, size_t stride_up,
    const float* __restrict__ scale_gate, const float* __restrict__ scale_up, uint16_t* __restrict__ h,
    float* __restrict__ dbg_gate, float* __restrict__ dbg_up) {
  __shared__ __attribute__((aligned(16))) uint8_t xb0[kXTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t xb1[kXTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t xb2[kXTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t xb3[kXTileBytes];
  __shared__ float lds_u[2][32][65];
  const int nrt = (inter + 63) / 64;
  const int npairs = (nrt + 1) / 2;
  const int a = blockIdx.x / npairs;
  const int pair = blockIdx.x % npairs;
  if (a >= *n_active) return;
  const int e = active[a];
  const int p0 = offsets[e], p1 = offsets[e + 1];
  const int nkt = (hidden + 255) / 256;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const bool is_up = wave >= 2;
  const int rt = 2 * pair + (wave & 1);
  // A wavefront past the last row tile streams the last one (not stored).
  const uint8_t* wrow = (is_up ? w_up + e * stride_up : w_gate + e * stride_gate) +
                        (size_t)(rt < nrt ? rt : nrt - 1) * nkt * kTileBytes;
  const float sg = scale_gate[e], su = scale_up[e];
  const int tok = lane & 31;
  for (int c0 = p0; c0 < p1; c0 += 32) {
    // Activation rows of this chunk, gathered through perm; rows past the
    // expert's last repeat it (their outputs are not stored).
    const uint16_t* rowp[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ps = c0 + stage_row(wave, j, lane);
      rowp[j] = x + (int64_t)(perm[ps < p1 ? ps : p1 - 1] / top_k) * hidden;
    }
    f32x16 acc_a = {}, acc_b = {};
    skinny_stream<4, KFULL>(wrow, 0, nkt, hidden, rowp, xb0, xb1, xb2, xb3, wave, lane, acc_a, acc_b);
    if (is_up) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        lds_u[wave & 1][tok][acc_row(0, i, lane)] = acc_a[i] * su;
        lds_u[wave & 1][tok][acc_row(1, i, lane)] = acc_b[i] * su;
      }
    }
    __syncthreads();
    const int p = c0 + tok;
    if (!is_up && rt < nrt && p < p1) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = acc_row(hh, i, lane);
          const int row = rt * 64 + r;
          if (row < inter) {
            const float gv = (hh ? acc_b[i] : acc_a[i]) * sg;
            const float uv = lds_u[wave & 1][tok][r];
            const float hv = (gv / (1.0f + expf(-gv))) * uv;
            h[(int64_t)p * inter + row] = to_bf16(hv);
            if (dbg_gate) dbg_gate[(int64_t)p * inter + row] = gv;
            if (dbg_up) dbg_up[(int64_t)p * inter + row] = uv;
          }
        }
      }
    }
    __syncthreads();  // lds_u is rewritten by the next chunk
  }
}

// a7: per workgroup (active expert a, row quad j): four down row tiles over the
// expert width, activation rows = the expert's rows of h.
template <bool KFULL>
__global__ __launch_bounds__(256, 1) void down_kernel(const uint16_t* __restrict__ h,
                                                      const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ active,
                                                      const int32_t* __restrict__ n_active, int hidden, int inter,
                                                      const uint8_t* __restrict__ w_down, size_t stride_down,
                                                      const float* __restrict__ scale_down, float* __restrict__ d) {
  __shared__ __attribute__((aligned(16))) uint8_t xb0[kXTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t xb1[kXTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t xb2[kXTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t xb3[kXTileBytes];
  const int nrt = (hidden + 63) / 64;
  const int nquads = (nrt + 3) / 4;
  const int a = blockIdx.x / nquads;
  const int quad = blockIdx.x % nquads;
  if (a >= *n_active) return;
  const int e = active[a];
  const int p0 = offsets[e], p1 = offsets[e + 1];
  const int nkt = (inter + 255) / 256;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int rt = 4 * quad + wave;
  const uint8_t* wrow = w_down + e * stride_down + (size_t)(rt < nrt ? rt : nrt - 1) * nkt * kTileBytes;
  const float sd = scale_down[e];
  const int tok = lane & 31;
  for (int c0 = p0; c0 < p1; c0 += 32) {
    const uint16_t* rowp[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ps = c0 + stage_row(wave, j, lane);
      rowp[j] = h + (int64_t)(ps < p1 ? ps : p1 - 1) * inter;
    }
    f32x16 acc_a = {}, acc_b = {};
    skinny_stream<4, KFULL>(wrow, 0, nkt, inter, rowp, xb0, xb1, xb2, xb3, wave, lane, acc_a, acc_b);
    const int p = c0 + tok;
    if (rt < nrt && p < p1) {
      float* drow = d + (int64_t)p * hidden;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int row = rt * 64 + acc_row(hh, 4 * e4, lane);
          const f32x16& acc = hh ? acc_b : acc_a;
          if (row + 4 <= hidden) {
            *reinterpret_cast<f32x4*>(drow + row) =
                f32x4{acc[4 * e4] * sd, acc[4 * e4 + 1] * sd, acc[4 * e4 + 2] * sd, acc[4 * e4 + 3] * sd};
          } else {
            for (int i = 0; i < 4; ++i)
              if (row + i < hidden) drow[row + i] = acc[4 * e4 + i] * sd;
          }
        }
      }
    }
  }
}

__global__ __launch_bounds__(256) void scatter_kernel(const float* __restrict__ d, const float* __restrict__ g,
                                                      const int32_t* __restrict__ pos, int64_t tokens, int top_k,
                                                      int hidden, void* __restrict__ y, int y_bf16) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= tokens * hidden) return;
  const int64_t t = i / hidden;
  const int o = (int)(i % hidden);
  float acc = 0.0f;
  for (int j = 0; j < top_k; ++j) {
    const int64_t f = t * top_k + j;
    acc = fmaf(g[f], d[(int64_t)pos[f] * hidden + o], acc);
  }
  if (y_bf16) static_cast<uint16_t*>(y)[i] = to_bf16(acc);
  else static_cast<float*>(y)[i] = acc;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct MoeWs {
  int32_t* pos;
  int32_t* active;
  int32_t* n_active;
  uint16_t* h;
  float* d;
};

MoeWs carve(void* ws, int64_t tokens, int64_t experts, int64_t top_k, int64_t hidden, int64_t inter, size_t* total) {
  uint8_t* p = static_cast<uint8_t*>(ws);
  size_t off = 0;
  MoeWs w;
  const int64_t f = tokens * top_k;
  w.pos = reinterpret_cast<int32_t*>(p + off); off = align256(off + (size_t)f * 4);
  w.active = reinterpret_cast<int32_t*>(p + off); off = align256(off + (size_t)experts * 4);
  w.n_active = reinterpret_cast<int32_t*>(p + off); off = align256(off + 16);
  w.h = reinterpret_cast<uint16_t*>(p + off); off = align256(off + (size_t)f * inter * 2);
  w.d = reinterpret_cast<float*>(p + off); off = align256(off + (size_t)f * hidden * 4);
  if (total) *total = off;
  return w;
}

}  // namespace

int64_t moe_max_experts() { return kMaxExperts; }

size_t moe_workspace_bytes(int64_t tokens, int64_t experts, int64_t top_k, int64_t hidden, int64_t inter) {
  size_t total = 0;
  carve(nullptr, tokens, experts, top_k, hidden, inter, &total);
  return total;
}

hipError_t launch_moe(const MoeLaunch& a, hipStream_t s) {
  if (a.tokens == 0) return hipSuccess;
  MoeWs w = carve(a.ws, a.tokens, a.experts, a.top_k, a.hidden, a.inter, nullptr);
  const int64_t flat = a.tokens * a.top_k;
  const unsigned route_blocks = (unsigned)((a.tokens + 3) / 4);
  if (a.experts <= 512)
    hipLaunchKernelGGL(route_kernel<8>, dim3(route_blocks), dim3(256), 0, s, a.logits, a.tokens, (int)a.experts,
                       (int)a.top_k, a.ids, a.g);
  else if (a.experts <= 1024)
    hipLaunchKernelGGL(route_kernel<16>, dim3(route_blocks), dim3(256), 0, s, a.logits, a.tokens, (int)a.experts,
                       (int)a.top_k, a.ids, a.g);
  else
    hipLaunchKernelGGL(route_kernel<32>, dim3(route_blocks), dim3(256), 0, s, a.logits, a.tokens, (int)a.experts,
                       (int)a.top_k, a.ids, a.g);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(group_kernel, dim3(1), dim3(1024), 0, s, a.ids, (int)flat, (int)a.experts, a.counts, a.offsets,
                     a.perm, w.pos, w.active, w.n_active);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int64_t max_active = a.experts < flat ? a.experts : flat;
  const int64_t pairs_i = ((a.inter + 63) / 64 + 1) / 2;
  const dim3 gu_grid((unsigned)(max_active * pairs_i));
  if (a.hidden % kTileK == 0)
    gate_up_kernel<true><<<gu_grid, dim3(256), 0, s>>>(a.x, a.perm, a.offsets, w.active, w.n_active, (int)a.top_k,
                                                       (int)a.hidden, (int)a.inter, a.w_gate, a.w_up, a.stride_gate,
                                                       a.stride_up, a.scale_gate, a.scale_up, w.h, a.dbg_gate,
                                                       a.dbg_up);
  else
    gate_up_kernel<false><<<gu_grid, dim3(256), 0, s>>>(a.x, a.perm, a.offsets, w.active, w.n_active, (int)a.top_k,
                                                        (int)a.hidden, (int)a.inter, a.w_gate, a.w_up, a.stride_gate,
                                                        a.stride_up, a.scale_gate, a.scale_up, w.h, a.dbg_gate,
                                                        a.dbg_up);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int64_t nrt_h = (a.hidden + 63) / 64;
  const int64_t wgs_h = (nrt_h + 3) / 4;
  float* d = a.dbg_down ? a.dbg_down : w.d;
  const dim3 dn_grid((unsigned)(max_active * wgs_h));
  if (a.inter % kTileK == 0)
    down_kernel<true><<<dn_grid, dim3(256), 0, s>>>(w.h, a.offsets, w.active, w.n_active, (int)a.hidden,
                                                    (int)a.inter, a.w_down, a.stride_down, a.scale_down, d);
  else
    down_kernel<false><<<dn_grid, dim3(256), 0, s>>>(w.h, a.offsets, w.active, w.n_active, (int)a.hidden,
                                                     (int)a.inter, a.w_down, a.stride_down, a.scale_down, d);
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

}  // namespace nvfp4
