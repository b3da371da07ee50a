// Ceiling probes for the benchmark: what the chip sustains on this machine for
// the two resources the products are bound by, measured the way the products
// use them.  Not part of the product library (built as libnvfp4_probes.so).
//
//  - probe_hbm_read: a streaming read of a buffer in the packed weights' unit,
//    one 9216-byte tile per wavefront with all of a lane's nine 16-byte loads
//    issued at once, non-temporal -- the GEMV's access pattern without its
//    arithmetic.  (Non-temporal loads stream faster here than ordinary ones:
//    measured, ~6 % at 186 MB and ~10 % at 400 MB.)
//  - probe_mfma_bf16: v_mfma_f32_32x32x16_bf16 issued back to back from
//    registers, 16 independent accumulators per wavefront, operands drawn from
//    a caller buffer of random bits (the matrix cores draw more power, and the
//    chip clocks lower, with random operands than with constant ones).
//  - probe_mfma_fp4: the same with the scaled FP4 instruction
//    v_mfma_scale_f32_32x32x64_f8f6f4 (E2M1 operands, E8M0 scales).
//  - probe_mfma_bf16_once / probe_mfma_fp4_once / probe_dot2_once: single
//    instructions on given operands, so that tests can measure how an
//    instruction rounds.
// Each kernel folds what it computed into one word and stores it only if it
// equals a caller value that it never equals in practice, so nothing is
// optimised away and nothing is written.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int kTileBytes = 9216;

__global__ __launch_bounds__(256) void read_kernel(const uint8_t* __restrict__ buf, int64_t tiles, unsigned magic,
                                                   unsigned* __restrict__ out) {
  const int64_t tile = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tile >= tiles) return;
  const int lane = threadIdx.x & 63;
  const uint8_t* t = buf + tile * kTileBytes + lane * 16;
  u32x4 v[9];
#pragma unroll
  for (int c = 0; c < 9; ++c) v[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(t + c * 1024));
  unsigned x = 0;
#pragma unroll
  for (int c = 0; c < 9; ++c) x ^= v[c][0] ^ v[c][1] ^ v[c][2] ^ v[c][3];
  if (x == magic) out[tile] = x;
}

__global__ __launch_bounds__(256, 1) void mfma_bf16_kernel(const u32x4* __restrict__ rnd, int iters, unsigned magic,
                                                           float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const u32x4* r = rnd + ((blockIdx.x * 4 + (threadIdx.x >> 6)) & 255) * 64 * 6 + lane;
  bf16x8 a[4], b[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = __builtin_bit_cast(bf16x8, r[64 * i]);
#pragma unroll
  for (int i = 0; i < 2; ++i) b[i] = __builtin_bit_cast(bf16x8, r[64 * (4 + i)]);
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[(i + j) & 1], acc[i][j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[i][j][e];
  if (__float_as_uint(s) == magic) out[blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256, 1) void mfma_fp4_kernel(const u32x4* __restrict__ rnd, int iters, unsigned magic,
                                                          float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const u32x4* r = rnd + ((blockIdx.x * 4 + (threadIdx.x >> 6)) & 255) * 64 * 6 + lane;
  v8i a[4], b[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 q = r[64 * i];
    a[i] = v8i{(int)q[0], (int)q[1], (int)q[2], (int)q[3], 0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const u32x4 q = r[64 * (4 + i)];
    b[i] = v8i{(int)q[0], (int)q[1], (int)q[2], (int)q[3], 0, 0, 0, 0};
  }
  // E8M0 scales near 2^0 (bytes 120..134), from the random bits.
  const int sa = 120 + (int)(r[0][0] % 15u), sb = 120 + (int)(r[64][1] % 15u);
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[(i + j) & 1], acc[i][j], 4, 4, 0, sa, 0, sb);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[i][j][e];
  if (__float_as_uint(s) == magic) out[blockIdx.x * 256 + threadIdx.x] = s;
}

// One matrix instruction per wavefront, on given operands, for checking how
// the instruction rounds (the error bounds of the products rest on it).
// Problem p: A [32][K] and B (as [32 columns][K]), C and D [32][32] fp32
// row-major.  Lane l supplies row (A) / column (B) l % 32 at k offsets
// (K / 2) * (l / 32) .. + K / 2 - 1, and holds accumulator element e of
// row 8 (e / 4) + 4 (l / 32) + e % 4, column l % 32.
__device__ __forceinline__ int acc_row_of(int e, int lane) { return 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); }

__global__ __launch_bounds__(64) void mfma_bf16_once_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                            const float* __restrict__ C, float* __restrict__ D) {
  const int p = blockIdx.x, l = threadIdx.x, r = l & 31, h = l >> 5;
  const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(A + ((size_t)p * 32 + r) * 16 + 8 * h));
  const bf16x8 b = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(B + ((size_t)p * 32 + r) * 16 + 8 * h));
  f32x16 c;
#pragma unroll
  for (int e = 0; e < 16; ++e) c[e] = C[((size_t)p * 32 + acc_row_of(e, l)) * 32 + r];
  const f32x16 d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
#pragma unroll
  for (int e = 0; e < 16; ++e) D[((size_t)p * 32 + acc_row_of(e, l)) * 32 + r] = d[e];
}

// FP4 operands: A and B as [32][32] bytes per problem (64 E2M1 codes along k,
// low nibble first), E8M0 scales SA / SB [32][2] (per row or column and
// 32-k half).
__global__ __launch_bounds__(64) void mfma_fp4_once_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
                                                           const uint8_t* __restrict__ SA, const uint8_t* __restrict__ SB,
                                                           const float* __restrict__ C, float* __restrict__ D) {
  const int p = blockIdx.x, l = threadIdx.x, r = l & 31, h = l >> 5;
  const u32x4 qa = *reinterpret_cast<const u32x4*>(A + ((size_t)p * 32 + r) * 32 + 16 * h);
  const u32x4 qb = *reinterpret_cast<const u32x4*>(B + ((size_t)p * 32 + r) * 32 + 16 * h);
  const v8i a = v8i{(int)qa[0], (int)qa[1], (int)qa[2], (int)qa[3], 0, 0, 0, 0};
  const v8i b = v8i{(int)qb[0], (int)qb[1], (int)qb[2], (int)qb[3], 0, 0, 0, 0};
  const int sa = SA[((size_t)p * 32 + r) * 2 + h], sb = SB[((size_t)p * 32 + r) * 2 + h];
  f32x16 c;
#pragma unroll
  for (int e = 0; e < 16; ++e) c[e] = C[((size_t)p * 32 + acc_row_of(e, l)) * 32 + r];
  const f32x16 d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 0, sa, 0, sb);
#pragma unroll
  for (int e = 0; e < 16; ++e) D[((size_t)p * 32 + acc_row_of(e, l)) * 32 + r] = d[e];
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// One v_dot2_f32_bf16 per thread: d[i] = c[i] + a[2i] b[2i] + a[2i+1] b[2i+1].
__global__ __launch_bounds__(256) void dot2_once_kernel(const uint32_t* __restrict__ a, const uint32_t* __restrict__ b,
                                                        const float* __restrict__ c, float* __restrict__ d, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  d[i] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a[i]), __builtin_bit_cast(bf16x2, b[i]), c[i], false);
}

}  // namespace

extern "C" {

// n independent v_dot2_f32_bf16 (a, b: bf16 pairs as uint32, c, d: fp32).
int probe_dot2_once(const uint32_t* a, const uint32_t* b, const float* c, float* d, int n, void* stream) {
  if (!a || !b || !c || !d || n <= 0) return 1;
  dot2_once_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream>>>(a, b, c, d, n);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// `count` independent D = A B + C by one v_mfma_f32_32x32x16_bf16 each
// (A [count][32][16] bf16, B [count][32 columns][16] bf16, C / D [count][32][32]).
int probe_mfma_bf16_once(const uint16_t* A, const uint16_t* B, const float* C, float* D, int count, void* stream) {
  if (!A || !B || !C || !D || count <= 0) return 1;
  mfma_bf16_once_kernel<<<dim3((unsigned)count), dim3(64), 0, (hipStream_t)stream>>>(A, B, C, D);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// `count` independent D = (A 2^(SA-127)) (B 2^(SB-127)) + C by one
// v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 operands each.
int probe_mfma_fp4_once(const uint8_t* A, const uint8_t* B, const uint8_t* SA, const uint8_t* SB, const float* C, float* D,
                        int count, void* stream) {
  if (!A || !B || !SA || !SB || !C || !D || count <= 0) return 1;
  mfma_fp4_once_kernel<<<dim3((unsigned)count), dim3(64), 0, (hipStream_t)stream>>>(A, B, SA, SB, C, D);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Reads `bytes` (a multiple of 9216, 16-byte aligned) of `buf`; `out` must
// hold bytes / 9216 words (written only if a tile's fold equals `magic`).
int probe_hbm_read(const void* buf, int64_t bytes, unsigned magic, unsigned* out, void* stream) {
  if (!buf || !out || bytes <= 0 || bytes % kTileBytes != 0 || (reinterpret_cast<uintptr_t>(buf) & 15u)) return 1;
  const int64_t tiles = bytes / kTileBytes;
  read_kernel<<<dim3((unsigned)((tiles + 3) / 4)), dim3(256), 0, (hipStream_t)stream>>>(
      static_cast<const uint8_t*>(buf), tiles, magic, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// `wgs` workgroups of four wavefronts, each issuing 16 * iters matrix
// instructions; `rnd` holds 256 * 6 * 1024 bytes of random bits, `out`
// 256 * wgs floats (written only if a lane's fold equals `magic`).
// Flops: wgs * 4 * 16 * iters * 32768 (bf16) or * 131072 (fp4).
int probe_mfma_bf16(const void* rnd, int wgs, int iters, unsigned magic, float* out, void* stream) {
  if (!rnd || !out || wgs <= 0 || iters <= 0) return 1;
  mfma_bf16_kernel<<<dim3((unsigned)wgs), dim3(256), 0, (hipStream_t)stream>>>(static_cast<const u32x4*>(rnd), iters,
                                                                             magic, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int probe_mfma_fp4(const void* rnd, int wgs, int iters, unsigned magic, float* out, void* stream) {
  if (!rnd || !out || wgs <= 0 || iters <= 0) return 1;
  mfma_fp4_kernel<<<dim3((unsigned)wgs), dim3(256), 0, (hipStream_t)stream>>>(static_cast<const u32x4*>(rnd), iters,
                                                                            magic, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
