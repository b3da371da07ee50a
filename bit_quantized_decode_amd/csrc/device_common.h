// Device-side helpers shared by the NVFP4 kernels (gfx950 / CDNA4 only).
//
// Packed layout (the one form every product kernel reads).  An [N][K] NVFP4
// matrix is padded to Np = ceil(N/64)*64 rows and Kp = ceil(K/256)*256 columns
// (padding: code 0, scale byte 0x00, i.e. weight 0) and cut into tiles of
// 64 rows x 256 k, stored row-tile-major: tile (rt, kt) starts at
// (rt * (Kp/256) + kt) * 9216 bytes.  Inside a tile, with r = l % 32 and
// h = l / 32 for lane l of a wavefront:
//   bytes [1024*c + 16*l, +16), c = 0..7 (k = 256*kt + 32*c + [0, 32)):
//        dword 0: row r,      k offsets 8h + [0, 8)
//        dword 1: row 32 + r, k offsets 8h + [0, 8)
//        dword 2: row r,      k offsets 16 + 8h + [0, 8)
//        dword 3: row 32 + r, k offsets 16 + 8h + [0, 8)
//        (rows relative to the tile, k offsets relative to the chunk; 8 codes
//        per dword in canonical order, k even in the low nibble).  This is
//        the A-operand layout of v_mfma_f32_32x32x16_bf16 for two 32-row
//        halves and two k steps, so a 1 KB coalesced wavefront load feeds four
//        matrix instructions without any lane exchange;
//   bytes [8192 + 32*r, +16): the 16 E4M3 scale bytes of row r for blocks
//        16*kt + [0, 16); bytes [8192 + 32*r + 16, +16): the same for row 32 + r.
// 9216 bytes per 16384 weights = 0.5625 bytes per weight, the format's own size.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr int kTileRows = 64;
constexpr int kTileK = 256;
constexpr int kTileCodeBytes = 8192;
constexpr int kTileBytes = 9216;
constexpr int kChunkK = 32;          // k per 1 KB wavefront chunk
constexpr int kChunksPerTile = 8;
constexpr int kScaleOffset = 8192;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));  // operand of the scaled FP4/FP8 MFMA

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// 16 bytes of a weight stream that is read once: a non-temporal load, so
// that the lines go early from the caches instead of pushing out data that
// is still wanted (activations, partial sums).
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two E2M1 codes (byte `SEL` of w: low nibble -> .x, high nibble -> .y) to fp32.
// The conversion's scale operand only contributes its exponent, so 1.0f gives
// the plain E2M1 values.
template <int SEL>
__device__ __forceinline__ f32x2 e2m1x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

// E4M3FN byte `SEL` of w to fp32 (exact; NaN for 0x7F / 0xFF).
template <int SEL>
__device__ __forceinline__ float e4m3(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8(w, SEL);
}

// Pack two fp32 values whose low 16 bits are zero (at most 8 significant
// bits: every dequantised weight qualifies) into a bf16 pair: truncation is
// exact for them, and one byte permute does it.
__device__ __forceinline__ uint32_t pack_exact_bf16x2(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Round-to-nearest-even fp32 -> bf16 of a pair, packed low/high (one
// v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ uint16_t to_bf16(float v) {
  __bf16 a = (__bf16)v;
  return __builtin_bit_cast(uint16_t, a);
}

// One 16-byte-per-lane load from memory straight into LDS: lane l's 16
// bytes land at dst + 16 l (dst is the same for the whole wavefront).  Kept
// out of lambdas: a lambda body is also compiled for the host, where this
// builtin does not exist.  Its completion is counted by vmcnt like any load.
__device__ __forceinline__ void load_lds16(const void* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(const_cast<void*>(src), (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}

// vmcnt-only wait (gfx9 s_waitcnt encoding; expcnt and lgkmcnt left free).
// Vector memory operations of a wavefront complete in issue order, so
// vmcnt <= N means that all but the N most recently issued have completed.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// vmcnt <= N and lgkmcnt == 0.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

// Workgroup barrier that adds no waits of its own: loads into LDS that the
// other wavefronts read after it are waited for explicitly (wait_vmcnt) first.
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// Exchange between the wavefront halves: afterwards lanes 32..63 of `hi_dst`
// hold what lanes 0..31 of `lo_src` held, and lanes 0..31 of `lo_src` hold what
// lanes 32..63 of `hi_dst` held; the other lanes keep their values.
__device__ __forceinline__ void swap_halves(uint32_t& hi_dst, uint32_t& lo_src) {
  auto r = __builtin_amdgcn_permlane32_swap(hi_dst, lo_src, false, false);
  hi_dst = r[0];
  lo_src = r[1];
}

// Split-K handoff between workgroups without floating-point atomics.
//
// Each workgroup writes its partial sums with store_coherent, then calls
// arrive_last; the workgroup that arrives last sees true and reads every
// partial with load_coherent, adding them in index order -- so the result does
// not depend on arrival order.  It also returns the counter to zero.
//
// Coherence without cache maintenance: the L2 of each XCD is not coherent with
// the others, and a device-scope fence would write back and invalidate the
// whole L2 (slow, and it evicts the weight stream of every other workgroup on
// that XCD).  Instead every partial is stored and loaded as a device-scope
// relaxed atomic (write-through / L2-bypassing accesses), each thread waits
// for its own stores to complete before the workgroup barrier, and only then
// does one thread bump the device-scope counter.  The reader's loads are
// issued after it has observed the final count.
// Must be called by every thread of the workgroup (contains barriers).
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// sum_{i < count} p[i * stride], added in index order.  The loads are issued
// in batches of sixteen so that their memory latencies overlap (one round trip
// for up to 16 parts); padding lanes of a batch re-read the last element and
// are not added.
__device__ __forceinline__ float sum_coherent(const float* p, size_t stride, int count) {
  float s = 0.0f;
  for (int i = 0; i < count; i += 16) {
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int idx = i + j < count ? i + j : count - 1;
      v[j] = load_coherent(p + (size_t)idx * stride);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) s = (i + j < count) ? s + v[j] : s;
  }
  return s;
}

// Sixteen 16-byte loads that bypass the non-coherent caches, issued together;
// the wait for them sits in the same asm statement, so no load is still in
// flight when the statement ends.
__device__ __forceinline__ void load16x4_coherent(const float* const (&p)[16], f32x4 (&v)[16]) {
  asm volatile(
      "global_load_dwordx4 %0, %16, off sc1\n"
      "global_load_dwordx4 %1, %17, off sc1\n"
      "global_load_dwordx4 %2, %18, off sc1\n"
      "global_load_dwordx4 %3, %19, off sc1\n"
      "global_load_dwordx4 %4, %20, off sc1\n"
      "global_load_dwordx4 %5, %21, off sc1\n"
      "global_load_dwordx4 %6, %22, off sc1\n"
      "global_load_dwordx4 %7, %23, off sc1\n"
      "global_load_dwordx4 %8, %24, off sc1\n"
      "global_load_dwordx4 %9, %25, off sc1\n"
      "global_load_dwordx4 %10, %26, off sc1\n"
      "global_load_dwordx4 %11, %27, off sc1\n"
      "global_load_dwordx4 %12, %28, off sc1\n"
      "global_load_dwordx4 %13, %29, off sc1\n"
      "global_load_dwordx4 %14, %30, off sc1\n"
      "global_load_dwordx4 %15, %31, off sc1\n"
      "s_waitcnt vmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7]),
        "=&v"(v[8]), "=&v"(v[9]), "=&v"(v[10]), "=&v"(v[11]), "=&v"(v[12]), "=&v"(v[13]), "=&v"(v[14]),
        "=&v"(v[15])
      : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "v"(p[5]), "v"(p[6]), "v"(p[7]), "v"(p[8]),
        "v"(p[9]), "v"(p[10]), "v"(p[11]), "v"(p[12]), "v"(p[13]), "v"(p[14]), "v"(p[15])
      : "memory");
}

__device__ __forceinline__ bool arrive_last(unsigned* counter, unsigned expected) {
  __shared__ unsigned s_last;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);  // keep the partial stores above the wait
  __builtin_amdgcn_s_waitcnt(0);            // this thread's partial stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned last = (prev == expected - 1u) ? 1u : 0u;
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last;
  }
  __syncthreads();
  return s_last != 0u;
}

}  // namespace nvfp4
