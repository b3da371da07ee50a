// Host-side launchers of the HIP kernels; called only by abi.cpp after it has
// validated every argument.  Each returns the hipError_t of its launch(es).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace nvfp4 {

struct Geometry {
  int64_t n, k;      // logical shape
  int64_t nrt, nkt;  // row tiles (64 rows), k tiles (256 k)
};

inline Geometry geometry(int64_t n, int64_t k) {
  Geometry g;
  g.n = n;
  g.k = k;
  g.nrt = (n + 63) / 64;
  g.nkt = (k + 255) / 256;
  return g;
}

inline size_t packed_bytes(const Geometry& g) { return (size_t)g.nrt * (size_t)g.nkt * 9216u; }

// Split workspaces (GEMV and skinny GEMM) start with a fixed counter area of
// kCounterSlots zero-initialised uint32 counters -- one per row tile or row
// group -- followed by the partial sums.  Because the counter area never moves,
// calls of different shapes can share one workspace: one call's partials can
// never land on another call's counters.
constexpr int64_t kCounterSlots = 65536;
constexpr size_t kCounterBytes = (size_t)kCounterSlots * 4;
constexpr int64_t kMaxSplitRows = kCounterSlots * 64;
// The longest k (and MoE hidden / inter) the products accept: the range over
// which the kernels' fp32 accumulation error is proven below 1e-5 sum|w x|.
constexpr int64_t kMaxProductK = 32768;

// Split-K plan shared by the GEMV and the skinny GEMM: `groups` workgroups per
// row tile, 4 wavefronts each, so the K tiles are cut into 4*groups parts.
struct SplitPlan {
  int groups;
  int parts;
};
SplitPlan gemv_plan(const Geometry& g);
SplitPlan skinny_plan(const Geometry& g);
size_t gemv_workspace_bytes(const Geometry& g);
size_t skinny_workspace_bytes(const Geometry& g);
size_t prefill_workspace_bytes(int64_t m, const Geometry& g);

// One product of a batched launch (host view).
struct Problem {
  const void* packed;
  int64_t n, k;
  float st;
  const uint16_t* x;
  int64_t ldx;
  void* y;
  int64_t ldy;
};
constexpr int kMaxBatch = 8;  // problems per kernel launch (more are split into launches)

size_t gemv_batch_workspace_bytes(const Problem* p, int count);
// Products of 1..kGemvRowsMax activation rows go to the GEMV's tile mapping
// (all rows in one launch) instead of the matrix-core skinny path.
constexpr int64_t kGemvRowsMax = 2;
size_t gemv_rows_batch_workspace_bytes(const Problem* p, int count, int64_t m);
hipError_t launch_gemv_rows_batch(const Problem* p, int count, int64_t m, bool y_bf16, void* ws, hipStream_t s);
hipError_t launch_gemv_batch(const Problem* p, int count, void* ws, hipStream_t s);
// The library's own scratch for the GEMV batch (nvfp4_gemv_batched_noalloc):
// a device array of kStaticScratchBytes per device; static_scratch() returns
// its address on the current device, setting it up on first use (its counter
// area zeroed on stream s).  No allocation anywhere.
constexpr size_t kStaticScratchBytes = kCounterBytes + ((size_t)8 << 20);
constexpr int kNoallocMaxProblems = 64;
hipError_t static_scratch(hipStream_t s, void** out);
size_t skinny_batch_workspace_bytes(const Problem* p, int count);
hipError_t launch_skinny_batch(const Problem* p, int count, int64_t m, bool y_bf16, void* ws, hipStream_t s);
size_t prefill_batch_workspace_bytes(const Problem* p, int count, int64_t m);
hipError_t launch_prefill_batch(const Problem* p, int count, int64_t m, bool y_bf16, void* ws, hipStream_t s);

hipError_t launch_pack(const uint8_t* codes, const uint8_t* scales, const Geometry& g, void* packed,
                       hipStream_t s);
hipError_t launch_unpack(const void* packed, const Geometry& g, uint8_t* codes, uint8_t* scales,
                         hipStream_t s);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
// Zero-fill y [m][ldy] (n columns used), fp32 or bf16.
hipError_t launch_zero_rows(void* y, int64_t m, int64_t n, int64_t ldy, bool y_bf16, hipStream_t s);
size_t mx_packed_bytes(int64_t rows, int64_t k);
hipError_t launch_mx_pack(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k, void* dst, hipStream_t s);
hipError_t launch_mx_unpack(const void* src, int64_t rows, int64_t k, uint8_t* codes, uint8_t* scales, hipStream_t s);
// W4A4 product: x quantised to MX tiles in the workspace, then the stream-K
// prefill schedule with MX operands (workspace: its counters and partial sums
// first, w4a4_streamk_bytes(), then x's MX tiles).
struct MxProblem {
  const uint8_t* w;  // weight MX tiles
  int64_t n, k;
  float st;
  const uint8_t* x;  // activation MX tiles (m rows)
  void* y;
  int64_t ldy;
};
size_t w4a4_streamk_bytes();
hipError_t launch_w4a4_batch(const MxProblem* p, int count, int64_t m, bool y_bf16, void* ws, hipStream_t s);
// Batches: Problem::packed holds the weights' MX tiles; x is quantised into
// the workspace after the stream-K area, problem after problem.
size_t w4a4_batch_workspace_bytes(const Problem* p, int count, int64_t m);
hipError_t launch_w4a4_gemm_batch(const Problem* p, int count, int64_t m, bool y_bf16, void* ws, hipStream_t s);
size_t w4a4_workspace_bytes(int64_t m, int64_t k);
hipError_t launch_w4a4_gemm(const void* mx_w, int64_t n, int64_t k, float st, const uint16_t* x, int64_t m,
                            int64_t ldx, void* y, int64_t ldy, bool y_bf16, void* ws, hipStream_t s);
size_t quantize_workspace_bytes();
hipError_t launch_quantize(const void* w, bool bf16, int64_t n, int64_t k, int64_t ldw, uint8_t* codes,
                           uint8_t* scales, float* tensor_scale, void* ws, hipStream_t s);
hipError_t launch_gemv(const void* packed, const Geometry& g, float st, const uint16_t* x, float* y,
                       void* ws, hipStream_t s);
hipError_t launch_skinny(const void* packed, const Geometry& g, float st, const uint16_t* x, int64_t m,
                         int64_t ldx, void* y, int64_t ldy, bool y_bf16, void* ws, hipStream_t s);
hipError_t launch_prefill(const void* packed, const Geometry& g, float st, const uint16_t* x, int64_t m,
                          int64_t ldx, void* y, int64_t ldy, bool y_bf16, void* ws, hipStream_t s);

struct MoeLaunch {
  int64_t tokens, experts, top_k, hidden, inter;
  const uint16_t* x;
  const float* logits;
  const uint8_t* w_gate;
  const uint8_t* w_up;
  const uint8_t* w_down;
  size_t stride_gate, stride_up, stride_down;
  const float* scale_gate;
  const float* scale_up;
  const float* scale_down;
  void* y;
  bool y_bf16;
  int32_t* ids;
  float* g;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  float* dbg_gate;
  float* dbg_up;
  uint16_t* dbg_h;
  float* dbg_down;
  void* ws;
  const int32_t* slot_table = nullptr;  // device [experts]: pool slot of each expert (nullptr: slot e)
};
size_t moe_workspace_bytes(int64_t tokens, int64_t experts, int64_t top_k, int64_t hidden, int64_t inter);
int64_t moe_max_experts();
hipError_t launch_moe(const MoeLaunch& a, hipStream_t s);
// The two halves of launch_moe: routing and grouping, then the expert GEMMs and the scatter.
hipError_t launch_moe_routing(const MoeLaunch& a, hipStream_t s);
hipError_t launch_moe_experts(const MoeLaunch& a, hipStream_t s);
// Copies of `count` byte ranges (multiples of 16 bytes, 16-byte aligned) from
// GPU-mapped pinned host memory into device memory, in one launch per 96.
hipError_t launch_expert_copies(const void* const* src, void* const* dst, const size_t* bytes, int count,
                                hipStream_t s);

}  // namespace nvfp4
