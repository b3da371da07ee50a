// The C ABI of libnvfp4.so (declared in include/nvfp4.h): argument
// validation, status codes and dispatch to the kernel launchers.  Nothing here
// allocates or frees device memory; the one synchronisation is
// nvfp4_moe_streamed's read-back of the expert counts.  No exception leaves
// this file.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "../../include/nvfp4.h"
#include "launchers.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return NVFP4_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(NVFP4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

constexpr int64_t kMaxDim = int64_t(1) << 30;

int check_shape(int64_t n, int64_t k) {
  if (n < 0 || k < 0) return fail(NVFP4_ERR_SHAPE, "negative size (n=%lld, k=%lld)", (long long)n, (long long)k);
  if (k % 16 != 0) return fail(NVFP4_ERR_SHAPE, "k=%lld is not a multiple of 16 (one E4M3 scale per 16 k)", (long long)k);
  if (n > kMaxDim || k > kMaxDim) return fail(NVFP4_ERR_SHAPE, "size above 2^30 (n=%lld, k=%lld)", (long long)n, (long long)k);
  const nvfp4::Geometry g = nvfp4::geometry(n, k);
  if (g.nkt > 0 && g.nrt > (int64_t(1) << 40) / (g.nkt * 9216)) return fail(NVFP4_ERR_SHAPE, "packed matrix too large");
  return NVFP4_OK;
}

// Products: n up to the split-K counters' row limit, and k up to the length
// over which every kernel's fp32 accumulation provably stays within
// 1e-5 * sum |w x| (refuse rather than run wrong).
int check_product(int64_t n, int64_t k) {
  if (n > nvfp4::kMaxSplitRows)
    return fail(NVFP4_ERR_SHAPE, "n=%lld above the %lld rows a product call supports", (long long)n,
                (long long)nvfp4::kMaxSplitRows);
  if (k > nvfp4::kMaxProductK)
    return fail(NVFP4_ERR_SHAPE, "k=%lld above the %lld a product call accepts (the accumulation bound's range)",
                (long long)k, (long long)nvfp4::kMaxProductK);
  return NVFP4_OK;
}

#define NVFP4_TRY(expr)              \
  do {                               \
    int s_ = (expr);                 \
    if (s_ != NVFP4_OK) return s_;   \
  } while (0)

#define NVFP4_GUARD_BEGIN try {
#define NVFP4_GUARD_END                                                    \
  }                                                                        \
  catch (...) {                                                            \
    return fail(NVFP4_ERR_ARG, "internal error: unexpected C++ exception"); \
  }

}  // namespace

extern "C" {

int nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

const char* nvfp4_status_str(int status) {
  switch (status) {
    case NVFP4_OK: return "NVFP4_OK";
    case NVFP4_ERR_NULL: return "NVFP4_ERR_NULL";
    case NVFP4_ERR_SHAPE: return "NVFP4_ERR_SHAPE";
    case NVFP4_ERR_ALIGN: return "NVFP4_ERR_ALIGN";
    case NVFP4_ERR_DTYPE: return "NVFP4_ERR_DTYPE";
    case NVFP4_ERR_WORKSPACE: return "NVFP4_ERR_WORKSPACE";
    case NVFP4_ERR_ARG: return "NVFP4_ERR_ARG";
    case NVFP4_ERR_HIP: return "NVFP4_ERR_HIP";
    default: return "unknown status";
  }
}

const char* nvfp4_last_error(void) { return g_last_error; }

int nvfp4_packed_bytes(int64_t n, int64_t k, size_t* bytes) {
  NVFP4_GUARD_BEGIN
  if (!bytes) return fail(NVFP4_ERR_NULL, "bytes is NULL");
  NVFP4_TRY(check_shape(n, k));
  *bytes = nvfp4::packed_bytes(nvfp4::geometry(n, k));
  return ok();
  NVFP4_GUARD_END
}

int nvfp4_pack(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k, void* packed, void* stream) {
  NVFP4_GUARD_BEGIN
  NVFP4_TRY(check_shape(n, k));
  if (n == 0 || k == 0) return ok();
  if (!codes || !scales || !packed) return fail(NVFP4_ERR_NULL, "codes, scales and packed must be non-NULL");
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(packed))
    return fail(NVFP4_ERR_ALIGN, "codes, scales and packed must be 16-byte aligned");
  return hip_status(nvfp4::launch_pack(codes, scales, nvfp4::geometry(n, k), packed, (hipStream_t)stream), "pack launch");
  NVFP4_GUARD_END
}

int nvfp4_unpack(const void* packed, int64_t n, int64_t k, uint8_t* codes, uint8_t* scales, void* stream) {
  NVFP4_GUARD_BEGIN
  NVFP4_TRY(check_shape(n, k));
  if (n == 0 || k == 0) return ok();
  if (!codes || !scales || !packed) return fail(NVFP4_ERR_NULL, "codes, scales and packed must be non-NULL");
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(packed))
    return fail(NVFP4_ERR_ALIGN, "codes, scales and packed must be 16-byte aligned");
  return hip_status(nvfp4::launch_unpack(packed, nvfp4::geometry(n, k), codes, scales, (hipStream_t)stream),
                    "unpack launch");
  NVFP4_GUARD_END
}

int nvfp4_gemv_workspace_bytes(int64_t n, int64_t k, size_t* bytes) {
  NVFP4_GUARD_BEGIN
  if (!bytes) return fail(NVFP4_ERR_NULL, "bytes is NULL");
  NVFP4_TRY(check_shape(n, k));
  NVFP4_TRY(check_product(n, k));
  *bytes = nvfp4::gemv_workspace_bytes(nvfp4::geometry(n, k));
  return ok();
  NVFP4_GUARD_END
}

static int check_mx_shape(int64_t rows, int64_t k) {
  NVFP4_TRY(check_shape(rows, k));
  if (k % 32 != 0) return fail(NVFP4_ERR_SHAPE, "k=%lld is not a multiple of 32 (one MX scale per 32 k)", (long long)k);
  return NVFP4_OK;
}

int nvfp4_mx_packed_bytes(int64_t rows, int64_t k, size_t* bytes) {
  NVFP4_GUARD_BEGIN
  if (!bytes) return fail(NVFP4_ERR_NULL, "bytes is NULL");
  NVFP4_TRY(check_mx_shape(rows, k));
  *bytes = nvfp4::mx_packed_bytes(rows, k);
  return ok();
  NVFP4_GUARD_END
}

int nvfp4_mx_pack(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k, void* mx_packed, void* stream) {
  NVFP4_GUARD_BEGIN
  NVFP4_TRY(check_mx_shape(n, k));
  if (n == 0 || k == 0) return ok();
  if (!codes || !scales || !mx_packed) return fail(NVFP4_ERR_NULL, "codes, scales and mx_packed must be non-NULL");
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(mx_packed))
    return fail(NVFP4_ERR_ALIGN, "codes, scales and mx_packed must be 16-byte aligned");
  return hip_status(nvfp4::launch_mx_pack(codes, scales, n, k, mx_packed, (hipStream_t)stream), "mx pack launch");
  NVFP4_GUARD_END
}

int nvfp4_mx_unpack(const void* mx_packed, int64_t rows, int64_t k, uint8_t* codes, uint8_t* scales, void* stream) {
  NVFP4_GUARD_BEGIN
  NVFP4_TRY(check_mx_shape(rows, k));
  if (rows == 0 || k == 0) return ok();
  if (!codes || !scales || !mx_packed) return fail(NVFP4_ERR_NULL, "codes, scales and mx_packed must be non-NULL");
  if (!aligned16(codes) || !aligned16(mx_packed)) return fail(NVFP4_ERR_ALIGN, "codes and mx_packed must be 16-byte aligned");
  return hip_status(nvfp4::launch_mx_unpack(mx_packed, rows, k, codes, scales, (hipStream_t)stream), "mx unpack launch");
  NVFP4_GUARD_END
}

int nvfp4_w4a4_workspace_bytes(int64_t m, int64_t k, size_t* bytes) {
  NVFP4_GUARD_BEGIN
  if (!bytes) return fail(NVFP4_ERR_NULL, "bytes is NULL");
  NVFP4_TRY(check_mx_shape(m, k));
  *bytes = nvfp4::w4a4_workspace_bytes(m, k);
  return ok();
  NVFP4_GUARD_END
}

int nvfp4_w4a4_gemm(const void* mx_packed, int64_t n, int64_t k, float tensor_scale, const uint16_t* x, int64_t m,
                    int64_t ldx, void* y, int64_t ldy, int y_dtype, void* workspace, size_t workspace_bytes,
                    void* stream) {
  NVFP4_GUARD_BEGIN
  NVFP4_TRY(check_mx_shape(n, k));
  NVFP4_TRY(check_product(n, k));
  if (m < 0 || m > (int64_t(1) << 24)) return fail(NVFP4_ERR_SHAPE, "m=%lld out of range", (long long)m);
  if (y_dtype != NVFP4_F32 && y_dtype != NVFP4_BF16) return fail(NVFP4_ERR_DTYPE, "unknown y_dtype %d", y_dtype);
  if (m == 0 || n == 0) return ok();
  if (k == 0) return hip_status(nvfp4::launch_zero_rows(y, m, n, ldy, y_dtype == NVFP4_BF16, (hipStream_t)stream), "zero fill");
  if (ldx < k || ldx % 8 != 0) return fail(NVFP4_ERR_SHAPE, "ldx=%lld must be >= k=%lld and a multiple of 8", (long long)ldx, (long long)k);
  if (ldy < n) return fail(NVFP4_ERR_SHAPE, "ldy=%lld must be >= n=%lld", (long long)ldy, (long long)n);
  if (!mx_packed || !x || !y) return fail(NVFP4_ERR_NULL, "mx_packed, x and y must be non-NULL");
  if (!aligned16(mx_packed) || !aligned16(x) || !aligned16(y)) return fail(NVFP4_ERR_ALIGN, "mx_packed, x and y must be 16-byte aligned");
  const size_t need = nvfp4::w4a4_workspace_bytes(m, k);
  if (!workspace || workspace_bytes < need)
    return fail(NVFP4_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need, workspace ? workspace_bytes : 0);
  if (!aligned16(workspace)) return fail(NVFP4_ERR_ALIGN, "workspace must be 16-byte aligned");
  return hip_status(nvfp4::launch_w4a4_gemm(mx_packed, n, k, tensor_scale, x, m, ldx, y, ldy, y_dtype == NVFP4_BF16,
                                            workspace, (hipStream_t)stream),
                    "w4a4 gemm launch");
  NVFP4_GUARD_END
}

int nvfp4_quantize_workspace_bytes(size_t* bytes) {
  NVFP4_GUARD_BEGIN
  if (!bytes) return fail(NVFP4_ERR_NULL, "bytes is NULL");
  *bytes = nvfp4::quantize_workspace_bytes();
  return ok();
  NVFP4_GUARD_END
}

int nvfp4_quantize(const void* w, int w_dtype, int64_t n, int64_t k, int64_t ldw, uint8_t* codes, uint8_t* scales,
                   float* tensor_scale, void* workspace, size_t workspace_bytes, void* stream) {
  NVFP4_GUARD_BEGIN
  NVFP4_TRY(check_shape(n, k));
  if (w_dtype != NVFP4_F32 && w_dtype != NVFP4_BF16) return fail(NVFP4_ERR_DTYPE, "w_dtype=%d unknown", w_dtype);
  if (n == 0 || k == 0) return ok();
  if (ldw < k || ldw % 8 != 0 || ldw > kMaxDim)
    return fail(NVFP4_ERR_SHAPE, "ldw=%lld must be >= k=%lld, a multiple of 8 and at most 2^30", (long long)ldw,
                (long long)k);
  if (!w || !codes || !scales || !tensor_scale)
    return fail(NVFP4_ERR_NULL, "w, codes, scales and tensor_scale must be non-NULL");
  if (!aligned16(w) || !aligned16(codes) || !aligned16(scales) || !aligned4(tensor_scale))
    return fail(NVFP4_ERR_ALIGN, "w, codes and scales must be 16-byte aligned, tensor_scale 4-byte aligned");
  const size_t need = nvfp4::quantize_workspace_bytes();
  if (!workspace || workspace_bytes < need)
    return fail(NVFP4_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need, workspace ? workspace_bytes : 0);
  if (!aligned16(workspace)) return fail(NVFP4_ERR_ALIGN, "workspace must be 16-byte aligned");
  return hip_status(nvfp4::launch_quantize(w, w_dtype == NVFP4_BF16, n, k, ldw, codes, scales, tensor_scale,
                                           workspace, (hipStream_t)stream),
                    "quantize launch");
  NVFP4_GUARD_END
}

int nvfp4_gemv(const void* packed, int64_t n, int64_t k, float tensor_scale, const uint16_t* x, float* y,
               void* workspace, size_t workspace_bytes, void* stream) {
  NVFP4_GUARD_BEGIN
  NVFP4_TRY(check_shape(n, k));
  NVFP4_TRY(check_product(n, k));
  if (n == 0) return ok();
  if (!y || (k > 0 && (!packed || !x))) return fail(NVFP4_ERR_NULL, "packed, x and y must be non-NULL");
  if (!aligned16(y) || (k > 0 && (!aligned16(packed) || !aligned16(x))))
    return fail(NVFP4_ERR_ALIGN, "packed, x and y must be 16-byte aligned");
  const nvfp4::Geometry g = nvfp4::geometry(n, k);
  const size_t need = nvfp4::gemv_workspace_bytes(g);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(NVFP4_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need, workspace ? workspace_bytes : 0);
  if (need > 0 && !aligned16(workspace)) return fail(NVFP4_ERR_ALIGN, "workspace must be 16-byte aligned");
  return hip_status(nvfp4::launch_gemv(packed, g, tensor_scale, x, y, workspace, (hipStream_t)stream), "gemv launch");
  NVFP4_GUARD_END
}

int nvfp4_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k, size_t* bytes) {
  NVFP4_GUARD_BEGIN
  if (!bytes) return fail(NVFP4_ERR_NULL, "bytes is NULL");
  NVFP4_TRY(check_shape(n, k));
  NVFP4_TRY(check_product(n, k));
  if (m < 0 || m > kMaxDim) return fail(NVFP4_ERR_SHAPE, "m=%lld out of range", (long long)m);
  const nvfp4::Geometry g = nvfp4::geometry(n, k);
  if (m <= nvfp4::kGemvRowsMax) {
    const nvfp4::Problem pr{nullptr, n, k, 1.0f, nullptr, k, nullptr, n};
    *bytes = nvfp4::gemv_rows_batch_workspace_bytes(&pr, 1, m);
  } else {
    *bytes = m <= 32 ? nvfp4::skinny_workspace_bytes(g) : nvfp4::prefill_workspace_bytes(m, g);
  }
  return ok();
  NVFP4_GUARD_END
}

int nvfp4_gemm(const void* packed, int64_t n, int64_t k, float tensor_scale, const uint16_t* x, int64_t m,
               int64_t ldx, void* y, int64_t ldy, int y_dtype, void* workspace, size_t workspace_bytes,
               void* stream) {
  NVFP4_GUARD_BEGIN
  NVFP4_TRY(check_shape(n, k));
  NVFP4_TRY(check_product(n, k));
  if (m < 0 || m > kMaxDim) return fail(NVFP4_ERR_SHAPE, "m=%lld out of range", (long long)m);
  if (y_dtype != NVFP4_F32 && y_dtype != NVFP4_BF16) return fail(NVFP4_ERR_DTYPE, "unknown y_dtype %d", y_dtype);
  if (m == 0 || n == 0) return ok();
  if (ldx < k || ldx % 8 != 0) return fail(NVFP4_ERR_SHAPE, "ldx=%lld must be >= k=%lld and a multiple of 8", (long long)ldx, (long long)k);
  if (ldy < n) return fail(NVFP4_ERR_SHAPE, "ldy=%lld must be >= n=%lld", (long long)ldy, (long long)n);
  if (!y || (k > 0 && (!packed || !x))) return fail(NVFP4_ERR_NULL, "packed, x and y must be non-NULL");
  if (!aligned16(y) || (k > 0 && (!aligned16(packed) || !aligned16(x))))
    return fail(NVFP4_ERR_ALIGN, "packed, x and y must be 16-byte aligned");
  const nvfp4::Geometry g = nvfp4::geometry(n, k);
  if (m <= nvfp4::kGemvRowsMax) {
    const nvfp4::Problem pr{packed, n, k, tensor_scale, x, ldx, y, ldy};
    const size_t need = nvfp4::gemv_rows_batch_workspace_bytes(&pr, 1, m);
    if (need > 0 && (!workspace || workspace_bytes < need))
      return fail(NVFP4_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need, workspace ? workspace_bytes : 0);
    if (need > 0 && !aligned16(workspace)) return fail(NVFP4_ERR_ALIGN, "workspace must be 16-byte aligned");
    return hip_status(nvfp4::launch_gemv_rows_batch(&pr, 1, m, y_dtype == NVFP4_BF16, workspace, (hipStream_t)stream),
                      "gemv rows launch");
  }
  const bool skinny = m <= 32;
  const size_t need = skinny ? nvfp4::skinny_workspace_bytes(g) : nvfp4::prefill_workspace_bytes(m, g);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(NVFP4_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need, workspace ? workspace_bytes : 0);
  if (need > 0 && !aligned16(workspace)) return fail(NVFP4_ERR_ALIGN, "workspace must be 16-byte aligned");
  const bool bf16 = y_dtype == NVFP4_BF16;
  hipError_t e = skinny ? nvfp4::launch_skinny(packed, g, tensor_scale, x, m, ldx, y, ldy, bf16, workspace, (hipStream_t)stream)
                        : nvfp4::launch_prefill(packed, g, tensor_scale, x, m, ldx, y, ldy, bf16, workspace, (hipStream_t)stream);
  return hip_status(e, skinny ? "skinny gemm launch" : "prefill gemm launch");
  NVFP4_GUARD_END
}

// Validate a batch and convert it; `gemm_m` < 0 for GEMV batches.
static int check_batch(const nvfp4_problem* pr, int count, int64_t gemm_m, int y_dtype, bool need_buffers,
                       nvfp4::Problem* out) {
  if (count < 0) return fail(NVFP4_ERR_ARG, "count=%d is negative", count);
  if (count > 0 && !pr) return fail(NVFP4_ERR_NULL, "problems is NULL");
  if (gemm_m >= 0 && y_dtype != NVFP4_F32 && y_dtype != NVFP4_BF16)
    return fail(NVFP4_ERR_DTYPE, "unknown y_dtype %d", y_dtype);
  if (gemm_m > kMaxDim) return fail(NVFP4_ERR_SHAPE, "m=%lld out of range", (long long)gemm_m);
  int64_t tiles = 0;
  for (int i = 0; i < count; ++i) {
    const nvfp4_problem& q = pr[i];
    NVFP4_TRY(check_shape(q.n, q.k));
    NVFP4_TRY(check_product(q.n, q.k));
    if (i % nvfp4::kMaxBatch == 0) tiles = 0;
    tiles += (q.n + 63) / 64;
    if (tiles > nvfp4::kCounterSlots)
      return fail(NVFP4_ERR_SHAPE, "a launch of %d problems exceeds %lld row tiles", nvfp4::kMaxBatch,
                  (long long)nvfp4::kCounterSlots);
    out[i] = nvfp4::Problem{q.packed, q.n, q.k, q.tensor_scale, q.x, q.ldx, q.y, q.ldy};
    if (!need_buffers || q.n == 0 || gemm_m == 0) continue;
    if (gemm_m > 0) {
      if (q.ldx < q.k || q.ldx % 8 != 0)
        return fail(NVFP4_ERR_SHAPE, "problem %d: ldx=%lld must be >= k and a multiple of 8", i, (long long)q.ldx);
      if (q.ldy < q.n) return fail(NVFP4_ERR_SHAPE, "problem %d: ldy=%lld must be >= n", i, (long long)q.ldy);
    }
    if (!q.y || (q.k > 0 && (!q.packed || !q.x))) return fail(NVFP4_ERR_NULL, "problem %d: NULL pointer", i);
    if (!aligned16(q.y) || (q.k > 0 && (!aligned16(q.packed) || !aligned16(q.x))))
      return fail(NVFP4_ERR_ALIGN, "problem %d: packed, x and y must be 16-byte aligned", i);
    for (int j = 0; j < i; ++j)
      if (pr[j].y == q.y && pr[j].n > 0) return fail(NVFP4_ERR_ARG, "problems %d and %d share an output", j, i);
  }
  return NVFP4_OK;
}

static int check_moe(const nvfp4_moe_args* a, bool need_buffers) {
  if (!a) return fail(NVFP4_ERR_NULL, "args is NULL");
  if (a->tokens < 0 || a->hidden <= 0 || a->inter <= 0 || a->experts <= 0)
    return fail(NVFP4_ERR_SHAPE, "tokens must be >= 0; experts, hidden and inter > 0");
  if (a->hidden % 16 != 0 || a->inter % 16 != 0)
    return fail(NVFP4_ERR_SHAPE, "hidden=%lld and inter=%lld must be multiples of 16", (long long)a->hidden, (long long)a->inter);
  if (a->tokens > kMaxDim) return fail(NVFP4_ERR_SHAPE, "tokens above 2^30");
  if (a->hidden > nvfp4::kMaxProductK || a->inter > nvfp4::kMaxProductK)
    return fail(NVFP4_ERR_SHAPE, "hidden=%lld and inter=%lld must be at most %lld (the accumulation bound's range)",
                (long long)a->hidden, (long long)a->inter, (long long)nvfp4::kMaxProductK);
  if (a->experts > nvfp4::moe_max_experts())
    return fail(NVFP4_ERR_ARG, "experts=%lld above the supported %lld", (long long)a->experts, (long long)nvfp4::moe_max_experts());
  if (a->top_k < 1 || a->top_k > a->experts || a->top_k > 64)
    return fail(NVFP4_ERR_ARG, "top_k=%lld must be in [1, min(experts, 64)]", (long long)a->top_k);
  if (a->tokens * a->top_k > (int64_t(1) << 30)) return fail(NVFP4_ERR_SHAPE, "tokens*top_k too large");
  if (!need_buffers) return NVFP4_OK;
  if (a->y_dtype != NVFP4_F32 && a->y_dtype != NVFP4_BF16) return fail(NVFP4_ERR_DTYPE, "unknown y_dtype %d", a->y_dtype);
  if (!a->x || !a->router_logits || !a->w_gate || !a->w_up || !a->w_down || !a->scale_gate || !a->scale_up ||
      !a->scale_down || !a->y || !a->topk_ids || !a->topk_weights || !a->expert_counts || !a->expert_offsets ||
      !a->perm || !a->workspace)
    return fail(NVFP4_ERR_NULL, "a required MoE pointer is NULL");
  if (!aligned16(a->x) || !aligned16(a->w_gate) || !aligned16(a->w_up) || !aligned16(a->w_down) ||
      !aligned16(a->workspace) || !aligned16(a->y) || (a->dbg_gate && !aligned16(a->dbg_gate)) ||
      (a->dbg_up && !aligned16(a->dbg_up)) || (a->dbg_h && !aligned16(a->dbg_h)) ||
      (a->dbg_down && !aligned16(a->dbg_down)))
    return fail(NVFP4_ERR_ALIGN, "x, weight pools, y, workspace and debug outputs must be 16-byte aligned");
  if (!aligned4(a->router_logits) || !aligned4(a->scale_gate) || !aligned4(a->scale_up) || !aligned4(a->scale_down) ||
      !aligned4(a->topk_ids) || !aligned4(a->topk_weights) || !aligned4(a->expert_counts) ||
      !aligned4(a->expert_offsets) || !aligned4(a->perm))
    return fail(NVFP4_ERR_ALIGN, "logits, scales and index outputs must be 4-byte aligned");
  const size_t gu = nvfp4::packed_bytes(nvfp4::geometry(a->inter, a->hidden));
  const size_t dn = nvfp4::packed_bytes(nvfp4::geometry(a->hidden, a->inter));
  if (a->stride_gate < gu || a->stride_up < gu || a->stride_down < dn)
    return fail(NVFP4_ERR_ARG, "expert strides must be at least the packed matrix size (%zu / %zu bytes)", gu, dn);
  if (a->stride_gate % 16 || a->stride_up % 16 || a->stride_down % 16)
    return fail(NVFP4_ERR_ALIGN, "expert strides must be multiples of 16 bytes");
  const size_t need = nvfp4::moe_workspace_bytes(a->tokens, a->experts, a->top_k, a->hidden, a->inter);
  if (a->workspace_bytes < need) return fail(NVFP4_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need, a->workspace_bytes);
  return NVFP4_OK;
}

static nvfp4::MoeLaunch moe_launch_of(const nvfp4_moe_args* a) {
  nvfp4::MoeLaunch l;
  l.tokens = a->tokens; l.experts = a->experts; l.top_k = a->top_k; l.hidden = a->hidden; l.inter = a->inter;
  l.x = a->x; l.logits = a->router_logits;
  l.w_gate = static_cast<const uint8_t*>(a->w_gate);
  l.w_up = static_cast<const uint8_t*>(a->w_up);
  l.w_down = static_cast<const uint8_t*>(a->w_down);
  l.stride_gate = a->stride_gate; l.stride_up = a->stride_up; l.stride_down = a->stride_down;
  l.scale_gate = a->scale_gate; l.scale_up = a->scale_up; l.scale_down = a->scale_down;
  l.y = a->y; l.y_bf16 = a->y_dtype == NVFP4_BF16;
  l.ids = a->topk_ids; l.g = a->topk_weights; l.counts = a->expert_counts; l.offsets = a->expert_offsets;
  l.perm = a->perm;
  l.dbg_gate = a->dbg_gate; l.dbg_up = a->dbg_up; l.dbg_h = a->dbg_h; l.dbg_down = a->dbg_down;
  l.ws = a->workspace;
  return l;
}

int nvfp4_gemv_batched_workspace_bytes(const nvfp4_problem* problems, int count, size_t* bytes) {
  NVFP4_GUARD_BEGIN
  if (!bytes) return fail(NVFP4_ERR_NULL, "bytes is NULL");
  std::vector<nvfp4::Problem> pr((size_t)(count > 0 ? count : 0));
  NVFP4_TRY(check_batch(problems, count, -1, NVFP4_F32, false, pr.data()));
  *bytes = nvfp4::gemv_batch_workspace_bytes(pr.data(), count);
  return ok();
  NVFP4_GUARD_END
}

int nvfp4_gemv_batched(const nvfp4_problem* problems, int count, void* workspace, size_t workspace_bytes,
                       void* stream) {
  NVFP4_GUARD_BEGIN
  std::vector<nvfp4::Problem> pr((size_t)(count > 0 ? count : 0));
  NVFP4_TRY(check_batch(problems, count, -1, NVFP4_F32, true, pr.data()));
  if (count == 0) return ok();
  const size_t need = nvfp4::gemv_batch_workspace_bytes(pr.data(), count);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(NVFP4_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need, workspace ? workspace_bytes : 0);
  if (need > 0 && !aligned16(workspace)) return fail(NVFP4_ERR_ALIGN, "workspace must be 16-byte aligned");
  return hip_status(nvfp4::launch_gemv_batch(pr.data(), count, workspace, (hipStream_t)stream), "gemv batch launch");
  NVFP4_GUARD_END
}

int nvfp4_gemv_batched_noalloc(const nvfp4_problem* problems, int count, void* stream) {
  NVFP4_GUARD_BEGIN
  if (count > nvfp4::kNoallocMaxProblems)
    return fail(NVFP4_ERR_ARG, "count=%d above the %d problems this call takes", count, nvfp4::kNoallocMaxProblems);
  nvfp4::Problem pr[nvfp4::kNoallocMaxProblems];
  NVFP4_TRY(check_batch(problems, count, -1, NVFP4_F32, true, pr));
  if (count <= 0) return ok();
  const size_t need = nvfp4::gemv_batch_workspace_bytes(pr, count);
  if (need > nvfp4::kStaticScratchBytes)
    return fail(NVFP4_ERR_WORKSPACE, "the batch needs %zu bytes of scratch; the library's static scratch holds %zu",
                need, nvfp4::kStaticScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = nvfp4::static_scratch((hipStream_t)stream, &ws);
    if (e != hipSuccess) return hip_status(e, "static scratch set-up");
  }
  return hip_status(nvfp4::launch_gemv_batch(pr, count, ws, (hipStream_t)stream), "gemv batch launch");
  NVFP4_GUARD_END
}

// W4A4 batches: the gemm batch's checks, and k % 32 == 0 for the MX scales.
static int check_w4a4_batch(const nvfp4_problem* pr, int count, int64_t m, int y_dtype, bool need_buffers,
                            nvfp4::Problem* out) {
  if (m < 0 || m > (int64_t(1) << 24)) return fail(NVFP4_ERR_SHAPE, "m=%lld out of range", (long long)m);
  NVFP4_TRY(check_batch(pr, count, m, y_dtype, need_buffers, out));
  for (int i = 0; i < count; ++i)
    if (pr[i].k % 32 != 0)
      return fail(NVFP4_ERR_SHAPE, "problem %d: k=%lld is not a multiple of 32 (one MX scale per 32 k)", i,
                  (long long)pr[i].k);
  return NVFP4_OK;
}

int nvfp4_w4a4_batched_workspace_bytes(const nvfp4_problem* problems, int count, int64_t m, size_t* bytes) {
  NVFP4_GUARD_BEGIN
  if (!bytes) return fail(NVFP4_ERR_NULL, "bytes is NULL");
  std::vector<nvfp4::Problem> pr((size_t)(count > 0 ? count : 0));
  NVFP4_TRY(check_w4a4_batch(problems, count, m, NVFP4_F32, false, pr.data()));
  *bytes = nvfp4::w4a4_batch_workspace_bytes(pr.data(), count, m);
  return ok();
  NVFP4_GUARD_END
}

int nvfp4_w4a4_batched(const nvfp4_problem* problems, int count, int64_t m, int y_dtype, void* workspace,
                       size_t workspace_bytes, void* stream) {
  NVFP4_GUARD_BEGIN
  std::vector<nvfp4::Problem> pr((size_t)(count > 0 ? count : 0));
  NVFP4_TRY(check_w4a4_batch(problems, count, m, y_dtype, true, pr.data()));
  if (count == 0 || m == 0) return ok();
  const size_t need = nvfp4::w4a4_batch_workspace_bytes(pr.data(), count, m);
  if (!workspace || workspace_bytes < need)
    return fail(NVFP4_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need, workspace ? workspace_bytes : 0);
  if (!aligned16(workspace)) return fail(NVFP4_ERR_ALIGN, "workspace must be 16-byte aligned");
  return hip_status(nvfp4::launch_w4a4_gemm_batch(pr.data(), count, m, y_dtype == NVFP4_BF16, workspace,
                                                  (hipStream_t)stream),
                    "w4a4 batch launch");
  NVFP4_GUARD_END
}

int nvfp4_gemm_batched_workspace_bytes(const nvfp4_problem* problems, int count, int64_t m, size_t* bytes) {
  NVFP4_GUARD_BEGIN
  if (!bytes) return fail(NVFP4_ERR_NULL, "bytes is NULL");
  if (m < 0) return fail(NVFP4_ERR_SHAPE, "m=%lld is negative", (long long)m);
  std::vector<nvfp4::Problem> pr((size_t)(count > 0 ? count : 0));
  NVFP4_TRY(check_batch(problems, count, m, NVFP4_F32, false, pr.data()));
  size_t need = 0;
  if (m <= nvfp4::kGemvRowsMax) {
    need = nvfp4::gemv_rows_batch_workspace_bytes(pr.data(), count, m);
  } else if (m <= 32) {
    need = nvfp4::skinny_batch_workspace_bytes(pr.data(), count);
  } else {
    need = nvfp4::prefill_batch_workspace_bytes(pr.data(), count, m);
  }
  *bytes = need;
  return ok();
  NVFP4_GUARD_END
}

int nvfp4_gemm_batched(const nvfp4_problem* problems, int count, int64_t m, int y_dtype, void* workspace,
                       size_t workspace_bytes, void* stream) {
  NVFP4_GUARD_BEGIN
  if (m < 0) return fail(NVFP4_ERR_SHAPE, "m=%lld is negative", (long long)m);
  std::vector<nvfp4::Problem> pr((size_t)(count > 0 ? count : 0));
  NVFP4_TRY(check_batch(problems, count, m, y_dtype, true, pr.data()));
  if (count == 0 || m == 0) return ok();
  const bool bf16 = y_dtype == NVFP4_BF16;
  if (m <= nvfp4::kGemvRowsMax) {
    const size_t need = nvfp4::gemv_rows_batch_workspace_bytes(pr.data(), count, m);
    if (need > 0 && (!workspace || workspace_bytes < need))
      return fail(NVFP4_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need, workspace ? workspace_bytes : 0);
    if (need > 0 && !aligned16(workspace)) return fail(NVFP4_ERR_ALIGN, "workspace must be 16-byte aligned");
    return hip_status(nvfp4::launch_gemv_rows_batch(pr.data(), count, m, bf16, workspace, (hipStream_t)stream),
                      "gemv rows batch launch");
  }
  if (m <= 32) {
    const size_t need = nvfp4::skinny_batch_workspace_bytes(pr.data(), count);
    if (need > 0 && (!workspace || workspace_bytes < need))
      return fail(NVFP4_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need, workspace ? workspace_bytes : 0);
    if (need > 0 && !aligned16(workspace)) return fail(NVFP4_ERR_ALIGN, "workspace must be 16-byte aligned");
    return hip_status(nvfp4::launch_skinny_batch(pr.data(), count, m, bf16, workspace, (hipStream_t)stream),
                      "skinny gemm batch launch");
  }
  const size_t need = nvfp4::prefill_batch_workspace_bytes(pr.data(), count, m);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(NVFP4_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need, workspace ? workspace_bytes : 0);
  if (need > 0 && !aligned16(workspace)) return fail(NVFP4_ERR_ALIGN, "workspace must be 16-byte aligned");
  return hip_status(nvfp4::launch_prefill_batch(pr.data(), count, m, bf16, workspace, (hipStream_t)stream),
                    "prefill gemm batch launch");
  NVFP4_GUARD_END
}

int nvfp4_moe_workspace_bytes(const nvfp4_moe_args* args, size_t* bytes) {
  NVFP4_GUARD_BEGIN
  if (!bytes) return fail(NVFP4_ERR_NULL, "bytes is NULL");
  NVFP4_TRY(check_moe(args, false));
  *bytes = nvfp4::moe_workspace_bytes(args->tokens, args->experts, args->top_k, args->hidden, args->inter);
  return ok();
  NVFP4_GUARD_END
}

int nvfp4_moe_grouped(const nvfp4_moe_args* a, void* stream) {
  NVFP4_GUARD_BEGIN
  if (a && a->tokens == 0) {
    NVFP4_TRY(check_moe(a, false));
    return ok();
  }
  NVFP4_TRY(check_moe(a, true));
  return hip_status(nvfp4::launch_moe(moe_launch_of(a), (hipStream_t)stream), "moe launch");
  NVFP4_GUARD_END
}

int nvfp4_expert_cache_reset(nvfp4_expert_cache* c) {
  NVFP4_GUARD_BEGIN
  if (!c) return fail(NVFP4_ERR_NULL, "cache is NULL");
  if (c->experts <= 0 || c->slots <= 0) return fail(NVFP4_ERR_ARG, "experts and slots must be positive");
  if (!c->slot_of || !c->expert_in || !c->last_use) return fail(NVFP4_ERR_NULL, "cache state arrays must be non-NULL");
  for (int64_t e = 0; e < c->experts; ++e) c->slot_of[e] = -1;
  for (int64_t s = 0; s < c->slots; ++s) {
    c->expert_in[s] = -1;
    c->last_use[s] = 0;
  }
  c->clock = 0;
  c->last_active = c->last_fetched = 0;
  c->last_bytes = 0;
  return ok();
  NVFP4_GUARD_END
}

int nvfp4_moe_streamed(const nvfp4_moe_args* a, nvfp4_expert_cache* c, void* stream) {
  NVFP4_GUARD_BEGIN
  if (!c) return fail(NVFP4_ERR_NULL, "cache is NULL");
  if (a && a->tokens == 0) {
    NVFP4_TRY(check_moe(a, false));
    c->last_active = c->last_fetched = 0;
    c->last_bytes = 0;
    return ok();
  }
  NVFP4_TRY(check_moe(a, true));
  if (c->experts != a->experts || c->slots <= 0)
    return fail(NVFP4_ERR_ARG, "cache covers %lld experts with %lld slots; the call has %lld experts",
                (long long)c->experts, (long long)c->slots, (long long)a->experts);
  if (a->w_gate != c->dev_gate || a->w_up != c->dev_up || a->w_down != c->dev_down ||
      a->stride_gate != c->stride_gate || a->stride_up != c->stride_up || a->stride_down != c->stride_down)
    return fail(NVFP4_ERR_ARG, "args' weight pools and strides must be the cache's device slot pools");
  if (!c->host_gate || !c->host_up || !c->host_down || !c->dev_slot_of || !c->host_counts || !c->host_slot_stage ||
      !c->slot_of || !c->expert_in || !c->last_use)
    return fail(NVFP4_ERR_NULL, "a cache buffer is NULL");
  if (!aligned4(c->dev_slot_of) || !aligned4(c->host_counts) || !aligned4(c->host_slot_stage))
    return fail(NVFP4_ERR_ALIGN, "the cache's int32 arrays must be 4-byte aligned");
  const hipStream_t s = (hipStream_t)stream;
  nvfp4::MoeLaunch l = moe_launch_of(a);
  NVFP4_TRY(hip_status(nvfp4::launch_moe_routing(l, s), "moe routing launch"));
  // Which experts this call routes to: one read-back of the counts.
  NVFP4_TRY(hip_status(hipMemcpyAsync(c->host_counts, a->expert_counts, (size_t)a->experts * 4, hipMemcpyDeviceToHost, s),
                       "expert counts read-back"));
  NVFP4_TRY(hip_status(hipStreamSynchronize(s), "expert counts read-back"));
  // The cache's new state is planned on copies and committed only once every
  // launch of the call has been enqueued: a failure leaves no expert marked
  // resident whose bytes never arrived.
  const uint64_t now = c->clock + 1;
  std::vector<int32_t> slot_of(c->slot_of, c->slot_of + a->experts);
  std::vector<int32_t> expert_in(c->expert_in, c->expert_in + c->slots);
  std::vector<uint64_t> last_use(c->last_use, c->last_use + c->slots);
  int64_t active = 0;
  for (int64_t e = 0; e < a->experts; ++e)
    if (c->host_counts[e] > 0) {
      ++active;
      if (slot_of[e] >= 0) last_use[slot_of[e]] = now;  // a hit: keep it this call
    }
  c->last_active = active;
  c->last_fetched = 0;
  c->last_bytes = 0;
  if (active > c->slots)
    return fail(NVFP4_ERR_ARG, "the call routes to %lld experts, more than the cache's %lld slots",
                (long long)active, (long long)c->slots);
  const size_t gu = nvfp4::packed_bytes(nvfp4::geometry(a->inter, a->hidden));
  const size_t dn = nvfp4::packed_bytes(nvfp4::geometry(a->hidden, a->inter));
  // The GPU reads the pinned pools directly (their device-side addresses).
  void* mapped[3] = {nullptr, nullptr, nullptr};
  const void* hosts[3] = {c->host_gate, c->host_up, c->host_down};
  for (int i = 0; i < 3; ++i)
    if (hipHostGetDevicePointer(&mapped[i], const_cast<void*>(hosts[i]), 0) != hipSuccess || !mapped[i])
      return fail(NVFP4_ERR_ARG, "host pools must be pinned host memory mapped for the GPU (hipHostMalloc)");
  const uint8_t* hg = static_cast<const uint8_t*>(mapped[0]);
  const uint8_t* hu = static_cast<const uint8_t*>(mapped[1]);
  const uint8_t* hd = static_cast<const uint8_t*>(mapped[2]);
  std::vector<const void*> csrc;
  std::vector<void*> cdst;
  std::vector<size_t> cbytes;
  std::vector<int64_t> victims;
  uint8_t* dg = static_cast<uint8_t*>(c->dev_gate);
  uint8_t* du = static_cast<uint8_t*>(c->dev_up);
  uint8_t* dd = static_cast<uint8_t*>(c->dev_down);
  int64_t fetched = 0;
  size_t fetched_bytes = 0;
  for (int64_t e = 0; e < a->experts; ++e) {
    if (c->host_counts[e] <= 0 || slot_of[e] >= 0) continue;
    // A miss: a free slot, else the least recently used slot not routed to in this call.
    int64_t v = -1;
    for (int64_t q = 0; q < c->slots; ++q)
      if (expert_in[q] < 0) {
        v = q;
        break;
      }
    if (v < 0)
      for (int64_t q = 0; q < c->slots; ++q)
        if (last_use[q] < now && (v < 0 || last_use[q] < last_use[v])) v = q;
    if (v < 0) return fail(NVFP4_ERR_ARG, "no free cache slot");  // cannot happen when active <= slots
    if (expert_in[v] >= 0) slot_of[expert_in[v]] = -1;
    expert_in[v] = (int32_t)e;
    slot_of[e] = (int32_t)v;
    last_use[v] = now;
    victims.push_back(v);
    csrc.push_back(hg + e * c->stride_gate);
    cdst.push_back(dg + v * c->stride_gate);
    cbytes.push_back(gu);
    csrc.push_back(hu + e * c->stride_up);
    cdst.push_back(du + v * c->stride_up);
    cbytes.push_back(gu);
    csrc.push_back(hd + e * c->stride_down);
    cdst.push_back(dd + v * c->stride_down);
    cbytes.push_back(dn);
    ++fetched;
    fetched_bytes += 2 * gu + dn;
  }
  // After a failure once copies may have been enqueued, the slots they write
  // hold nothing usable: they are emptied in the cache.
  auto drop_victims = [&]() {
    for (int64_t v : victims) {
      if (c->expert_in[v] >= 0) c->slot_of[c->expert_in[v]] = -1;
      c->expert_in[v] = -1;
      c->last_use[v] = 0;
    }
  };
  if (!csrc.empty()) {
    const hipError_t e = nvfp4::launch_expert_copies(csrc.data(), cdst.data(), cbytes.data(), (int)csrc.size(), s);
    if (e != hipSuccess) {
      drop_victims();
      return hip_status(e, "expert copy launch");
    }
  }
  // The slot table (entries of experts not routed to are never read).
  for (int64_t e = 0; e < a->experts; ++e) c->host_slot_stage[e] = slot_of[e] < 0 ? 0 : slot_of[e];
  const hipError_t ec =
      hipMemcpyAsync(c->dev_slot_of, c->host_slot_stage, (size_t)a->experts * 4, hipMemcpyHostToDevice, s);
  if (ec != hipSuccess) {
    drop_victims();
    return hip_status(ec, "slot table copy");
  }
  // Every copy is enqueued: commit the cache's new state.
  c->clock = now;
  std::copy(slot_of.begin(), slot_of.end(), c->slot_of);
  std::copy(expert_in.begin(), expert_in.end(), c->expert_in);
  std::copy(last_use.begin(), last_use.end(), c->last_use);
  c->last_fetched = fetched;
  c->last_bytes = fetched_bytes;
  l.slot_table = c->dev_slot_of;
  return hip_status(nvfp4::launch_moe_experts(l, s), "moe expert launch");
  NVFP4_GUARD_END
}

}  // extern "C"
