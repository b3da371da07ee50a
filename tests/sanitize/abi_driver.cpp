// Calls every entry point of the C ABI with arguments it must refuse before
// any launch, and the host-only ones (sizes, status strings, the expert cache
// reset) with host buffers of exactly the documented sizes, so that an
// AddressSanitizer / UndefinedBehaviorSanitizer build of the library's host
// code reports any out-of-bounds access or undefined operation.  No call here
// reaches a kernel launch.  Exit status 0 and a final "ok" line on success.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "nvfp4.h"

static int failures = 0;
static void expect(int got, int want, const char* what) {
  if (got != want) {
    std::printf("%s: status %d (%s), expected %d\n", what, got, nvfp4_status_str(got), want);
    ++failures;
  }
  (void)nvfp4_last_error();
}

int main() {
  void* A = reinterpret_cast<void*>(0x10000);   // placeholders: never dereferenced on these paths
  void* M = reinterpret_cast<void*>(0x10008);   // misaligned
  const uint16_t* X = static_cast<const uint16_t*>(A);
  size_t sz = 0;
  std::printf("abi %d, %s, %s\n", nvfp4_abi_version(), nvfp4_status_str(5), nvfp4_status_str(99));

  expect(nvfp4_packed_bytes(1024, 1024, &sz), NVFP4_OK, "packed_bytes");
  expect(nvfp4_packed_bytes(4, 40, &sz), NVFP4_ERR_SHAPE, "packed_bytes k%16");
  expect(nvfp4_packed_bytes(4, 64, nullptr), NVFP4_ERR_NULL, "packed_bytes null");
  expect(nvfp4_pack(nullptr, nullptr, 4, 64, nullptr, nullptr), NVFP4_ERR_NULL, "pack null");
  expect(nvfp4_pack(static_cast<uint8_t*>(M), static_cast<uint8_t*>(A), 4, 64, A, nullptr), NVFP4_ERR_ALIGN, "pack align");
  expect(nvfp4_unpack(A, 4, 48 + 8, static_cast<uint8_t*>(A), static_cast<uint8_t*>(A), nullptr), NVFP4_ERR_SHAPE,
         "unpack shape");
  expect(nvfp4_gemv_workspace_bytes(17408, 5120, &sz), NVFP4_OK, "gemv ws");
  expect(nvfp4_gemv_workspace_bytes(64, 32784, &sz), NVFP4_ERR_SHAPE, "gemv ws k limit");
  expect(nvfp4_gemv(A, 64, 64, 1.0f, nullptr, static_cast<float*>(A), nullptr, 0, nullptr), NVFP4_ERR_NULL, "gemv null");
  expect(nvfp4_gemv(A, 4194305, 1280, 1.0f, X, static_cast<float*>(A), A, (size_t)1 << 40, nullptr), NVFP4_ERR_SHAPE,
         "gemv rows");
  for (int64_t m : {2, 32, 64}) {
    expect(nvfp4_gemm_workspace_bytes(m, 5120, 17408, &sz), NVFP4_OK, "gemm ws");
    expect(nvfp4_gemm(A, 64, 64, 1.0f, X, m, 64, A, 60, 1, nullptr, 0, nullptr), NVFP4_ERR_SHAPE, "gemm ldy");
    expect(nvfp4_gemm(A, 64, 64, 1.0f, X, m, 64, A, 64, 9, nullptr, 0, nullptr), NVFP4_ERR_DTYPE, "gemm dtype");
  }
  expect(nvfp4_gemm(A, 5120, 17408, 1.0f, X, 32, 17408, A, 5120, 1, A, 16, nullptr), NVFP4_ERR_WORKSPACE, "gemm ws");
  expect(nvfp4_quantize_workspace_bytes(&sz), NVFP4_OK, "quantize ws");
  expect(nvfp4_quantize(A, NVFP4_F32, 4, 64, 60, static_cast<uint8_t*>(A), static_cast<uint8_t*>(A),
                        static_cast<float*>(A), A, sz, nullptr), NVFP4_ERR_SHAPE, "quantize ldw");
  expect(nvfp4_mx_packed_bytes(512, 5120, &sz), NVFP4_OK, "mx bytes");
  expect(nvfp4_mx_packed_bytes(512, 48, &sz), NVFP4_ERR_SHAPE, "mx bytes k%32");
  expect(nvfp4_w4a4_workspace_bytes(512, 5120, &sz), NVFP4_OK, "w4a4 ws");
  expect(nvfp4_w4a4_gemm(A, 64, 64, 1.0f, X, 4, 64, A, 64, 1, nullptr, 0, nullptr), NVFP4_ERR_WORKSPACE, "w4a4 ws");
  expect(nvfp4_mx_pack(nullptr, nullptr, 4, 64, nullptr, nullptr), NVFP4_ERR_NULL, "mx pack");
  expect(nvfp4_mx_unpack(A, 4, 48, static_cast<uint8_t*>(A), static_cast<uint8_t*>(A), nullptr), NVFP4_ERR_SHAPE,
         "mx unpack");

  // Batches: host arrays of exactly `count` problems.
  std::vector<nvfp4_problem> pr(3);
  for (int i = 0; i < 3; ++i) {
    pr[i].packed = A;
    pr[i].n = 64;
    pr[i].k = 256;
    pr[i].tensor_scale = 1.0f;
    pr[i].x = X;
    pr[i].ldx = 256;
    pr[i].y = reinterpret_cast<void*>(0x20000 + 0x1000 * i);
    pr[i].ldy = 64;
  }
  expect(nvfp4_gemv_batched_workspace_bytes(pr.data(), 3, &sz), NVFP4_OK, "gemv batch ws");
  expect(nvfp4_gemm_batched_workspace_bytes(pr.data(), 3, 32, &sz), NVFP4_OK, "gemm batch ws");
  expect(nvfp4_w4a4_batched_workspace_bytes(pr.data(), 3, 300, &sz), NVFP4_OK, "w4a4 batch ws");
  pr[1].k = 40;
  expect(nvfp4_gemv_batched(pr.data(), 3, nullptr, 0, nullptr), NVFP4_ERR_SHAPE, "gemv batch shape");
  expect(nvfp4_gemv_batched_noalloc(pr.data(), 3, nullptr), NVFP4_ERR_SHAPE, "noalloc shape");
  pr[1].k = 256;
  pr[2].y = pr[0].y;
  expect(nvfp4_gemm_batched(pr.data(), 3, 32, 1, nullptr, 0, nullptr), NVFP4_ERR_ARG, "gemm batch shared y");
  expect(nvfp4_w4a4_batched(pr.data(), 3, 300, 1, nullptr, 0, nullptr), NVFP4_ERR_ARG, "w4a4 batch shared y");
  std::vector<nvfp4_problem> many(65, pr[0]);
  expect(nvfp4_gemv_batched_noalloc(many.data(), 65, nullptr), NVFP4_ERR_ARG, "noalloc count");
  std::vector<nvfp4_problem> big(2, pr[0]);
  big[0].n = (1 << 20) + 64;           // 2 k-groups: 8 MiB + 512 B of partials, past the static scratch
  big[0].k = 2048;
  big[1].y = reinterpret_cast<void*>(0x90000);
  expect(nvfp4_gemv_batched_noalloc(big.data(), 2, nullptr), NVFP4_ERR_WORKSPACE, "noalloc scratch size");

  // The MoE layer: refusals before any launch.
  nvfp4_moe_args a;
  std::memset(&a, 0, sizeof a);
  a.tokens = 32; a.experts = 512; a.top_k = 10; a.hidden = 2048; a.inter = 512;
  a.x = X; a.router_logits = static_cast<const float*>(A);
  a.w_gate = a.w_up = a.w_down = A;
  a.stride_gate = a.stride_up = a.stride_down = 589824;
  a.scale_gate = a.scale_up = a.scale_down = static_cast<const float*>(A);
  a.y = A; a.y_dtype = NVFP4_F32;
  a.topk_ids = static_cast<int32_t*>(A); a.topk_weights = static_cast<float*>(A);
  a.expert_counts = static_cast<int32_t*>(A); a.expert_offsets = static_cast<int32_t*>(A);
  a.perm = static_cast<int32_t*>(A);
  expect(nvfp4_moe_workspace_bytes(&a, &sz), NVFP4_OK, "moe ws");
  a.workspace = A; a.workspace_bytes = 1024;
  expect(nvfp4_moe_grouped(&a, nullptr), NVFP4_ERR_WORKSPACE, "moe ws small");
  a.workspace_bytes = sz;
  a.top_k = 0;
  expect(nvfp4_moe_grouped(&a, nullptr), NVFP4_ERR_ARG, "moe top_k");
  a.top_k = 10;
  a.hidden = 32784;
  expect(nvfp4_moe_grouped(&a, nullptr), NVFP4_ERR_SHAPE, "moe hidden limit");
  a.hidden = 2048;
  a.x = reinterpret_cast<const uint16_t*>(0x10004);
  expect(nvfp4_moe_grouped(&a, nullptr), NVFP4_ERR_ALIGN, "moe align");
  a.x = X;

  // The expert cache: reset writes every state array (exact sizes here).
  nvfp4_expert_cache c;
  std::memset(&c, 0, sizeof c);
  std::vector<int32_t> slot_of(512), expert_in(64);
  std::vector<uint64_t> last_use(64, 7);
  c.experts = 512; c.slots = 64;
  c.slot_of = slot_of.data(); c.expert_in = expert_in.data(); c.last_use = last_use.data();
  c.clock = 99;
  expect(nvfp4_expert_cache_reset(&c), NVFP4_OK, "cache reset");
  for (int32_t v : slot_of) if (v != -1) ++failures;
  for (int32_t v : expert_in) if (v != -1) ++failures;
  for (uint64_t v : last_use) if (v != 0) ++failures;
  expect(nvfp4_moe_streamed(&a, nullptr, nullptr), NVFP4_ERR_NULL, "streamed null cache");
  expect(nvfp4_moe_streamed(&a, &c, nullptr), NVFP4_ERR_ARG, "streamed pools");

  std::printf(failures ? "FAILED %d\n" : "ok\n", failures);
  return failures ? 1 : 0;
}
