/*
 * nvfp4.h -- NVFP4 weight x bf16 activation products on AMD Instinct MI355X (gfx950).
 *
 * The only way into the library (libnvfp4.so).  A flat C boundary with plain
 * pointers and sizes, as the Ignis README's introduction describes for its own
 * kernel library ("a flat, device-resident step-level C ABI" under the Rust
 * host) and as the imp README's "Using it" section offers its C library.
 *
 * ---- The weight format (NVFP4) ----------------------------------------------
 * An [N][K] weight matrix W (N output rows, K inputs, K a multiple of 16) is
 *   codes   uint8 [N][K/2]   two 4-bit E2M1 codes per byte, element k = 2i in
 *                            the low nibble of byte i, k = 2i+1 in the high nibble
 *   scales  uint8 [N][K/16]  one FP8 E4M3FN scale per 16 consecutive K of a row
 *   s_t     float            one fp32 per-tensor scale
 * and W[n][k] = s_t * e2m1(code) * e4m3(scale[n][k/16]).  E2M1 takes the 16
 * values {0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6} (OCP MX v1.0); E4M3FN has no
 * infinities, 0x7F/0xFF are NaN (a NaN scale makes its block NaN), subnormals
 * are m * 2^-9.  The imp README ("How does it work?") keeps weights in this
 * 4-bit format and computes on it directly instead of unpacking to 16 bits.
 *
 * ---- Conventions for every call ---------------------------------------------
 *  - Pointers are DEVICE memory unless marked (host).  The caller owns all
 *    memory; the library never allocates or frees it, and synchronises only
 *    in nvfp4_moe_streamed (one read-back of the expert counts).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued on
 *    it and runs asynchronously; results are ready after the caller
 *    synchronises with the stream.
 *  - Arguments are validated on the host before anything is enqueued.  A
 *    failed check returns its status and enqueues nothing, in the spirit of the
 *    imp README's "Will it fit?" (refuse rather than run wrong).
 *  - Device pointers to bulk data (codes, scales, packed buffers, activations,
 *    outputs, workspaces) must be 16-byte aligned; the small per-token and
 *    per-expert arrays of the MoE call (logits, tensor scales, ids, weights,
 *    counts, offsets, perm) 4-byte aligned (NVFP4_ERR_ALIGN otherwise).
 *  - A launch failure returns NVFP4_ERR_HIP; nvfp4_last_error() then holds the
 *    HIP error text.  Faults during execution surface at the caller's next
 *    synchronisation.
 *  - No C++ exception crosses this boundary.  The library keeps no mutable
 *    global state apart from the thread-local error text and, once
 *    nvfp4_gemv_batched_noalloc has run on a device, that device's address of
 *    the library's static scratch array.
 *  - Workspaces: calls that split a reduction across workgroups take a caller
 *    workspace of at least the size the matching *_workspace_bytes() returns.
 *    For nvfp4_gemv / nvfp4_gemm its first 262144 bytes are counters that must
 *    be all zero before the first use (allocate it zeroed); every call leaves
 *    them zero again, so one workspace serves calls of any shape in stream
 *    order.  Calls that share one workspace must not run concurrently.
 *    nvfp4_gemv / nvfp4_gemm accept n up to 4194304 rows.
 *  - Products accumulate in fp32.  Every product of a weight and a bf16
 *    activation is exact in fp32; the per-tensor scale is applied after
 *    accumulation.  The sum order is fixed, so repeated calls give
 *    bit-identical results (no floating-point atomics anywhere).
 */
#ifndef NVFP4_H_
#define NVFP4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_ABI_VERSION 1

typedef enum nvfp4_status {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = 1,       /* a required pointer is NULL */
  NVFP4_ERR_SHAPE = 2,      /* a size is negative, K % 16 != 0, a leading dimension too small, ... */
  NVFP4_ERR_ALIGN = 3,      /* a device pointer (or a byte stride) is not 16-byte aligned */
  NVFP4_ERR_DTYPE = 4,      /* unknown nvfp4_dtype */
  NVFP4_ERR_WORKSPACE = 5,  /* workspace missing or smaller than required */
  NVFP4_ERR_ARG = 6,        /* other invalid argument (top_k > experts, stride too small, ...) */
  NVFP4_ERR_HIP = 7         /* a HIP launch failed; see nvfp4_last_error() */
} nvfp4_status;

typedef enum nvfp4_dtype {
  NVFP4_F32 = 0,            /* float32 */
  NVFP4_BF16 = 1            /* bfloat16, rounded to nearest even */
} nvfp4_dtype;

/* NVFP4_ABI_VERSION of the built library. */
int nvfp4_abi_version(void);

/* A static string naming `status` ("NVFP4_OK", ...); "unknown status" otherwise. */
const char* nvfp4_status_str(int status);

/* Thread-local text describing this thread's last failed call ("" if none). */
const char* nvfp4_last_error(void);

/* ---- offline repack -------------------------------------------------------
 * The packed buffer is the only form the product kernels read.  Its layout is
 * private to the library (a gfx950 tile layout); only nvfp4_packed_bytes() and
 * nvfp4_unpack() expose it.  It holds exactly the NVFP4 information (0.5625
 * bytes per weight) plus zero padding of N to a multiple of 64 and of K to a
 * multiple of 256.  imp converts weights once at first load and caches the
 * result (imp README, "Install"); packing is likewise a one-off step outside
 * the timed path.
 */

/* (host) *bytes = size of the packed buffer for an [n][k] matrix.
 * n >= 0, k >= 0, k % 16 == 0. */
int nvfp4_packed_bytes(int64_t n, int64_t k, size_t* bytes);

/* Repack canonical codes [n][k/2] and scales [n][k/16] (both row-major,
 * contiguous) into `packed` (nvfp4_packed_bytes() bytes, fully written,
 * padding included).  n == 0 or k == 0 is a no-op. */
int nvfp4_pack(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k,
               void* packed, void* stream);

/* The inverse of nvfp4_pack (a test hook): writes codes [n][k/2] and scales [n][k/16]. */
int nvfp4_unpack(const void* packed, int64_t n, int64_t k, uint8_t* codes, uint8_t* scales,
                 void* stream);

/* ---- quantiser (the step before nvfp4_pack) ---------------------------------
 * Encodes an [n][k] weight matrix, fp32 or bf16 (w_dtype), rows ldw elements
 * apart, as canonical NVFP4: codes [n][k/2], scales [n][k/16] (the layouts
 * nvfp4_pack() reads) and one fp32 per-tensor scale written to *tensor_scale
 * (device memory).  The pages keep weights in NVFP4 and convert them once
 * (imp README, "How does it work?"); they leave the encoder open.  This one:
 *   s_t      = amax / 2688  (amax: the largest |w|; 6 * 448 = 2688 puts it on the
 *              largest E2M1 value times the largest E4M3 value; 1 if all zero)
 *   scale_b  = E4M3FN nearest to amax_b / (6 * s_t)   (amax_b: block b's largest |w|)
 *   code     = E2M1 nearest to |w| / (e4m3(scale_b) * s_t), sign bit = w's sign bit
 * Nearest means ties to an even mantissa, saturating at 448 and 6; a block
 * whose scale is 0 gets code 0 throughout.  Every quotient and product is a
 * single-precision operation in the order shown, so results are bit-exact and
 * deterministic.  Inputs must be finite (NaN or infinity give unspecified
 * bytes).  n >= 0, k % 16 == 0, ldw >= k and ldw % 8 == 0; w, codes, scales
 * 16-byte aligned, tensor_scale 4-byte aligned; workspace: at least
 * nvfp4_quantize_workspace_bytes() bytes, 16-byte aligned, no initial contents
 * required.  n == 0 or k == 0 is a no-op (nothing written).
 */
int nvfp4_quantize_workspace_bytes(size_t* bytes /* host */);
int nvfp4_quantize(const void* w, int w_dtype, int64_t n, int64_t k, int64_t ldw, uint8_t* codes,
                   uint8_t* scales, float* tensor_scale, void* workspace, size_t workspace_bytes,
                   void* stream);

/* ---- GEMV, one activation vector ----------------------------------------
 * y[j] = s_t * sum_k e2m1(c[j][k]) * e4m3(sigma[j][k/16]) * x[k],   j < n.
 * x: bf16 bit patterns [k];  y: float32 [n].
 * The memory-bound decode product: the Ignis README ("The decode round")
 * measures its decode round as weight streaming at the card's bandwidth, the
 * backbone GEMM at full roofline.  n == 0 or k == 0: y is zero-filled (k == 0)
 * or nothing is done (n == 0).
 */
int nvfp4_gemv_workspace_bytes(int64_t n, int64_t k, size_t* bytes /* host */);
int nvfp4_gemv(const void* packed, int64_t n, int64_t k, float tensor_scale,
               const uint16_t* x, float* y, void* workspace, size_t workspace_bytes,
               void* stream);

/* ---- GEMM, m activation rows -----------------------------------------
 * y[i][j] = s_t * sum_k W[j][k] * x[i][k],   i < m, j < n.
 * x: bf16 bit patterns, row i at x + i*ldx (ldx >= k, ldx % 8 == 0);
 * y: y_dtype, row i at y + i*ldy elements (ldy >= n).
 * m <= 2 runs the GEMV's mapping with both rows in one launch (each row's
 * outputs bit-identical to nvfp4_gemv of that row, fp32, before the output
 * rounding); 2 < m <= 32 runs the skinny (decode-batch) kernel on the matrix
 * cores: the imp README's 32-users table and the Ignis README's batch-wide
 * decode round of widths 1..8.  Larger m runs the prefill kernel, which
 * dequantises each weight x block-scale exactly to bf16 and runs bf16 MFMA.
 * m == 0 or n == 0 is a no-op.
 */
int nvfp4_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k, size_t* bytes /* host */);
int nvfp4_gemm(const void* packed, int64_t n, int64_t k, float tensor_scale,
               const uint16_t* x, int64_t m, int64_t ldx,
               void* y, int64_t ldy, int y_dtype,
               void* workspace, size_t workspace_bytes, void* stream);

/* ---- W4A4 prefill on the FP4 matrix cores (an approximation) -------------
 * The pages' prefill runs native FP4 on weights and activations (imp README,
 * "How does it work?").  gfx950's FP4 matrix instruction takes the OCP MX
 * format: E2M1 values with one power-of-two (E8M0) scale per 32 k.  Both
 * operands are requantised to it -- so this product approximates the NVFP4 one
 * (for N(0,1) activations a median of ~0.3 % and at most a few % of sum|w x|
 * away from it) and is defined by its own rule:
 *   block of 32: X = 2^(floor(log2 amax) - 2), exponent clamped to [-127, 127];
 *   code = E2M1 nearest v / X (ties to even, +-6 beyond 6, sign of v); an
 *   all-zero block has X = 2^-127 and zero codes;
 *   weights: the NVFP4 values e2m1 * e4m3 (s_t left out) in blocks along k;
 *   activations: the bf16 values in blocks along k;
 *   y[i][j] = s_t * sum_k w'[j][k] x'[i][k]  (fp32 accumulation).
 * k % 32 == 0, n within the product calls' row limit.  nvfp4_mx_pack()
 * converts a canonical NVFP4 matrix (once, like nvfp4_pack) into "MX tiles" of
 * nvfp4_mx_packed_bytes() bytes; nvfp4_w4a4_gemm() quantises x into the
 * workspace and runs the product on the prefill's stream-K schedule.  The
 * workspace (at least nvfp4_w4a4_workspace_bytes(m, k), 16-byte aligned) holds
 * the schedule's counters and partial sums first -- like the gemm workspace,
 * all zero before the first use and left so by every call -- and then x's MX
 * tiles, at byte offset nvfp4_w4a4_workspace_bytes(m, k) -
 * nvfp4_mx_packed_bytes(m, k) (the same for every m and k), which stay there
 * after the call.  m <= 2^24.  nvfp4_mx_unpack() (a test hook) turns MX tiles
 * back into codes [rows][k/2] and E8M0 scales [rows][k/32].
 */
int nvfp4_mx_packed_bytes(int64_t rows, int64_t k, size_t* bytes /* host */);
int nvfp4_mx_pack(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k, void* mx_packed, void* stream);
int nvfp4_mx_unpack(const void* mx_packed, int64_t rows, int64_t k, uint8_t* codes, uint8_t* scales, void* stream);
int nvfp4_w4a4_workspace_bytes(int64_t m, int64_t k, size_t* bytes /* host */);
int nvfp4_w4a4_gemm(const void* mx_packed, int64_t n, int64_t k, float tensor_scale, const uint16_t* x, int64_t m,
                    int64_t ldx, void* y, int64_t ldy, int y_dtype, void* workspace, size_t workspace_bytes,
                    void* stream);

/* ---- Batched products: several independent matrices in one launch ----------
 * A decode step multiplies several weight matrices of a layer by their own
 * activations (gate, up, down, QKV, O); the Ignis README's decode round runs
 * them as one replayed sequence.  These calls take a host array of problems
 * and compute each as nvfp4_gemv / nvfp4_gemm would, but as one launch per
 * eight problems, so that the launch ramp and the cross-workgroup reduction
 * tail are paid once per batch and the split of K is balanced over the whole
 * batch.  GEMV results are bit-identical to single calls; a GEMM of a batch may
 * split K differently from a single call, so its results meet the same error
 * bound but may differ in the last bits.  Problems must not share outputs.
 * The workspace rules are those of nvfp4_gemv / nvfp4_gemm.
 */
typedef struct nvfp4_problem {
  const void* packed;       /* packed weights of an [n][k] matrix */
  int64_t n, k;
  float tensor_scale;
  const uint16_t* x;        /* bf16 activations: [k] (gemv) or [m][ldx] (gemm) */
  int64_t ldx;              /* gemm only: row stride of x in elements (>= k, multiple of 8) */
  void* y;                  /* fp32 [n] (gemv) or y_dtype [m][ldy] (gemm) */
  int64_t ldy;              /* gemm only: row stride of y in elements (>= n) */
} nvfp4_problem;

int nvfp4_gemv_batched_workspace_bytes(const nvfp4_problem* problems /* host */, int count,
                                       size_t* bytes /* host */);
int nvfp4_gemv_batched(const nvfp4_problem* problems /* host */, int count, void* workspace,
                       size_t workspace_bytes, void* stream);
/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops that forbid allocation): nvfp4_gemv_batched without
 * a workspace argument.  Its split-K counters and partial sums live in a
 * static device array of the library, 8 MiB + 256 KiB on each GPU the library
 * runs on, held until the process ends; the call allocates nothing.  A batch
 * whose nvfp4_gemv_batched_workspace_bytes() exceeds that returns
 * NVFP4_ERR_WORKSPACE; count must be <= 64 (NVFP4_ERR_ARG).  Results are
 * bit-identical to nvfp4_gemv_batched.  Every call on a GPU shares that GPU's
 * array: calls that may overlap on one GPU (other streams, other threads) race
 * and must be serialised by the caller.  The first call on a device also
 * enqueues, on `stream`, a fill of the array's counters with zeros; every call
 * leaves them zero.  Other validation and statuses as nvfp4_gemv_batched. */
int nvfp4_gemv_batched_noalloc(const nvfp4_problem* problems /* host */, int count, void* stream);
/* All problems of a batch share m and y_dtype. */
int nvfp4_gemm_batched_workspace_bytes(const nvfp4_problem* problems /* host */, int count, int64_t m,
                                       size_t* bytes /* host */);
int nvfp4_gemm_batched(const nvfp4_problem* problems /* host */, int count, int64_t m, int y_dtype,
                       void* workspace, size_t workspace_bytes, void* stream);
/* W4A4 batch (the W4A4 rule above for each problem; `packed` holds the MX
 * tiles of nvfp4_mx_pack): one stream-K launch per eight problems, so that
 * the split tiles' fix-up is shared like the gemm batch's.  The workspace holds
 * the schedule's counters and partial sums (zero before the first use, left
 * so) and then each problem's x as MX tiles, in problem order.  k % 32 == 0,
 * m <= 2^24.  Validation and statuses as nvfp4_gemm_batched (NVFP4_ERR_SHAPE
 * also for k % 32 != 0); n == 0 problems are skipped, k == 0 ones get zero
 * outputs. */
int nvfp4_w4a4_batched_workspace_bytes(const nvfp4_problem* problems /* host */, int count, int64_t m,
                                       size_t* bytes /* host */);
int nvfp4_w4a4_batched(const nvfp4_problem* problems /* host */, int count, int64_t m, int y_dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

/* ---- top-k routed mixture-of-experts layer ----------------------------
 * Per token t (CHImp-Alpha-v1.0 model card, "How it fits on one GPU": each
 * token is routed to 10 of 512 experts and only those experts' weights are read):
 *   ids[t][0..top_k)  the top_k experts by router logit, descending, equal
 *                     logits ranked by smaller expert id (logits must not be NaN);
 *   g[t][j]           exp(l_j - l_0) / sum_j' exp(l_j' - l_0)  (softmax over the
 *                     selected logits, fp32);
 *   for each j, with e = ids[t][j]:
 *     h_j = bf16( silu(Wg_e x_t) * (Wu_e x_t) ),  silu(z) = z / (1 + exp(-z)),
 *     d_j = Wd_e h_j                                (fp32)
 *   y[t] = sum_{j = 0..top_k-1} g[t][j] * d_j      (summed in j order).
 * Wg_e, Wu_e are [inter][hidden], Wd_e is [hidden][inter], each packed with
 * nvfp4_pack(); expert e's packed matrix starts e*stride bytes into its pool.
 * Grouping outputs (bit-exact, deterministic):
 *   expert_counts[e]   number of (t, j) with ids[t][j] == e
 *   expert_offsets[e]  exclusive prefix sum of the counts (offsets[E] = tokens*top_k)
 *   perm[p]            the flat indices f = t*top_k + j ordered by expert, and by f
 *                      within an expert (a stable sort by expert id)
 * Optional stage outputs (NULL to skip), rows in perm order p:
 *   dbg_gate, dbg_up  fp32 [tokens*top_k][inter]   Wg_e x_t, Wu_e x_t (tensor scale applied)
 *   dbg_h             bf16 [tokens*top_k][inter]
 *   dbg_down          fp32 [tokens*top_k][hidden]  d_j
 * tokens == 0 is a no-op.  Experts with no tokens are never read.
 */
typedef struct nvfp4_moe_args {
  int64_t tokens, experts, top_k, hidden, inter;
  const uint16_t* x;              /* bf16 [tokens][hidden] */
  const float* router_logits;     /* fp32 [tokens][experts] */
  const void* w_gate;             /* packed pools */
  const void* w_up;
  const void* w_down;
  size_t stride_gate, stride_up, stride_down;   /* bytes between experts in each pool */
  const float* scale_gate;        /* per-expert tensor scales, device fp32 [experts] */
  const float* scale_up;
  const float* scale_down;
  void* y;                        /* [tokens][hidden], y_dtype */
  int y_dtype;
  int32_t* topk_ids;              /* [tokens][top_k] (out) */
  float* topk_weights;            /* [tokens][top_k] (out) */
  int32_t* expert_counts;         /* [experts] (out) */
  int32_t* expert_offsets;        /* [experts + 1] (out) */
  int32_t* perm;                  /* [tokens * top_k] (out) */
  float* dbg_gate;                /* optional, see above */
  float* dbg_up;
  uint16_t* dbg_h;
  float* dbg_down;
  void* workspace;
  size_t workspace_bytes;
} nvfp4_moe_args;

int nvfp4_moe_workspace_bytes(const nvfp4_moe_args* args /* host */, size_t* bytes /* host */);
int nvfp4_moe_grouped(const nvfp4_moe_args* args /* host */, void* stream);

/* ---- routed experts streamed from host memory --------------------------
 * The imp README runs mixture-of-experts models larger than the card with the
 * experts in host RAM ("Will it fit?"); only the routed experts' weights are
 * needed per token (CHImp-Alpha-v1.0 model card, "How it fits on one GPU").
 * Here every expert's packed gate, up and down matrices stay in pinned host
 * pools; a device cache of `slots` expert slots keeps recently used experts.
 * nvfp4_moe_streamed() routes and groups on the GPU, reads the expert counts
 * back (it synchronises `stream` once), copies each routed expert that is not
 * cached into a free slot or, failing that, the least recently used slot no
 * routed expert of this call occupies -- one kernel on `stream` reads all of
 * the call's missing matrices from the pinned pools over PCIe -- and then
 * runs the expert GEMMs on the slots.  Outputs are bit-identical to
 * nvfp4_moe_grouped() with the same weights device-resident.
 *
 * The caller owns every buffer.  Device: dev_gate/dev_up/dev_down (slot s at
 * s * stride_*, 16-byte aligned strides of at least the packed matrix size),
 * dev_slot_of [experts] int32.  Pinned host memory mapped for the GPU
 * (hipHostMalloc; NVFP4_ERR_ARG otherwise): host_gate/host_up/
 * host_down (expert e at e * stride_*, same strides), host_counts [experts]
 * and host_slot_stage [experts] int32.  Host (any): slot_of [experts] int32,
 * expert_in [slots] int32, last_use [slots] uint64 -- the cache state, set up
 * by nvfp4_expert_cache_reset() and kept across calls.  Calls sharing a cache
 * must be issued in order on one stream.
 * In nvfp4_moe_streamed(), args->w_gate/w_up/w_down and the strides must be
 * the cache's device slot pools and strides; every other argument is as for
 * nvfp4_moe_grouped().  If a call routes to more experts than there are
 * slots it returns NVFP4_ERR_ARG after routing (topk_ids, topk_weights,
 * expert_counts, expert_offsets and perm are then valid, y is not).
 * last_active / last_fetched / last_bytes: the routed experts, the experts
 * copied and the bytes copied by the last call.
 */
typedef struct nvfp4_expert_cache {
  int64_t experts, slots;
  const void* host_gate;
  const void* host_up;
  const void* host_down;
  void* dev_gate;
  void* dev_up;
  void* dev_down;
  size_t stride_gate, stride_up, stride_down;
  int32_t* dev_slot_of;
  int32_t* host_counts;
  int32_t* host_slot_stage;
  int32_t* slot_of;
  int32_t* expert_in;
  uint64_t* last_use;
  uint64_t clock;
  int64_t last_active, last_fetched;
  size_t last_bytes;
} nvfp4_expert_cache;

/* Empty the cache: every slot free, every expert uncached, statistics zero. */
int nvfp4_expert_cache_reset(nvfp4_expert_cache* cache /* host */);
int nvfp4_moe_streamed(const nvfp4_moe_args* args /* host */, nvfp4_expert_cache* cache /* host */, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4_H_ */
