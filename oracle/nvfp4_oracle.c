/*
 * NVFP4 weight x bf16 activation product: the CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. The GPU path shares no
 * code with it, and it shares none with the GPU path.
 *
 * What it computes, and where that is defined:
 *   - NVFP4 weights: every weight is a 4-bit E2M1 code, every run of 16
 *     consecutive input (K) elements of one output row shares one E4M3 scale
 *     byte, and the whole matrix has one fp32 per-tensor scale.  The weight's
 *     value is  s_t * e2m1(code) * e4m3(scale).  The imp README ("How does it
 *     work?") keeps weights in this format and computes on it directly; the
 *     E2M1 and E4M3 encodings themselves are those of the OCP Microscaling
 *     Formats v1.0 (FP4 E2M1) and OCP 8-bit Floating Point (E4M3FN) specs.
 *   - The product is the plain definition y[m][n] = sum_k W[n][k] * x[m][k]
 *     evaluated in fp64.  Every product of a dequantised weight and a bf16
 *     activation is exact in fp64; only the summation rounds, by at most
 *     (K-1) * 2^-53 * sum_k |W[n][k] x[m][k]|.
 *   - The mixture-of-experts layer: each token goes to the 10 of 512 experts
 *     with the largest router logits (CHImp-Alpha-v1.0 model card, "How it fits
 *     on one GPU"), the routing weights are a softmax over the selected logits,
 *     each expert is a SiLU-gated unit (gate, up, down), and a token's output is
 *     the routing-weighted sum of its experts' outputs.
 *
 * Readings taken where the pages are silent (each is listed in the design notes):
 *   - element 2i of a row sits in the low nibble of byte i, element 2i+1 in the
 *     high nibble; scales are [N][K/16] row-major;
 *   - E4M3 is the FN variant: no infinities, 0x7F/0xFF are NaN, subnormals
 *     are m * 2^-9;
 *   - top-k ranks by fp32 logit, descending, ties going to the smaller expert id;
 *   - the expert activation is h = silu(gate) * up, silu(z) = z / (1 + e^-z);
 *   - the permutation orders the flat (token*top_k + j) indices stably by expert.
 *
 * Parity pins (tests marked "not gpu"): the E2M1 table against a fixture of the
 * spec's values, the E4M3 decoder against torch.float8_e4m3fn for all 256
 * bytes, the product against torch.float64 matmul of an independently decoded
 * matrix, identity / one-hot / integer-exact closed forms, the routing against
 * a brute-force sort and numpy's stable argsort.
 *
 * Plain loops, fp64, OpenMP over output rows. Built with -O2, no fast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- element decoders --------------------------------------------------- */

/* FP4 E2M1 magnitudes for codes 0..7 (sign is bit 3): OCP MX v1.0, E2M1. */
static const double kE2M1Magnitude[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double nvo_e2m1(uint32_t code) {
  double mag = kE2M1Magnitude[code & 7u];
  return (code & 8u) ? -mag : mag;
}

/* FP8 E4M3FN: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0. */
double nvo_e4m3(uint32_t byte) {
  uint32_t s = (byte >> 7) & 1u, e = (byte >> 3) & 15u, m = byte & 7u;
  double v;
  if (e == 15u && m == 7u) return NAN;
  if (e == 0u) v = ldexp((double)m, -9);          /* subnormal: m/8 * 2^(1-7) */
  else v = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
  return s ? -v : v;
}

/* bf16 -> fp64, exact: a bf16 is the top half of an fp32. */
double nvo_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Weight (n, k) of an [N][K] NVFP4 matrix in canonical layout, times s_t. */
static double weight(const uint8_t* codes, const uint8_t* scales, int64_t k_dim,
                     double st, int64_t n, int64_t k) {
  uint8_t byte = codes[n * (k_dim / 2) + k / 2];
  uint32_t code = (k & 1) ? (byte >> 4) : (byte & 15u);
  double sc = nvo_e4m3(scales[n * (k_dim / 16) + k / 16]);
  return st * nvo_e2m1(code) * sc;
}

/* Dequantise the whole matrix: w[n][k] = s_t * e2m1 * e4m3, fp64. */
void nvo_dequant(const uint8_t* codes, const uint8_t* scales, int64_t n_dim,
                 int64_t k_dim, float st, double* w) {
  for (int64_t n = 0; n < n_dim; ++n)
    for (int64_t k = 0; k < k_dim; ++k)
      w[n * k_dim + k] = weight(codes, scales, k_dim, (double)st, n, k);
}

/* ---- dense product ------------------------------------------------------ */

/*
 * y[m][j] = sum_k W[rows[j]][k] * x[m][k] and s[m][j] = sum_k |W[rows[j]][k] * x[m][k]|
 * for the output rows listed in `rows` (all N rows, in order, when rows is NULL).
 * x is bf16 [M][ldx]; y and s are fp64 [M][nrows] (s may be NULL).
 */
void nvo_gemm(const uint8_t* codes, const uint8_t* scales, int64_t n_dim, int64_t k_dim,
              float st, const uint16_t* x, int64_t m_dim, int64_t ldx,
              const int64_t* rows, int64_t nrows, double* y, double* s, int nthreads) {
  if (rows == NULL) nrows = n_dim;
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel num_threads(nthreads)
  {
    double* w = (double*)malloc(sizeof(double) * (size_t)(k_dim > 0 ? k_dim : 1));
#pragma omp for schedule(static)
    for (int64_t j = 0; j < nrows; ++j) {
      int64_t n = rows ? rows[j] : j;
      for (int64_t k = 0; k < k_dim; ++k) w[k] = weight(codes, scales, k_dim, (double)st, n, k);
      for (int64_t m = 0; m < m_dim; ++m) {
        double acc = 0.0, mag = 0.0;
        for (int64_t k = 0; k < k_dim; ++k) {
          double p = w[k] * nvo_bf16(x[m * ldx + k]);
          acc += p;
          mag += fabs(p);
        }
        y[m * nrows + j] = acc;
        if (s) s[m * nrows + j] = mag;
      }
    }
    free(w);
  }
}

/* ---- mixture-of-experts routing ---------------------------------------- */

typedef struct { float logit; int32_t id; } ranked;

/* Descending logit; equal logits: smaller expert id first. */
static int rank_cmp(const void* pa, const void* pb) {
  const ranked* a = (const ranked*)pa;
  const ranked* b = (const ranked*)pb;
  if (a->logit > b->logit) return -1;
  if (a->logit < b->logit) return 1;
  return (a->id < b->id) ? -1 : (a->id > b->id);
}

/*
 * Per token: the top_k experts by logit (full sort of all E) and their routing
 * weights g_j = exp(l_j - l_0) / sum_j' exp(l_j' - l_0), fp64 (a softmax taken
 * over the selected logits, which equals the full softmax renormalised over them).
 */
void nvo_route(const float* logits, int64_t tokens, int64_t experts, int64_t top_k,
               int32_t* ids, double* g) {
  ranked* r = (ranked*)malloc(sizeof(ranked) * (size_t)(experts > 0 ? experts : 1));
  for (int64_t t = 0; t < tokens; ++t) {
    for (int64_t e = 0; e < experts; ++e) { r[e].logit = logits[t * experts + e]; r[e].id = (int32_t)e; }
    qsort(r, (size_t)experts, sizeof(ranked), rank_cmp);
    double lmax = (double)r[0].logit, denom = 0.0;
    for (int64_t j = 0; j < top_k; ++j) denom += exp((double)r[j].logit - lmax);
    for (int64_t j = 0; j < top_k; ++j) {
      ids[t * top_k + j] = r[j].id;
      g[t * top_k + j] = exp((double)r[j].logit - lmax) / denom;
    }
  }
  free(r);
}

/*
 * Group the flat assignments f = t*top_k + j by expert:
 *   counts[e]  = number of f with ids[f] == e
 *   offsets[e] = sum of counts[0..e-1]   (offsets[E] = tokens*top_k)
 *   perm[p]    = the f's listed expert by expert, each expert's f's ascending
 *   pos[f]     = the p with perm[p] == f
 */
void nvo_group(const int32_t* ids, int64_t tokens, int64_t top_k, int64_t experts,
               int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* pos) {
  int64_t total = tokens * top_k;
  for (int64_t e = 0; e < experts; ++e) counts[e] = 0;
  for (int64_t f = 0; f < total; ++f) counts[ids[f]] += 1;
  offsets[0] = 0;
  for (int64_t e = 0; e < experts; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int64_t p = 0;
  for (int64_t e = 0; e < experts; ++e)
    for (int64_t f = 0; f < total; ++f)
      if (ids[f] == e) { perm[p] = (int32_t)f; if (pos) pos[f] = (int32_t)p; ++p; }
}

/* silu(z) = z / (1 + e^-z) */
double nvo_silu(double z) { return z / (1.0 + exp(-z)); }

/*
 * The whole expert layer in fp64.  Expert e's matrices are at
 *   gate: codes gc + e*(inter*hidden/2), scales gs + e*(inter*hidden/16), [inter][hidden]
 *   up:   the same shapes in uc/us
 *   down: codes dc + e*(hidden*inter/2), scales ds + e*(hidden*inter/16), [hidden][inter]
 * with per-tensor scales sg[e], su[e], sd[e].  x is bf16 [tokens][hidden].
 * Outputs: ids [tokens][top_k], g fp64 [tokens][top_k], y fp64 [tokens][hidden],
 * and ybound[t][o] = sum_j g_j * sum_i |Wd[o][i] * h_j[i]|.
 */
void nvo_moe(const uint8_t* gc, const uint8_t* gs, const float* sg,
             const uint8_t* uc, const uint8_t* us, const float* su,
             const uint8_t* dc, const uint8_t* ds, const float* sd,
             const uint16_t* x, const float* logits,
             int64_t tokens, int64_t experts, int64_t top_k, int64_t hidden, int64_t inter,
             int32_t* ids, double* g, double* y, double* ybound, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  nvo_route(logits, tokens, experts, top_k, ids, g);
  int64_t wgu = inter * hidden;   /* weights per gate / up matrix */
  int64_t wd = hidden * inter;    /* weights per down matrix */
  for (int64_t i = 0; i < tokens * hidden; ++i) { y[i] = 0.0; ybound[i] = 0.0; }
#pragma omp parallel num_threads(nthreads)
  {
    double* h = (double*)malloc(sizeof(double) * (size_t)(inter > 0 ? inter : 1));
#pragma omp for schedule(dynamic)
    for (int64_t t = 0; t < tokens; ++t) {
      for (int64_t j = 0; j < top_k; ++j) {
        int64_t e = ids[t * top_k + j];
        const uint8_t* gce = gc + e * (wgu / 2); const uint8_t* gse = gs + e * (wgu / 16);
        const uint8_t* uce = uc + e * (wgu / 2); const uint8_t* use = us + e * (wgu / 16);
        const uint8_t* dce = dc + e * (wd / 2);  const uint8_t* dse = ds + e * (wd / 16);
        for (int64_t i = 0; i < inter; ++i) {
          double ga = 0.0, ua = 0.0;
          for (int64_t k = 0; k < hidden; ++k) {
            double xv = nvo_bf16(x[t * hidden + k]);
            ga += weight(gce, gse, hidden, (double)sg[e], i, k) * xv;
            ua += weight(uce, use, hidden, (double)su[e], i, k) * xv;
          }
          h[i] = nvo_silu(ga) * ua;
        }
        double gj = g[t * top_k + j];
        for (int64_t o = 0; o < hidden; ++o) {
          double d = 0.0, mag = 0.0;
          for (int64_t i = 0; i < inter; ++i) {
            double p = weight(dce, dse, inter, (double)sd[e], o, i) * h[i];
            d += p;
            mag += fabs(p);
          }
          y[t * hidden + o] += gj * d;
          ybound[t * hidden + o] += gj * mag;
        }
      }
    }
    free(h);
  }
}

int nvo_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---- NVFP4 quantiser: weights -> codes, block scales, tensor scale ----------
 *
 * The step before the repack: the imp README ("How does it work?") keeps
 * weights in NVFP4 and converts them once; the pages do not spell out the
 * encoder.  The readings taken (each listed in the design notes):
 *   - the per-tensor scale maps the matrix's largest magnitude amax onto the
 *     largest value the two levels hold, 6 (E2M1) times 448 (E4M3):
 *     s_t = amax / 2688 as an fp32 division, and 1 for an all-zero matrix;
 *   - block b's scale byte is the E4M3FN value nearest to amax_b / (6 s_t)
 *     (amax_b: the block's largest magnitude), ties going to the even
 *     mantissa; above 448 the nearest value is 448;
 *   - element w's code: the E2M1 magnitude nearest to |w| / (e4m3(scale_b) s_t),
 *     ties to the even mantissa, values above 6 giving 6; the code's sign bit
 *     is w's sign bit; a block whose scale byte is 0 gets code 0 throughout;
 *   - these quotients and products are single-precision operations, in the
 *     order written: the integer decisions are taken in fp32, the precision
 *     the GPU encoder works in.  Inputs are finite.
 * The rounding is written as a search for the nearest table value (plain and
 * slow, on purpose).
 */

/* Nearest non-negative finite E4M3FN byte (0x00..0x7E) to q >= 0; ties to the
 * even byte (the byte's low bit is the mantissa's). */
static uint32_t e4m3_nearest(float q) {
  uint32_t best = 0;
  double bd = fabs((double)q);
  for (uint32_t b = 1; b <= 0x7Eu; ++b) {
    const double d = fabs((double)q - nvo_e4m3(b));
    if (d < bd || (d == bd && (b & 1u) == 0u)) {
      best = b;
      bd = d;
    }
  }
  return best;
}

/* Nearest E2M1 magnitude code (0..7) to a >= 0; ties to the even code. */
static uint32_t e2m1_nearest(float a) {
  uint32_t best = 0;
  double bd = fabs((double)a);
  for (uint32_t c = 1; c < 8u; ++c) {
    const double d = fabs((double)a - kE2M1Magnitude[c]);
    if (d < bd || (d == bd && (c & 1u) == 0u)) {
      best = c;
      bd = d;
    }
  }
  return best;
}

static float input_value(const void* w, int bf16, int64_t i) {
  if (bf16) return (float)nvo_bf16(((const uint16_t*)w)[i]);
  return ((const float*)w)[i];
}

/* The per-tensor scale of an [n][k] matrix (row stride ldw elements);
 * bf16 != 0: bf16 bit patterns, else fp32. */
float nvo_tensor_scale(const void* w, int bf16, int64_t n, int64_t k, int64_t ldw) {
  float amax = 0.0f;
  for (int64_t r = 0; r < n; ++r)
    for (int64_t c = 0; c < k; ++c) {
      const float a = fabsf(input_value(w, bf16, r * ldw + c));
      if (a > amax) amax = a;
    }
  return amax > 0.0f ? amax / 2688.0f : 1.0f;
}

/* Codes [n][k/2] (element 2i in the low nibble of byte i) and scales [n][k/16]
 * of an [n][k] matrix under tensor scale st (OpenMP over rows). */
void nvo_quantize(const void* w, int bf16, int64_t n, int64_t k, int64_t ldw, float st, uint8_t* codes,
                  uint8_t* scales) {
  const float six_st = 6.0f * st;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r)
    for (int64_t b = 0; b < k / 16; ++b) {
      float v[16];
      float amax = 0.0f;
      for (int i = 0; i < 16; ++i) {
        v[i] = input_value(w, bf16, r * ldw + 16 * b + i);
        if (fabsf(v[i]) > amax) amax = fabsf(v[i]);
      }
      const float q = amax / six_st;
      const uint32_t sb = e4m3_nearest(q);
      scales[r * (k / 16) + b] = (uint8_t)sb;
      const float d = (float)nvo_e4m3(sb) * st;
      for (int i = 0; i < 16; ++i) {
        uint32_t c = 0;
        if (sb != 0u) {
          const float rq = v[i] / d;
          c = e2m1_nearest(fabsf(rq)) | (signbit(v[i]) ? 8u : 0u);
        }
        uint8_t* byte = codes + r * (k / 2) + 8 * b + i / 2;
        if (i % 2 == 0) *byte = (uint8_t)c;
        else *byte = (uint8_t)(*byte | (c << 4));
      }
    }
}

/* ---- W4A4: both operands in the OCP MX FP4 block format ---------------------
 *
 * The pages' prefill runs native FP4 on both operands (imp README, "How does
 * it work?"); on this hardware the FP4 matrix instructions take the OCP MX
 * format: 32 consecutive k elements share one E8M0 (power-of-two) scale.
 * Readings (each listed in the design notes):
 *   - a 32-element block v with largest magnitude amax gets the scale
 *     X = 2^(floor(log2 amax) - 2) (2 is the exponent of E2M1's largest
 *     power of two, 4), the exponent clamped to [-127, 127]; an all-zero
 *     block gets the smallest scale (byte 0) and zero codes;
 *   - each element's code is the E2M1 value nearest v / X (ties to the even
 *     mantissa, +-6 beyond 6; v / X is exact, X being a power of two); the
 *     sign bit is v's;
 *   - weights: an NVFP4 matrix's values e2m1(c) * e4m3(sigma) (exact, s_t left
 *     out) are requantised this way along k; activations: the bf16 values;
 *   - y = s_t * sum_k w'[n][k] * x'[m][k] over the requantised values, in
 *     fp64 here (every product is exact).
 * The block is 32 k elements along each row; K is a multiple of 32.
 */

/* E8M0 byte and the 32 codes (low nibble first) of one block of doubles. */
static void mx_block(const double* v, uint8_t* codes16, uint8_t* scale) {
  double amax = 0.0;
  for (int i = 0; i < 32; ++i)
    if (fabs(v[i]) > amax) amax = fabs(v[i]);
  memset(codes16, 0, 16);
  if (amax == 0.0) {
    *scale = 0;
    return;
  }
  int e2 = 0;
  frexp(amax, &e2);              /* amax = f * 2^e2, f in [0.5, 1): floor(log2 amax) = e2 - 1 */
  int ex = (e2 - 1) - 2;
  if (ex < -127) ex = -127;
  if (ex > 127) ex = 127;
  *scale = (uint8_t)(ex + 127);
  for (int i = 0; i < 32; ++i) {
    const double q = ldexp(fabs(v[i]), -ex);
    uint32_t best = 0;
    double bd = q;
    for (uint32_t c = 1; c < 8u; ++c) {
      const double d = fabs(q - kE2M1Magnitude[c]);
      if (d < bd || (d == bd && (c & 1u) == 0u)) {
        best = c;
        bd = d;
      }
    }
    const uint32_t code = best | (signbit(v[i]) ? 8u : 0u);
    codes16[i / 2] |= (uint8_t)((i & 1) ? (code << 4) : code);
  }
}

static double mx_value(const uint8_t* codes16, uint8_t scale, int i) {
  const uint32_t c = (i & 1) ? (codes16[i / 2] >> 4) : (codes16[i / 2] & 15u);
  return nvo_e2m1(c) * ldexp(1.0, (int)scale - 127);
}

/* MX-requantise an [n][k] NVFP4 matrix (s_t left out): codes [n][k/2], E8M0
 * scales [n][k/32]. */
void nvo_mx_from_nvfp4(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k, uint8_t* mx_codes,
                       uint8_t* mx_scales) {
  for (int64_t r = 0; r < n; ++r)
    for (int64_t b = 0; b < k / 32; ++b) {
      double v[32];
      for (int i = 0; i < 32; ++i) v[i] = weight(codes, scales, k, 1.0, r, 32 * b + i);
      mx_block(v, mx_codes + r * (k / 2) + 16 * b, mx_scales + r * (k / 32) + b);
    }
}

/* MX-quantise bf16 activations [m][ldx] (k used): codes [m][k/2], scales [m][k/32]. */
void nvo_mx_from_bf16(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, uint8_t* mx_codes, uint8_t* mx_scales) {
  for (int64_t r = 0; r < m; ++r)
    for (int64_t b = 0; b < k / 32; ++b) {
      double v[32];
      for (int i = 0; i < 32; ++i) v[i] = nvo_bf16(x[r * ldx + 32 * b + i]);
      mx_block(v, mx_codes + r * (k / 2) + 16 * b, mx_scales + r * (k / 32) + b);
    }
}

/* y[m][j] = st * sum_k w'[rows[j]][k] x'[m][k] and s[m][j] = st * sum_k |w' x'|
 * from MX operands (both [..][k/2] codes, [..][k/32] scales). */
void nvo_mx_gemm(const uint8_t* wc, const uint8_t* ws, int64_t n, int64_t k, float st, const uint8_t* xc,
                 const uint8_t* xs, int64_t m, const int64_t* rows, int64_t nrows, double* y, double* s,
                 int nthreads) {
  if (rows == NULL) nrows = n;
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(static) num_threads(nthreads)
  for (int64_t j = 0; j < nrows; ++j) {
    const int64_t r = rows ? rows[j] : j;
    for (int64_t t = 0; t < m; ++t) {
      double acc = 0.0, mag = 0.0;
      for (int64_t b = 0; b < k / 32; ++b)
        for (int i = 0; i < 32; ++i) {
          const double p = mx_value(wc + r * (k / 2) + 16 * b, ws[r * (k / 32) + b], i) *
                           mx_value(xc + t * (k / 2) + 16 * b, xs[t * (k / 32) + b], i);
          acc += p;
          mag += fabs(p);
        }
      y[t * nrows + j] = (double)st * acc;
      if (s) s[t * nrows + j] = (double)st * mag;
    }
  }
}
