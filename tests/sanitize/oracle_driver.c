/* Exercises every function of the CPU oracle on small inputs in buffers of
 * exactly the documented sizes, so that an AddressSanitizer /
 * UndefinedBehaviorSanitizer build reports any out-of-bounds access or
 * undefined operation.  Exit status 0 and a final "ok" line on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double nvo_e2m1(uint32_t code);
double nvo_e4m3(uint32_t byte);
double nvo_bf16(uint16_t h);
double nvo_silu(double z);
void nvo_dequant(const uint8_t*, const uint8_t*, int64_t, int64_t, float, double*);
void nvo_gemm(const uint8_t*, const uint8_t*, int64_t, int64_t, float, const uint16_t*, int64_t, int64_t,
              const int64_t*, int64_t, double*, double*, int);
void nvo_route(const float*, int64_t, int64_t, int64_t, int32_t*, double*);
void nvo_group(const int32_t*, int64_t, int64_t, int64_t, int32_t*, int32_t*, int32_t*, int32_t*);
void nvo_moe(const uint8_t*, const uint8_t*, const float*, const uint8_t*, const uint8_t*, const float*,
             const uint8_t*, const uint8_t*, const float*, const uint16_t*, const float*, int64_t, int64_t, int64_t,
             int64_t, int64_t, int32_t*, double*, double*, double*, int);
float nvo_tensor_scale(const void*, int, int64_t, int64_t, int64_t);
void nvo_quantize(const void*, int, int64_t, int64_t, int64_t, float, uint8_t*, uint8_t*);
void nvo_mx_from_nvfp4(const uint8_t*, const uint8_t*, int64_t, int64_t, uint8_t*, uint8_t*);
void nvo_mx_from_bf16(const uint16_t*, int64_t, int64_t, int64_t, uint8_t*, uint8_t*);
void nvo_mx_gemm(const uint8_t*, const uint8_t*, int64_t, int64_t, float, const uint8_t*, const uint8_t*, int64_t,
                 const int64_t*, int64_t, double*, double*, int);

static uint32_t rng = 12345u;
static uint32_t next(void) { rng = rng * 1664525u + 1013904223u; return rng >> 8; }
static void* fill(size_t n) {
  uint8_t* p = (uint8_t*)malloc(n ? n : 1);
  for (size_t i = 0; i < n; ++i) p[i] = (uint8_t)next();
  return p;
}
/* bf16 values N-ish in (-4, 4), never NaN / infinity */
static uint16_t* bf16s(size_t n) {
  uint16_t* p = (uint16_t*)malloc(2 * (n ? n : 1));
  for (size_t i = 0; i < n; ++i) {
    float f = ((float)(next() % 2001) - 1000.0f) / 250.0f;
    uint32_t u;
    memcpy(&u, &f, 4);
    p[i] = (uint16_t)(u >> 16);
  }
  return p;
}
/* E4M3 scale bytes without NaN (0x00..0x7E) */
static uint8_t* scales(size_t n) {
  uint8_t* p = (uint8_t*)malloc(n ? n : 1);
  for (size_t i = 0; i < n; ++i) p[i] = (uint8_t)(next() % 0x7F);
  return p;
}

int main(void) {
  double acc = 0.0;
  for (uint32_t c = 0; c < 16; ++c) acc += nvo_e2m1(c);
  for (uint32_t b = 0; b < 256; ++b) if (!isnan(nvo_e4m3(b))) acc += nvo_e4m3(b);
  acc += nvo_bf16(0x3F80) + nvo_silu(-3.0) + nvo_silu(0.0);

  const int64_t n = 5, k = 48, m = 3;
  uint8_t* codes = fill(n * k / 2);
  uint8_t* sc = scales(n * k / 16);
  uint16_t* x = bf16s(m * k);
  double* w = (double*)malloc(sizeof(double) * n * k);
  nvo_dequant(codes, sc, n, k, 0.5f, w);
  double* y = (double*)malloc(sizeof(double) * m * n);
  double* s = (double*)malloc(sizeof(double) * m * n);
  nvo_gemm(codes, sc, n, k, 0.5f, x, m, k, NULL, 0, y, s, 2);
  int64_t rows[2] = {4, 0};
  double* y2 = (double*)malloc(sizeof(double) * m * 2);
  nvo_gemm(codes, sc, n, k, 0.5f, x, m, k, rows, 2, y2, NULL, 1);

  const int64_t t = 4, e = 6, tk = 2, hidden = 32, inter = 16;
  float* logits = (float*)malloc(sizeof(float) * t * e);
  for (int64_t i = 0; i < t * e; ++i) logits[i] = (float)(next() % 100) / 10.0f;
  int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * t * tk);
  double* g = (double*)malloc(sizeof(double) * t * tk);
  nvo_route(logits, t, e, tk, ids, g);
  int32_t *cnt = (int32_t*)malloc(4 * e), *off = (int32_t*)malloc(4 * (e + 1));
  int32_t *perm = (int32_t*)malloc(4 * t * tk), *pos = (int32_t*)malloc(4 * t * tk);
  nvo_group(ids, t, tk, e, cnt, off, perm, pos);
  uint8_t *gc = fill(e * inter * hidden / 2), *uc = fill(e * inter * hidden / 2), *dc = fill(e * hidden * inter / 2);
  uint8_t *gs = scales(e * inter * hidden / 16), *us = scales(e * inter * hidden / 16), *ds = scales(e * hidden * inter / 16);
  float st[6] = {0.5f, 0.25f, 1.0f, 0.125f, 2.0f, 1.0f};
  uint16_t* xm = bf16s(t * hidden);
  double *ym = (double*)malloc(sizeof(double) * t * hidden), *yb = (double*)malloc(sizeof(double) * t * hidden);
  nvo_moe(gc, gs, st, uc, us, st, dc, ds, st, xm, logits, t, e, tk, hidden, inter, ids, g, ym, yb, 2);

  float* wf = (float*)malloc(sizeof(float) * n * k);
  for (int64_t i = 0; i < n * k; ++i) wf[i] = ((float)(next() % 4001) - 2000.0f) / 300.0f;
  uint8_t *qc = (uint8_t*)malloc(n * k / 2), *qs = (uint8_t*)malloc(n * k / 16);
  const float ts = nvo_tensor_scale(wf, 0, n, k, k);
  nvo_quantize(wf, 0, n, k, k, ts, qc, qs);
  const float tsb = nvo_tensor_scale(x, 1, m, k, k);
  uint8_t *qcb = (uint8_t*)malloc(m * k / 2), *qsb = (uint8_t*)malloc(m * k / 16);
  nvo_quantize(x, 1, m, k, k, tsb, qcb, qsb);

  const int64_t kk = 64;
  uint8_t* c2 = fill(n * kk / 2);
  uint8_t* s2 = scales(n * kk / 16);
  uint16_t* x2 = bf16s(m * kk);
  uint8_t *wc = (uint8_t*)malloc(n * kk / 2), *wsc = (uint8_t*)malloc(n * kk / 32);
  uint8_t *xc = (uint8_t*)malloc(m * kk / 2), *xsc = (uint8_t*)malloc(m * kk / 32);
  nvo_mx_from_nvfp4(c2, s2, n, kk, wc, wsc);
  nvo_mx_from_bf16(x2, m, kk, kk, xc, xsc);
  double *y3 = (double*)malloc(sizeof(double) * m * n), *s3 = (double*)malloc(sizeof(double) * m * n);
  nvo_mx_gemm(wc, wsc, n, kk, 0.25f, xc, xsc, m, NULL, 0, y3, s3, 2);
  nvo_mx_gemm(wc, wsc, n, kk, 0.25f, xc, xsc, m, rows, 2, y2, NULL, 1);

  for (int64_t i = 0; i < m * n; ++i) acc += y[i] + s[i] + y3[i] + s3[i];
  for (int64_t i = 0; i < t * hidden; ++i) acc += ym[i] + yb[i];
  printf("checksum %.6g\nok\n", acc);
  free(codes); free(sc); free(x); free(w); free(y); free(s); free(y2); free(logits); free(ids); free(g);
  free(cnt); free(off); free(perm); free(pos); free(gc); free(uc); free(dc); free(gs); free(us); free(ds);
  free(xm); free(ym); free(yb); free(wf); free(qc); free(qs); free(qcb); free(qsb); free(c2); free(s2); free(x2);
  free(wc); free(wsc); free(xc); free(xsc); free(y3); free(s3);
  return 0;
}
