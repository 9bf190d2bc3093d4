/*
 * sanitize_main.c -- drives every entry point of the CPU oracle on tiny
 * shapes, for a build with AddressSanitizer and UndefinedBehaviorSanitizer
 * (oracle/build.py, build_sanitized).  TEST INFRASTRUCTURE ONLY.
 *
 * Covers: fp32 and bf16 activations with fp32, bf16, fp8 e4m3 and MXFP4
 * expert weights; a causal prefill of two requests with ragged lengths, a
 * second (chained) prefill, a denoising pass with every tap and with
 * injected router logits, the uniform re-noise and the masked update, the
 * counter-based generator and the format conversions.  The inputs are
 * arbitrary bit patterns from a fixed linear congruential sequence (only
 * memory safety and defined behaviour are checked here; values are checked
 * by the Python tests).  Exit status 0 when every call returned 0.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static uint64_t lcg = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {
  lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(lcg >> 32);
}
/* uniform in [-0.05, 0.05) */
static float next_small(void) { return ((float)(next_u32() >> 8) / 16777216.0f - 0.5f) * 0.1f; }

static void* alloc(size_t n) {
  void* p = calloc(n ? n : 1, 1);
  if (!p) {
    fprintf(stderr, "out of memory\n");
    exit(2);
  }
  return p;
}

/* a tensor of n elements in storage type dt */
static void* tensor(int dt, size_t n) {
  if (dt == OR_F32) {
    float* p = alloc(n * 4);
    for (size_t i = 0; i < n; i++) p[i] = next_small();
    return p;
  }
  if (dt == OR_BF16) {
    uint16_t* p = alloc(n * 2);
    for (size_t i = 0; i < n; i++) p[i] = or_bf16_bits(next_small());
    return p;
  }
  if (dt == OR_FP8E4M3) {
    uint8_t* p = alloc(n);
    for (size_t i = 0; i < n; i++) {
      uint8_t c = (uint8_t)next_u32();
      if ((c & 0x7F) == 0x7F) c ^= 1; /* no NaN codes */
      p[i] = c;
    }
    return p;
  }
  /* MXFP4: two codes per byte */
  uint8_t* p = alloc((n + 1) / 2);
  for (size_t i = 0; i < (n + 1) / 2; i++) p[i] = (uint8_t)next_u32();
  return p;
}

static float* gains(int n) {
  float* g = alloc((size_t)n * 4);
  for (int i = 0; i < n; i++) g[i] = 1.0f + next_small();
  return g;
}

static uint8_t* mx_scales(size_t n) {
  uint8_t* s = alloc(n);
  for (size_t i = 0; i < n; i++) s[i] = (uint8_t)(120 + next_u32() % 10);
  return s;
}

static int fails = 0;
static void check(int rc, const char* what) {
  if (rc != 0) {
    fprintf(stderr, "%s returned %d\n", what, rc);
    fails++;
  }
}

static void run(int act, int ex, int nthreads) {
  or_config c = {2, 64, 4, 2, 16, 4, 2, 32, 64, 1e-6, act, ex};
  const int qkv = (c.Hq + 2 * c.Hkv) * c.hd;
  or_layer layers[2];
  memset(layers, 0, sizeof layers);
  for (int l = 0; l < c.L; l++) {
    or_layer* y = &layers[l];
    y->g1 = gains(c.D);
    y->wq = tensor(act, (size_t)c.Hq * c.hd * c.D);
    y->wk = tensor(act, (size_t)c.Hkv * c.hd * c.D);
    y->wv = tensor(act, (size_t)c.Hkv * c.hd * c.D);
    y->wo = tensor(act, (size_t)c.D * c.Hq * c.hd);
    y->g2 = gains(c.D);
    y->wr = tensor(act, (size_t)c.E * c.D);
    y->wg = tensor(ex, (size_t)c.E * c.F * c.D);
    y->wu = tensor(ex, (size_t)c.E * c.F * c.D);
    y->wd = tensor(ex, (size_t)c.E * c.D * c.F);
    if (ex == OR_FP8E4M3) {
      float* s = alloc((size_t)c.E * 3 * 4);
      for (int i = 0; i < c.E * 3; i++) s[i] = 0.01f + fabsf(next_small());
      y->escale = s;
    }
    if (ex == OR_MXFP4) {
      y->wg_mx = mx_scales((size_t)c.E * c.F * (c.D / 32));
      y->wu_mx = mx_scales((size_t)c.E * c.F * (c.D / 32));
      y->wd_mx = mx_scales((size_t)c.E * c.D * (c.F / 32));
    }
  }
  or_weights w = {tensor(act, (size_t)c.V * c.D), layers, gains(c.D), tensor(act, (size_t)c.V * c.D)};

  const int B = 2, cap = 16, es = act == OR_F32 ? 4 : 2;
  void* kc[2];
  void* vc[2];
  for (int l = 0; l < c.L; l++) {
    kc[l] = alloc((size_t)B * c.Hkv * cap * c.hd * es);
    vc[l] = alloc((size_t)B * c.Hkv * cap * c.hd * es);
  }
  int32_t len[2] = {0, 3};
  int32_t tok[2 * 5];
  for (int i = 0; i < B * 5; i++) tok[i] = (int32_t)(next_u32() % (uint32_t)c.V);

  /* prefill with every per-layer tap, then a chained one without taps */
  const int R = B * 5;
  or_taps pt;
  memset(&pt, 0, sizeof pt);
  pt.qkv = alloc((size_t)c.L * R * qkv * es);
  pt.attn = alloc((size_t)c.L * R * c.Hq * c.hd * es);
  pt.x1 = alloc((size_t)c.L * R * c.D * es);
  pt.u2 = alloc((size_t)c.L * R * c.D * es);
  pt.router = alloc((size_t)c.L * R * c.E * 4);
  pt.ids = alloc((size_t)c.L * R * c.k * 4);
  pt.gates = alloc((size_t)c.L * R * c.k * 4);
  pt.counts = alloc((size_t)c.L * c.E * 4);
  pt.offsets = alloc((size_t)c.L * (c.E + 1) * 4);
  pt.perm = alloc((size_t)c.L * R * c.k * 4);
  pt.hmid = alloc((size_t)c.L * R * c.k * c.F * es);
  pt.yexp = alloc((size_t)c.L * R * c.k * c.D * es);
  pt.xout = alloc((size_t)c.L * R * c.D * es);
  check(or_kv_prefill(&c, &w, kc, vc, cap, len, tok, B, 5, &pt, nthreads), "prefill");
  check(or_kv_prefill(&c, &w, kc, vc, cap, len, tok, B, 2, NULL, nthreads), "chained prefill");
  /* a prefill past the capacity must fail without writing */
  int32_t full[2] = {cap - 1, 0};
  if (or_kv_prefill(&c, &w, kc, vc, cap, full, tok, B, 2, NULL, nthreads) != -2) fails++;

  /* a pass over 3-slot canvases with every tap, then with injected routing */
  const int N = 3, BN = B * N;
  int32_t canvas[6], am[6];
  float cf[6];
  for (int i = 0; i < BN; i++) canvas[i] = (int32_t)(next_u32() % (uint32_t)c.V);
  or_taps t;
  memset(&t, 0, sizeof t);
  t.qkv = alloc((size_t)c.L * BN * qkv * es);
  t.attn = alloc((size_t)c.L * BN * c.Hq * c.hd * es);
  t.x1 = alloc((size_t)c.L * BN * c.D * es);
  t.u2 = alloc((size_t)c.L * BN * c.D * es);
  t.router = alloc((size_t)c.L * BN * c.E * 4);
  t.ids = alloc((size_t)c.L * BN * c.k * 4);
  t.gates = alloc((size_t)c.L * BN * c.k * 4);
  t.counts = alloc((size_t)c.L * c.E * 4);
  t.offsets = alloc((size_t)c.L * (c.E + 1) * 4);
  t.perm = alloc((size_t)c.L * BN * c.k * 4);
  t.hmid = alloc((size_t)c.L * BN * c.k * c.F * es);
  t.yexp = alloc((size_t)c.L * BN * c.k * c.D * es);
  t.xout = alloc((size_t)c.L * BN * c.D * es);
  t.uf = alloc((size_t)BN * c.D * es);
  t.logits = alloc((size_t)BN * c.V * 4);
  check(or_denoise_pass(&c, &w, (const void* const*)kc, (const void* const*)vc, cap, len, canvas, B, N,
                        am, cf, &t, nthreads),
        "pass");
  float* inj = alloc((size_t)c.L * BN * c.E * 4);
  for (int i = 0; i < c.L * BN * c.E; i++) inj[i] = (float)(next_u32() % 4); /* ties */
  t.inject_router = inj;
  check(or_denoise_pass(&c, &w, (const void* const*)kc, (const void* const*)vc, cap, len, canvas, B, N,
                        am, cf, &t, nthreads),
        "pass with injected routing");

  /* between-pass updates */
  int32_t pos0[2] = {len[0], len[1]};
  uint32_t req[2] = {7, 9};
  check(or_renoise(canvas, NULL, NULL, 0.5f, 1234567ull, 0, pos0, NULL, B, N, c.V), "initial noise");
  cf[1] = NAN;
  check(or_renoise(canvas, am, cf, 0.5f, 1234567ull, 3, pos0, req, B, N, c.V), "re-noise");
  int32_t changed[2], left[2];
  for (int i = 0; i < BN; i++) canvas[i] = c.V - 1;
  check(or_unmask(canvas, am, cf, 0.5f, c.V - 1, 0, B, N, changed, left), "unmask");
  check(or_unmask(canvas, am, cf, 0.5f, c.V - 1, 1, B, N, NULL, NULL), "unmask, last pass");

  /* free everything (ASan reports leaks at exit) */
  free(inj);
  void* tp[] = {t.qkv, t.attn, t.x1, t.u2, t.router, t.ids, t.gates, t.counts, t.offsets, t.perm,
                t.hmid, t.yexp, t.xout, t.uf, t.logits, pt.qkv, pt.attn, pt.x1, pt.u2, pt.router,
                pt.ids, pt.gates, pt.counts, pt.offsets, pt.perm, pt.hmid, pt.yexp, pt.xout};
  for (size_t i = 0; i < sizeof tp / sizeof tp[0]; i++) free(tp[i]);
  for (int l = 0; l < c.L; l++) {
    or_layer* y = &layers[l];
    free((void*)y->g1);
    free((void*)y->wq);
    free((void*)y->wk);
    free((void*)y->wv);
    free((void*)y->wo);
    free((void*)y->g2);
    free((void*)y->wr);
    free((void*)y->wg);
    free((void*)y->wu);
    free((void*)y->wd);
    free((void*)y->escale);
    free((void*)y->wg_mx);
    free((void*)y->wu_mx);
    free((void*)y->wd_mx);
    free(kc[l]);
    free(vc[l]);
  }
  free((void*)w.emb);
  free((void*)w.gf);
  free((void*)w.lm);
}

int main(void) {
#ifdef SANITIZER_SELFCHECK
  {
    /* a heap read one element past the end: an instrumented build stops here */
    int* volatile p = alloc(4 * sizeof(int));
    const int x = p[4];
    free(p);
    return x == 12345 ? 0 : 3;
  }
#endif
  const int combos[][2] = {{OR_F32, OR_F32}, {OR_BF16, OR_BF16}, {OR_BF16, OR_FP8E4M3}, {OR_BF16, OR_MXFP4}};
  for (int i = 0; i < 4; i++)
    for (int nt = 1; nt <= 2; nt++) run(combos[i][0], combos[i][1], nt);
  uint64_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, out[4];
  or_philox4x64_10(ctr, key, out);
  double acc = 0;
  for (int code = 0; code < 256; code++) {
    const double a = or_fp8e4m3_decode((uint8_t)code), b = or_fp4e2m1_decode((uint8_t)code);
    const double s = or_e8m0_decode((uint8_t)code);
    acc += (isnan(a) ? 0 : a) + b + (isnan(s) ? 0 : s * 0);
  }
  acc += or_round_to(OR_BF16, 1.0 / 3.0) + or_round_to(OR_FP8E4M3, 1e9) + (double)out[0] * 0;
  if (fails) {
    fprintf(stderr, "%d oracle calls failed\n", fails);
    return 1;
  }
  printf("oracle sanitized run ok (%g)\n", acc);
  return 0;
}
