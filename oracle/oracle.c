/*
 * oracle.c -- plain CPU reference of the block-diffusion denoising pass.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h): loaded by the tests, the smoke
 * check and the CPU-baseline leg of the benchmark, never by the product.
 *
 * Per-token loops, double-precision arithmetic, one rounding wherever a
 * tensor is stored.  OpenMP only splits independent outputs (tokens, heads,
 * vocabulary rows are never reduced across threads), so results do not depend
 * on the thread count.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* storage types                                                            */
/* ------------------------------------------------------------------------ */

/* OCP FP8 E4M3 ("fn" variant: no infinities, S.1111.111 is NaN, max 448):
 * 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, subnormals at
 * exponent field 0 with value m * 2^-9. */
double or_fp8e4m3_decode(uint8_t code) {
  int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m, -9);
  else v = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* OCP FP4 E2M1: 1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit;
 * exponent field 0 is subnormal with value m * 2^-1.  No infinities or NaN. */
double or_fp4e2m1_decode(uint8_t code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double v = e == 0 ? 0.5 * m : ldexp(1.0 + m / 2.0, e - 1);
  return s ? -v : v;
}

/* OCP E8M0 block scale: 2^(e - 127); the all-ones code is NaN. */
double or_e8m0_decode(uint8_t code) {
  if (code == 0xFF) return NAN;
  return ldexp(1.0, (int)code - 127);
}

static double bf16_bits_to_double(uint16_t h) {
  uint32_t b = (uint32_t)h << 16;
  float f;
  memcpy(&f, &b, 4);
  return (double)f;
}

/* Round-to-nearest-even from double to bf16 (8 exponent bits, 7 stored
 * mantissa bits), without double rounding: first round to float with
 * round-to-odd (truncate, then set the last bit when inexact), then
 * round-to-nearest-even the float to bf16.  Round-to-odd into a format with
 * at least two more bits than the target gives the correctly rounded result. */
uint16_t or_bf16_bits(double x) {
  if (isnan(x)) return (uint16_t)(signbit(x) ? 0xFFC0 : 0x7FC0);
  float f = (float)x;
  uint32_t b;
  memcpy(&b, &f, 4);
  if ((double)f != x) {
    if (fabs((double)f) > fabs(x)) b -= 1; /* step the magnitude toward zero */
    b |= 1u;                               /* sticky bit: round-to-odd */
  }
  uint32_t lsb = (b >> 16) & 1u;
  b += 0x7FFFu + lsb;
  return (uint16_t)(b >> 16);
}

double or_round_to(int dt, double x) {
  if (dt == OR_F32) return (double)(float)x;
  if (dt == OR_BF16) return bf16_bits_to_double(or_bf16_bits(x));
  return x;
}

static double ld(const void* p, int dt, size_t i) {
  if (dt == OR_F32) return (double)((const float*)p)[i];
  if (dt == OR_BF16) return bf16_bits_to_double(((const uint16_t*)p)[i]);
  return or_fp8e4m3_decode(((const uint8_t*)p)[i]);
}

/* element i of a row-major expert matrix in storage type dt; MXFP4 codes
 * take their block's scale (rows hold a multiple of 32 elements, so the block
 * of flat element i is i / 32) */
static double ldw(const void* p, const uint8_t* mx, int dt, size_t i) {
  if (dt != OR_MXFP4) return ld(p, dt, i);
  uint8_t byte = ((const uint8_t*)p)[i >> 1];
  uint8_t code = (i & 1) ? (byte >> 4) : (byte & 15);
  return or_fp4e2m1_decode(code) * or_e8m0_decode(mx[i >> 5]);
}

static void st(void* p, int dt, size_t i, double x) {
  if (dt == OR_F32) ((float*)p)[i] = (float)x;
  else ((uint16_t*)p)[i] = or_bf16_bits(x);
}

/* ------------------------------------------------------------------------ */
/* Philox4x64-10 (Salmon et al., SC'11): each round multiplies counter words */
/* 0 and 2 by the two round constants, swaps and xors the high halves with   */
/* the other counter words and the key; the key is bumped by the two Weyl    */
/* constants between rounds.                                                */
/* ------------------------------------------------------------------------ */

#define PHX_M0 0xD2E7470EE14C6C93ULL
#define PHX_M1 0xCA5A826395121157ULL
#define PHX_W0 0x9E3779B97F4A7C15ULL
#define PHX_W1 0xBB67AE8584CAA73BULL

void or_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]) {
  uint64_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
  uint64_t k0 = key[0], k1 = key[1];
  for (int r = 0; r < 10; r++) {
    if (r > 0) {
      k0 += PHX_W0;
      k1 += PHX_W1;
    }
    unsigned __int128 p0 = (unsigned __int128)PHX_M0 * c0;
    unsigned __int128 p1 = (unsigned __int128)PHX_M1 * c2;
    uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0;
    uint64_t hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

/* ------------------------------------------------------------------------ */
/* re-noise ("Uniform State Diffusion": low-confidence tokens are replaced   */
/* by a fresh uniformly random vocabulary token)                            */
/* ------------------------------------------------------------------------ */

int or_renoise(int32_t* canvas, const int32_t* argmax, const float* conf, float tau,
               uint64_t seed, uint32_t pass_tag, const int32_t* pos0, const uint32_t* req_id,
               int B, int N, int V) {
  if (!canvas || !pos0 || B < 0 || N < 0 || V <= 0) return -1;
  if (conf && !argmax) return -1;
  for (int b = 0; b < B; b++) {
    for (int i = 0; i < N; i++) {
      size_t t = (size_t)b * N + i;
      /* keep when conf >= tau; a NaN confidence compares false and is noised */
      if (conf && conf[t] >= tau) {
        canvas[t] = argmax[t];
        continue;
      }
      uint64_t ctr[4] = {(uint64_t)(int64_t)(pos0[b] + i), (uint64_t)pass_tag,
                         (uint64_t)(req_id ? req_id[b] : (uint32_t)b), 0};
      uint64_t key[2] = {seed, 0};
      uint64_t r[4];
      or_philox4x64_10(ctr, key, r);
      /* uniform index: floor(r0 * V / 2^64) */
      canvas[t] = (int32_t)(uint64_t)(((unsigned __int128)r[0] * (uint64_t)V) >> 64);
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* masked ("absorbing") diffusion, the earlier sampler the explainer        */
/* contrasts with uniform-state noise ("First attempt: masked diffusion"):   */
/* slots start as a [MASK] token; a pass's prediction fills a masked slot,   */
/* and a filled slot is locked in for good.  Reading: a masked slot is      */
/* filled when its confidence reaches tau (the same rule that keeps a slot  */
/* under uniform-state noise); the canvas's last pass fills every slot.     */
/* ------------------------------------------------------------------------ */

int or_unmask(int32_t* canvas, const int32_t* argmax, const float* conf, float tau, int32_t mask_id,
              int final_pass, int B, int N, int32_t* changed, int32_t* masked_left) {
  if (!canvas || !argmax || !conf || B < 0 || N < 0) return -1;
  for (int b = 0; b < B; b++) {
    int nchanged = 0, nleft = 0;
    for (int i = 0; i < N; i++) {
      size_t t = (size_t)b * N + i;
      if (canvas[t] == mask_id && (final_pass || conf[t] >= tau)) {
        if (argmax[t] != canvas[t]) nchanged++;
        canvas[t] = argmax[t];
      }
      if (canvas[t] == mask_id) nleft++;
    }
    if (changed) changed[b] = nchanged;
    if (masked_left) masked_left[b] = nleft;
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* layer pieces                                                             */
/* ------------------------------------------------------------------------ */

static int nthreads_or_default(int n) { return n > 0 ? n : 1; }

/* u = x / sqrt(mean(x^2) + eps) * gain, rounded to dt */
static void rmsnorm_row(const double* x, const float* gain, int D, double eps, int dt, double* u) {
  double ss = 0.0;
  for (int d = 0; d < D; d++) ss += x[d] * x[d];
  double r = 1.0 / sqrt(ss / D + eps);
  for (int d = 0; d < D; d++) u[d] = or_round_to(dt, x[d] * r * (double)gain[d]);
}

/* y[o] = sum_d x[d] * W[o][d]  (W row-major [O][I]) in double, unrounded */
static void linear_row(const double* x, const void* W, int dt, int O, int I, double* y) {
  for (int o = 0; o < O; o++) {
    double acc = 0.0;
    size_t base = (size_t)o * I;
    for (int d = 0; d < I; d++) acc += x[d] * ld(W, dt, base + d);
    y[o] = acc;
  }
}

static double silu(double a) { return a / (1.0 + exp(-a)); }

typedef struct ctx {
  const or_config* c;
  int QKV;   /* (Hq + 2 Hkv) * hd */
  int QD;    /* Hq * hd */
  int KD;    /* Hkv * hd */
} ctx;

/* K or V element of request b, kv head g, key position j, dim d from a cache */
static double cache_at(const ctx* x, const void* cache, int cap, int b, int g, int j, int d) {
  const or_config* c = x->c;
  size_t idx = (((size_t)b * c->Hkv + g) * cap + j) * c->hd + d;
  return ld(cache, c->act_dt, idx);
}

/*
 * One transformer layer over M = B*T token rows (rows b*T .. b*T+T-1 belong
 * to request b), pre-norm:  x1 = x + Attn(N1(x)) Wo^T;  x = x1 + MoE(N2(x1)).
 *
 * mode 0 (denoise): keys of request b are cache[0, len[b]) followed by the T
 *   canvas rows of b, all visible to every canvas query (bidirectional).
 * mode 1 (prefill): the new K/V are written at [len[b], len[b]+T) first;
 *   query i then sees cache keys 0 .. len[b]+i (causal).
 * stop_after_kv: prefill of the last layer -- nothing downstream reads the
 *   attention or MoE output, so the layer ends after the cache write.
 */
static void layer_forward(const ctx* X, const or_layer* lw, int li, double* x, int B, int T,
                          void* kc_w, const void* kc, void* vc_w, const void* vc, int cap,
                          const int32_t* len, int mode, int stop_after_kv, const or_taps* tp,
                          int nth) {
  const or_config* c = X->c;
  const int D = c->D, M = B * T, G = c->Hq / c->Hkv, hd = c->hd, E = c->E, K = c->k, F = c->F;
  const int adt = c->act_dt, edt = c->exp_dt;
  const size_t BN = (size_t)M;

  double* u = (double*)malloc(sizeof(double) * (size_t)M * D);
  double* qkv = (double*)malloc(sizeof(double) * (size_t)M * X->QKV);

  /* N1 and the q/k/v projections, each rounded to the activation type */
#pragma omp parallel for schedule(dynamic, 1) num_threads(nth)
  for (int t = 0; t < M; t++) {
    rmsnorm_row(x + (size_t)t * D, lw->g1, D, c->eps, adt, u + (size_t)t * D);
    double* r = qkv + (size_t)t * X->QKV;
    linear_row(u + (size_t)t * D, lw->wq, adt, X->QD, D, r);
    linear_row(u + (size_t)t * D, lw->wk, adt, X->KD, D, r + X->QD);
    linear_row(u + (size_t)t * D, lw->wv, adt, X->KD, D, r + X->QD + X->KD);
    for (int o = 0; o < X->QKV; o++) r[o] = or_round_to(adt, r[o]);
  }
  if (tp && tp->qkv)
    for (size_t i = 0; i < (size_t)M * X->QKV; i++)
      st(tp->qkv, adt, (size_t)li * M * X->QKV + i, qkv[i]);

  if (mode == 1) {
    /* write the new keys and values into the cache ("Prefill mode ... writes
     * to the KV cache") */
    for (int b = 0; b < B; b++)
      for (int i = 0; i < T; i++)
        for (int g = 0; g < c->Hkv; g++)
          for (int d = 0; d < hd; d++) {
            const double* r = qkv + ((size_t)b * T + i) * X->QKV;
            size_t idx = (((size_t)b * c->Hkv + g) * cap + (len[b] + i)) * hd + d;
            st(kc_w, adt, idx, r[X->QD + g * hd + d]);
            st(vc_w, adt, idx, r[X->QD + X->KD + g * hd + d]);
          }
    if (stop_after_kv) {
      free(u);
      free(qkv);
      return;
    }
  }

  /* attention: softmax(q k^T / sqrt(hd)) v over the keys the block mask allows */
  double* o = (double*)malloc(sizeof(double) * (size_t)M * X->QD);
  int maxkeys = 0;
  for (int b = 0; b < B; b++)
    if (len[b] + T > maxkeys) maxkeys = len[b] + T;
  const double scale = 1.0 / sqrt((double)hd);
#pragma omp parallel num_threads(nth)
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(maxkeys > 0 ? maxkeys : 1));
#pragma omp for collapse(2) schedule(dynamic, 4)
    for (int t = 0; t < M; t++) {
      for (int h = 0; h < c->Hq; h++) {
        int b = t / T, i = t % T, g = h / G;
        const double* q = qkv + (size_t)t * X->QKV + (size_t)h * hd;
        /* number of keys and where each comes from */
        int nk = (mode == 0) ? len[b] + T : len[b] + i + 1;
        double mx = -INFINITY;
        for (int j = 0; j < nk; j++) {
          double acc = 0.0;
          if (mode == 0 && j >= len[b]) {
            const double* kr = qkv + ((size_t)b * T + (j - len[b])) * X->QKV + X->QD + g * hd;
            for (int d = 0; d < hd; d++) acc += q[d] * kr[d];
          } else {
            for (int d = 0; d < hd; d++) acc += q[d] * cache_at(X, kc, cap, b, g, j, d);
          }
          s[j] = acc * scale;
          if (s[j] > mx) mx = s[j];
        }
        double den = 0.0;
        for (int j = 0; j < nk; j++) {
          s[j] = exp(s[j] - mx);
          den += s[j];
        }
        double* out = o + (size_t)t * X->QD + (size_t)h * hd;
        for (int d = 0; d < hd; d++) {
          double acc = 0.0;
          for (int j = 0; j < nk; j++) {
            double vv;
            if (mode == 0 && j >= len[b])
              vv = qkv[((size_t)b * T + (j - len[b])) * X->QKV + X->QD + X->KD + g * hd + d];
            else
              vv = cache_at(X, vc, cap, b, g, j, d);
            acc += s[j] * vv;
          }
          out[d] = or_round_to(adt, acc / den);
        }
      }
    }
    free(s);
  }
  if (tp && tp->attn)
    for (size_t i = 0; i < (size_t)M * X->QD; i++)
      st(tp->attn, adt, (size_t)li * M * X->QD + i, o[i]);

  /* x1 = round(x + o Wo^T); u2 = N2(x1); router logits in fp32 */
  double* x1 = (double*)malloc(sizeof(double) * (size_t)M * D);
  double* u2 = (double*)malloc(sizeof(double) * (size_t)M * D);
  float* rl = (float*)malloc(sizeof(float) * (size_t)M * E);
#pragma omp parallel num_threads(nth)
  {
    double* tmp = (double*)malloc(sizeof(double) * (size_t)(D > E ? D : E));
#pragma omp for schedule(dynamic, 1)
    for (int t = 0; t < M; t++) {
      linear_row(o + (size_t)t * X->QD, lw->wo, adt, D, X->QD, tmp);
      for (int d = 0; d < D; d++)
        x1[(size_t)t * D + d] = or_round_to(adt, x[(size_t)t * D + d] + tmp[d]);
      rmsnorm_row(x1 + (size_t)t * D, lw->g2, D, c->eps, adt, u2 + (size_t)t * D);
      if (tp && tp->inject_router) {
        for (int e = 0; e < E; e++)
          rl[(size_t)t * E + e] = tp->inject_router[((size_t)li * M + t) * E + e];
      } else {
        linear_row(u2 + (size_t)t * D, lw->wr, adt, E, D, tmp);
        for (int e = 0; e < E; e++) rl[(size_t)t * E + e] = (float)tmp[e];
      }
    }
    free(tmp);
  }
  free(o);
  if (tp && tp->x1)
    for (size_t i = 0; i < (size_t)M * D; i++) st(tp->x1, adt, (size_t)li * M * D + i, x1[i]);
  if (tp && tp->u2)
    for (size_t i = 0; i < (size_t)M * D; i++) st(tp->u2, adt, (size_t)li * M * D + i, u2[i]);
  if (tp && tp->router)
    memcpy(tp->router + (size_t)li * M * E, rl, sizeof(float) * (size_t)M * E);

  /* top-k by (logit descending, expert index ascending); gates are the
   * softmax of the k selected logits */
  int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)M * K);
  double* gates = (double*)malloc(sizeof(double) * (size_t)M * K);
  for (int t = 0; t < M; t++) {
    const float* r = rl + (size_t)t * E;
    int32_t* sel = ids + (size_t)t * K;
    for (int j = 0; j < K; j++) {
      int best = -1;
      for (int e = 0; e < E; e++) {
        int taken = 0;
        for (int jj = 0; jj < j; jj++)
          if (sel[jj] == e) taken = 1;
        if (taken) continue;
        if (best < 0 || r[e] > r[best]) best = e; /* strict: the lower index wins ties */
      }
      sel[j] = best;
    }
    double den = 0.0, r0 = (double)r[sel[0]];
    for (int j = 0; j < K; j++) den += exp((double)r[sel[j]] - r0);
    for (int j = 0; j < K; j++) gates[(size_t)t * K + j] = exp((double)r[sel[j]] - r0) / den;
  }
  if (tp && tp->ids) memcpy(tp->ids + (size_t)li * M * K, ids, sizeof(int32_t) * (size_t)M * K);
  if (tp && tp->gates)
    for (size_t i = 0; i < (size_t)M * K; i++) tp->gates[(size_t)li * M * K + i] = (float)gates[i];

  /* permutation: counting sort of the (token, slot) entries by expert; within
   * an expert, entries stay in (token, slot) order */
  if (tp && (tp->counts || tp->offsets || tp->perm)) {
    int32_t* cnt = (int32_t*)calloc((size_t)E, sizeof(int32_t));
    int32_t* off = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t* fill = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * BN * K);
    for (size_t i = 0; i < BN * K; i++) cnt[ids[i]]++;
    off[0] = 0;
    for (int e = 0; e < E; e++) off[e + 1] = off[e] + cnt[e];
    memcpy(fill, off, sizeof(int32_t) * (size_t)E);
    for (size_t i = 0; i < BN * K; i++) perm[fill[ids[i]]++] = (int32_t)i;
    if (tp->counts) memcpy(tp->counts + (size_t)li * E, cnt, sizeof(int32_t) * (size_t)E);
    if (tp->offsets) memcpy(tp->offsets + (size_t)li * (E + 1), off, sizeof(int32_t) * (size_t)(E + 1));
    if (tp->perm) memcpy(tp->perm + (size_t)li * BN * K, perm, sizeof(int32_t) * BN * K);
    free(cnt);
    free(off);
    free(fill);
    free(perm);
  }

  /* experts, per token and slot: h = round(silu(u2 Wg^T) * (u2 Wu^T)),
   * y = round(h Wd^T); fp8 weights are decoded exactly and the per-expert
   * scale multiplies the accumulated sum.  x = round(x1 + sum_j g_j y_j). */
#pragma omp parallel num_threads(nth)
  {
    double* hcol = (double*)malloc(sizeof(double) * (size_t)F);
    double* y = (double*)malloc(sizeof(double) * (size_t)K * D);
#pragma omp for schedule(dynamic, 1)
    for (int t = 0; t < M; t++) {
      const double* a_in = u2 + (size_t)t * D;
      for (int j = 0; j < K; j++) {
        int e = ids[(size_t)t * K + j];
        double sg = 1.0, su = 1.0, sd = 1.0;
        if (edt == OR_FP8E4M3) {
          sg = lw->escale[e * 3 + 0];
          su = lw->escale[e * 3 + 1];
          sd = lw->escale[e * 3 + 2];
        }
        for (int f = 0; f < F; f++) {
          double a = 0.0, cc = 0.0;
          size_t base = ((size_t)e * F + f) * D;
          for (int d = 0; d < D; d++) a += a_in[d] * ldw(lw->wg, lw->wg_mx, edt, base + d);
          for (int d = 0; d < D; d++) cc += a_in[d] * ldw(lw->wu, lw->wu_mx, edt, base + d);
          a *= sg;
          cc *= su;
          hcol[f] = or_round_to(adt, silu(a) * cc);
        }
        double* yj = y + (size_t)j * D;
        for (int d = 0; d < D; d++) {
          double acc = 0.0;
          size_t base = ((size_t)e * D + d) * F;
          for (int f = 0; f < F; f++) acc += hcol[f] * ldw(lw->wd, lw->wd_mx, edt, base + f);
          yj[d] = or_round_to(adt, acc * sd);
        }
        if (tp && tp->hmid)
          for (int f = 0; f < F; f++)
            st(tp->hmid, adt, (((size_t)li * M + t) * K + j) * F + f, hcol[f]);
        if (tp && tp->yexp)
          for (int d = 0; d < D; d++)
            st(tp->yexp, adt, (((size_t)li * M + t) * K + j) * D + d, yj[d]);
      }
      for (int d = 0; d < D; d++) {
        double acc = x1[(size_t)t * D + d];
        double mix = 0.0;
        for (int j = 0; j < K; j++) mix += gates[(size_t)t * K + j] * y[(size_t)j * D + d];
        x[(size_t)t * D + d] = or_round_to(adt, acc + mix);
      }
    }
    free(hcol);
    free(y);
  }
  if (tp && tp->xout)
    for (size_t i = 0; i < (size_t)M * D; i++) st(tp->xout, adt, (size_t)li * M * D + i, x[i]);

  free(ids);
  free(gates);
  free(x1);
  free(u2);
  free(rl);
  free(u);
  free(qkv);
}

static int check_cfg(const or_config* c) {
  if (!c) return 0;
  if (c->L <= 0 || c->D <= 0 || c->Hq <= 0 || c->Hkv <= 0 || c->hd <= 0 || c->E <= 0 ||
      c->k <= 0 || c->k > c->E || c->F <= 0 || c->V <= 0)
    return 0;
  if (c->Hq % c->Hkv) return 0;
  if (c->act_dt != OR_F32 && c->act_dt != OR_BF16) return 0;
  if (c->exp_dt != OR_F32 && c->exp_dt != OR_BF16 && c->exp_dt != OR_FP8E4M3 && c->exp_dt != OR_MXFP4)
    return 0;
  if (c->exp_dt == OR_MXFP4 && (c->D % 32 || c->F % 32)) return 0;
  return 1;
}

static double* embed(const or_config* c, const or_weights* w, const int32_t* tok, int M) {
  double* x = (double*)malloc(sizeof(double) * (size_t)M * c->D);
  for (int t = 0; t < M; t++)
    for (int d = 0; d < c->D; d++)
      x[(size_t)t * c->D + d] = ld(w->emb, c->act_dt, (size_t)tok[t] * c->D + d);
  return x;
}

int or_kv_prefill(const or_config* cfg, const or_weights* w, void* const* kc, void* const* vc,
                  int cap, int32_t* len, const int32_t* tokens, int B, int T,
                  const or_taps* taps, int nthreads) {
  if (!check_cfg(cfg) || !w || !kc || !vc || !len || !tokens || B <= 0 || T <= 0) return -1;
  for (int b = 0; b < B; b++)
    if (len[b] < 0 || len[b] + T > cap) return -2;
  for (int t = 0; t < B * T; t++)
    if (tokens[t] < 0 || tokens[t] >= cfg->V) return -1;
  ctx X = {cfg, (cfg->Hq + 2 * cfg->Hkv) * cfg->hd, cfg->Hq * cfg->hd, cfg->Hkv * cfg->hd};
  int nth = nthreads_or_default(nthreads);
  double* x = embed(cfg, w, tokens, B * T);
  for (int l = 0; l < cfg->L; l++)
    layer_forward(&X, &w->layers[l], l, x, B, T, kc[l], kc[l], vc[l], vc[l], cap, len, 1,
                  l == cfg->L - 1, taps, nth);
  free(x);
  for (int b = 0; b < B; b++) len[b] += T;
  return 0;
}

int or_denoise_pass(const or_config* cfg, const or_weights* w, const void* const* kc,
                    const void* const* vc, int cap, const int32_t* len, const int32_t* canvas,
                    int B, int N, int32_t* argmax, float* conf, const or_taps* taps, int nthreads) {
  if (!check_cfg(cfg) || !w || !canvas || !argmax || !conf || B <= 0 || N <= 0) return -1;
  if (!len) return -1;
  for (int b = 0; b < B; b++)
    if (len[b] < 0 || len[b] > cap || (len[b] > 0 && (!kc || !vc))) return -1;
  for (int t = 0; t < B * N; t++)
    if (canvas[t] < 0 || canvas[t] >= cfg->V) return -1;
  ctx X = {cfg, (cfg->Hq + 2 * cfg->Hkv) * cfg->hd, cfg->Hq * cfg->hd, cfg->Hkv * cfg->hd};
  const int D = cfg->D, V = cfg->V, M = B * N;
  int nth = nthreads_or_default(nthreads);
  double* x = embed(cfg, w, canvas, M);
  for (int l = 0; l < cfg->L; l++)
    layer_forward(&X, &w->layers[l], l, x, B, N, NULL, kc ? kc[l] : NULL, NULL,
                  vc ? vc[l] : NULL, cap, len, 0, 0, taps, nth);

  /* head: final norm, exact logits, argmax on the fp32 logits (lowest index
   * among equal maxima), confidence = softmax probability of the maximum */
#pragma omp parallel num_threads(nth)
  {
    double* uf = (double*)malloc(sizeof(double) * (size_t)D);
    double* lg = (double*)malloc(sizeof(double) * (size_t)V);
#pragma omp for schedule(dynamic, 1)
    for (int t = 0; t < M; t++) {
      rmsnorm_row(x + (size_t)t * D, w->gf, D, cfg->eps, cfg->act_dt, uf);
      if (taps && taps->uf)
        for (int d = 0; d < D; d++) st(taps->uf, cfg->act_dt, (size_t)t * D + d, uf[d]);
      linear_row(uf, w->lm, cfg->act_dt, V, D, lg);
      int am = 0;
      float best = (float)lg[0];
      double mx = lg[0];
      for (int v = 1; v < V; v++) {
        if ((float)lg[v] > best) {
          best = (float)lg[v];
          am = v;
        }
        if (lg[v] > mx) mx = lg[v];
      }
      double den = 0.0;
      for (int v = 0; v < V; v++) den += exp(lg[v] - mx);
      argmax[t] = am;
      conf[t] = (float)(1.0 / den);
      if (taps && taps->logits)
        for (int v = 0; v < V; v++) taps->logits[(size_t)t * V + v] = (float)lg[v];
    }
    free(uf);
    free(lg);
  }
  free(x);
  return 0;
}
