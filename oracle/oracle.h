/*
 * oracle.h -- plain CPU reference of the block-diffusion denoising pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or
 * calls this library: only the test-suite, the smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no source, header, table or
 * helper with the GPU library.
 *
 * What it follows (pages cited by title and section):
 *  - "DiffusionGemma" explainer, "Two modes, one model": prefill is causal and
 *    writes the KV cache; denoising attends bidirectionally over the canvas
 *    and the cache.  "Long-form text: chaining canvases": a finished canvas is
 *    appended to the cache by a prefill step.  "Uniform State Diffusion":
 *    low-confidence positions are replaced by fresh random vocabulary tokens.
 *  - "Module 12. Diffusion Language Models", exercise solution on the block
 *    mask: prefix rows are causal, block rows see prefix and block.
 *  - newsletter comment under "A Visual Guide to DiffusionGemma": every canvas
 *    position goes through the MoE router, so a pass reads the union of the
 *    selected experts.
 *  - Philox4x64-10: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
 *    Easy as 1, 2, 3" (SC'11), section on the Philox construction.
 *
 * Arithmetic: every product and sum in double precision, in the order the
 * definition states (plain loops, no blocking).  Values are rounded to the
 * storage type exactly where a tensor is stored (the rounding points are
 * listed at each function).  Router logits and LM-head logits are never
 * rounded to the activation type; decisions taken on floats (top-k, argmax)
 * are taken on the fp32 rounding of the exact value, the precision the GPU
 * computes them in.
 *
 * Parity pins: see tests/test_oracle_*.py.  Full-size values of the pass on
 * random weights are not printed by any page: those are "parity unpinned"
 * beyond the invariants and special cases that the tests check.
 */
#ifndef DG_ORACLE_H
#define DG_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* storage types */
enum { OR_F32 = 0, OR_BF16 = 1, OR_FP8E4M3 = 2, OR_MXFP4 = 3 };

typedef struct or_config {
  int L, D, Hq, Hkv, hd, E, k, F, V;
  double eps;       /* RMSNorm epsilon */
  int act_dt;       /* OR_F32 or OR_BF16: embeddings, attention/router/head weights, activations, KV cache */
  int exp_dt;       /* OR_F32, OR_BF16, OR_FP8E4M3 or OR_MXFP4: expert weights */
} or_config;

typedef struct or_layer {
  const float* g1;      /* [D] RMSNorm gain before attention */
  const void* wq;       /* [Hq*hd, D]  act_dt */
  const void* wk;       /* [Hkv*hd, D] act_dt */
  const void* wv;       /* [Hkv*hd, D] act_dt */
  const void* wo;       /* [D, Hq*hd]  act_dt */
  const float* g2;      /* [D] RMSNorm gain before the MoE */
  const void* wr;       /* [E, D] act_dt router */
  const void* wg;       /* [E, F, D] exp_dt gate */
  const void* wu;       /* [E, F, D] exp_dt up */
  const void* wd;       /* [E, D, F] exp_dt down */
  const float* escale;  /* [E, 3] (gate, up, down) dequant scales, fp8 only; NULL otherwise */
  /* MXFP4 (OCP microscaling FP4): wg, wu, wd hold 4-bit E2M1 codes, two per
   * byte (element 2i in the low nibble), of the row-major matrices above; the
   * scales are one E8M0 byte per 32 consecutive elements of a row, [E, rows,
   * cols/32]; NULL otherwise */
  const uint8_t* wg_mx;
  const uint8_t* wu_mx;
  const uint8_t* wd_mx;
} or_layer;

typedef struct or_weights {
  const void* emb;          /* [V, D] act_dt */
  const or_layer* layers;   /* [L] */
  const float* gf;          /* [D] final RMSNorm gain */
  const void* lm;           /* [V, D] act_dt */
} or_weights;

/* Optional host outputs of a denoising pass; every field may be NULL.
 * Shapes use BN = B*N.  Layout is token-major, slots in top-k order. */
typedef struct or_taps {
  void* qkv;            /* [L][BN][(Hq+2Hkv)*hd] act_dt */
  void* attn;           /* [L][BN][Hq*hd] act_dt  attention output before Wo */
  void* x1;             /* [L][BN][D] act_dt  residual after attention */
  void* u2;             /* [L][BN][D] act_dt  normed input of router/experts */
  float* router;        /* [L][BN][E] fp32 router logits */
  int32_t* ids;         /* [L][BN][k] selected experts */
  float* gates;         /* [L][BN][k] */
  int32_t* counts;      /* [L][E] */
  int32_t* offsets;     /* [L][E+1] */
  int32_t* perm;        /* [L][BN*k] entries t*k+j sorted by (expert, t, j) */
  void* hmid;           /* [L][BN][k][F] act_dt  SwiGLU output per slot */
  void* yexp;           /* [L][BN][k][D] act_dt  expert output per slot */
  void* xout;           /* [L][BN][D] act_dt  layer output */
  void* uf;             /* [BN][D] act_dt  final normed state */
  float* logits;        /* [BN][V] fp32 rounding of the exact logits */
  const float* inject_router;  /* input: [L][BN][E] if set, routing uses these logits */
} or_taps;

/* Causal prefill (append).  Writes K/V of T new tokens per request at
 * positions [len[b], len[b]+T) of every layer's cache and advances len[b].
 * kc[l], vc[l]: [B][Hkv][cap][hd] act_dt.  taps (nullable) take the same
 * per-layer tensors as a pass with BN = B*T rows; the last layer stops after
 * its cache write, so only its qkv tap is written.  Returns 0, or -1 bad
 * argument, -2 capacity exceeded (nothing written). */
int or_kv_prefill(const or_config* cfg, const or_weights* w, void* const* kc, void* const* vc,
                  int cap, int32_t* len, const int32_t* tokens, int B, int T,
                  const or_taps* taps, int nthreads);

/* One denoising pass over canvases [B][N]; the cache is read only.
 * Outputs argmax [B][N] and conf [B][N] (softmax probability of the argmax). */
int or_denoise_pass(const or_config* cfg, const or_weights* w, const void* const* kc,
                    const void* const* vc, int cap, const int32_t* len, const int32_t* canvas,
                    int B, int N, int32_t* argmax, float* conf, const or_taps* taps, int nthreads);

/* Uniform-state re-noise of canvases [B][N] in place.  conf == NULL noises
 * every slot (canvas initialisation).  Slot i of request b keeps argmax when
 * conf >= tau, otherwise takes the Philox token for counter
 * (pos0[b]+i, pass_tag, req_id[b] or b, 0) and key (seed, 0). */
int or_renoise(int32_t* canvas, const int32_t* argmax, const float* conf, float tau,
               uint64_t seed, uint32_t pass_tag, const int32_t* pos0, const uint32_t* req_id,
               int B, int N, int V);

/* Masked ("absorbing") diffusion update of canvases [B][N] in place: a slot
 * holding mask_id takes argmax when conf >= tau (every masked slot when
 * final_pass is set); any other slot is left as it is (filled slots are
 * locked in).  changed[b] (may be NULL) receives the number of slots of
 * request b whose token changed, masked_left[b] (may be NULL) the number
 * still holding mask_id. */
int or_unmask(int32_t* canvas, const int32_t* argmax, const float* conf, float tau, int32_t mask_id,
              int final_pass, int B, int N, int32_t* changed, int32_t* masked_left);

/* Philox4x64 with 10 rounds, exposed for the known-answer tests. */
void or_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]);

/* Conversions, exposed for the exhaustive tests. */
double or_round_to(int dt, double x);          /* RNE to the storage type, returned as double */
double or_fp8e4m3_decode(uint8_t code);
double or_fp4e2m1_decode(uint8_t code);        /* low 4 bits */
double or_e8m0_decode(uint8_t code);
uint16_t or_bf16_bits(double x);               /* RNE bf16 bit pattern of x */

#ifdef __cplusplus
}
#endif
#endif
