/*
 * dgpass.h -- C ABI of libdgpass: one block-diffusion denoising pass over a
 * canvas of vocabulary tokens, on an MI355X (gfx950).
 *
 * The method (pages cited by title and section):
 *  - explainer "DiffusionGemma", "Two modes, one model": a causal prefill
 *    writes the KV cache; a denoising pass attends bidirectionally over the
 *    canvas and the cache.  "Uniform State Diffusion": noise is random
 *    vocabulary tokens, every position is updated in parallel each pass and
 *    low-confidence positions are replaced by fresh random tokens.  "Long-form
 *    text: chaining canvases": each finished canvas is appended to the cache
 *    by a prefill step and a fresh canvas is opened.
 *  - course page "Module 12. Diffusion Language Models", block-mask exercise:
 *    prefix rows causal, block rows see prefix and block; prefix K/V are
 *    reused across denoising steps, block states are recomputed every pass.
 *  - newsletter comment under "A Visual Guide to DiffusionGemma": every canvas
 *    token goes through the MoE router, so a pass reads the union of the
 *    selected experts; the comment asks for the expert coverage per step.
 *
 * Layer (pre-norm; plain readings where the pages are silent: no positional
 * terms, attention scale 1/sqrt(hd), RMSNorm with gain, no shared expert):
 *   u  = rmsnorm(x) * g1;  q,k,v = u Wq^T, u Wk^T, u Wv^T
 *   o  = softmax(q k^T / sqrt(hd)) v  over the keys the block mask allows
 *   x1 = x + o Wo^T;  u2 = rmsnorm(x1) * g2;  r = u2 Wr^T (fp32)
 *   top-k experts by (r descending, index ascending); gates = softmax of the
 *   k selected logits;  x = x1 + sum_j g_j * (silu(u2 Wg_e^T) * (u2 Wu_e^T)) Wd_e^T
 * Head: uf = rmsnorm(x) * gf;  logits = uf W_lm^T (fp32); argmax = lowest
 * index of the maximum; conf = softmax probability of the maximum.
 * Stored tensors are rounded (RNE) to the activation type: u, q, k, v (hence
 * the cache), o, x1, u2, SwiGLU output, expert outputs, x, uf.  Router and
 * head logits stay fp32.
 *
 * Conventions of every call:
 *  - Device pointers are HIP device memory owned by the caller.  Host pointers
 *    are marked "host".  The library allocates nothing and keeps no global
 *    state; every call enqueues on `stream` (a hipStream_t, NULL = the null
 *    stream) and returns without synchronising.
 *  - Activations, caches and the embedding table are row-major [rows][cols].
 *    The weight matrices a GEMM streams (wq, wk, wv, wo, wr, wg, wu, wd, lm;
 *    logically [out][in]) are passed in the packed layout below, written by
 *    dg_pack_weight from the row-major matrix.
 *  - Arguments are validated before the first launch; a call that returns an
 *    error has enqueued nothing and changed nothing.  Device faults surface at
 *    the caller's next synchronisation.  No C++ exception crosses the ABI.
 *  - Two calls that share a workspace must be ordered (same stream).
 */
#ifndef DGPASS_H
#define DGPASS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t dg_status;
#define DG_OK 0
#define DG_ERR_INVALID (-1)      /* null pointer, bad shape or value */
#define DG_ERR_CAPACITY (-2)     /* len[b] + T exceeds the cache capacity */
#define DG_ERR_UNSUPPORTED (-3)  /* shape or dtype outside what the kernels implement */
#define DG_ERR_WORKSPACE (-4)    /* workspace too small */
#define DG_ERR_HIP (-5)          /* a launch failed (hipGetLastError) */

/* storage types */
#define DG_F32 0
#define DG_BF16 1
#define DG_FP8E4M3 2   /* OCP e4m3 (max 448, no infinities), expert weights only */
#define DG_MXFP4 3     /* OCP microscaling FP4, expert weights only: 4-bit E2M1 codes, two
                          per byte (element 2i in the low nibble), and one E8M0 scale byte
                          (2^(s-127)) per 32 consecutive elements of a row */

#define DG_MAX_LAYERS 64
#define DG_MAX_BATCH 64

/* Model shape.  Supported: act_dtype F32 with expert_dtype F32, or act_dtype
 * BF16 with expert_dtype BF16, FP8E4M3 or MXFP4; hd in {64, 128}; Hq/Hkv in
 * {1, 2, 4, 8, 16}; D a multiple of 128; F and Hq*hd multiples of 64 (F of
 * 128 with FP8E4M3 experts; D and F of 256 with MXFP4 experts); 1 <= k <= 8;
 * k <= E <= 256. */
typedef struct dg_config {
  int32_t L, D, Hq, Hkv, hd, E, k, F, V;
  float eps;               /* RMSNorm epsilon */
  int32_t act_dtype;       /* embeddings, attention/router/head weights, activations, KV cache */
  int32_t expert_dtype;    /* expert weights */
} dg_config;

/* Packed weight layout.  A logical row-major matrix [rows][cols] whose rows
 * hold rb = cols * (element bytes) bytes, rb a multiple of 128, is stored as
 * tiles of 16 rows x 128 bytes: tile (rg, kb) -- row group rg = 0 ..
 * ceil(rows/16)-1, column block kb = 0 .. rb/128-1 -- occupies the 2048 bytes
 * at offset (rg * rb/128 + kb) * 2048.  Inside a tile, the 16 bytes at offset
 * 1024 h + 16 l (h in {0, 1}, l in 0..63) hold row 16 rg + l % 16, bytes
 * 128 kb + 64 h + 16 (l / 16) .. +15 of that row; rows past the matrix are
 * zero.  One 64-lane load of 16 bytes per lane then reads 1 KB of contiguous
 * memory and leaves every lane with its matrix-core operand fragment.  An
 * expert tensor [E][F][D] is packed as one [E*F][D] matrix (F is a multiple
 * of 16, so no tile straddles two experts).  MXFP4 codes are packed the same
 * way (rb = cols / 2).  Their E8M0 scales ([rows][cols/32] bytes) are packed
 * to match: the 128 bytes at offset (rg * cols/256 + kb) * 128 belong to code
 * tile (rg, kb), and byte 64 h + l holds the scale of row 16 rg + l % 16,
 * block 8 kb + 4 h + l / 16 -- the block of the 32 codes that lane l of load
 * h of that tile reads. */

/* Device pointers of one layer. */
typedef struct dg_layer_weights {
  const float* g1;     /* [D] f32 */
  const void* wq;      /* [Hq*hd][D] act, packed */
  const void* wk;      /* [Hkv*hd][D] act, packed */
  const void* wv;      /* [Hkv*hd][D] act, packed */
  const void* wo;      /* [D][Hq*hd] act, packed */
  const float* g2;     /* [D] f32 */
  const void* wr;      /* [E][D] act, packed (rows padded to 16) */
  const void* wg;      /* [E][F][D] expert dtype, packed as [E*F][D] */
  const void* wu;      /* [E][F][D] expert dtype, packed as [E*F][D] */
  const void* wd;      /* [E][D][F] expert dtype, packed as [E*D][F] */
  const float* escale; /* [E][3] f32 (gate, up, down) multipliers of the
                          accumulated fp8 products; NULL unless FP8E4M3 */
  const uint8_t* wg_mx; /* MXFP4: E8M0 scales of wg, wu, wd, packed (above); */
  const uint8_t* wu_mx; /* NULL unless MXFP4 */
  const uint8_t* wd_mx;
} dg_layer_weights;

typedef struct dg_weights {
  const void* emb;     /* [V][D] act, row-major (rows are gathered by token) */
  const float* gf;     /* [D] f32 final norm gain */
  const void* lm;      /* [V][D] act, packed (rows padded to 16) */
  dg_layer_weights layers[DG_MAX_LAYERS];
} dg_weights;

/* Immutable description of a model; a host struct the caller owns. */
typedef struct dg_model {
  dg_config cfg;
  dg_weights w;
  uint32_t magic;
} dg_model;

/* KV cache: per layer K and V, device [B][Hkv][cap][hd] act.  len is a host
 * array [B] of valid prefix lengths; kv_prefill advances it. */
typedef struct dg_kv {
  void* k[DG_MAX_LAYERS];
  void* v[DG_MAX_LAYERS];
  int32_t cap;
  int32_t* len;
} dg_kv;

/* Stages a pass or prefill can bracket with HIP events (dg_taps.stage_events). */
#define DG_STAGE_ATTN 0     /* attention (and the merge of its key splits) */
#define DG_STAGE_GATEUP 1   /* grouped gate/up expert GEMM + SwiGLU */
#define DG_STAGE_DOWN 2     /* grouped down expert GEMM */
#define DG_STAGE_HEAD 3     /* LM head + argmax/confidence partials (pass only; layer L-1's slots) */
#define DG_NSTAGES 4

/* Optional device outputs (debug taps), injected inputs and stage events of a
 * pass or prefill; every field may be NULL.  BN = B*N (or B*T for a prefill).
 * Token-major, slots in top-k order.  Writing taps adds work; leave them NULL
 * when timing.
 *
 * Injected inputs replace a value the call would compute by one given by the
 * caller, so that a stage can be checked on inputs identical to another
 * implementation's (the taps still record what this call computed):
 *  - inject_x: layer l starts from inject_x[l] instead of the previous
 *    layer's output (layer 0: instead of the embedding rows); its first
 *    RMSNorm is taken of the injected rows;
 *  - inject_router: routing of layer l uses inject_router[l] instead of the
 *    router logits (the router GEMM is skipped);
 *  - inject_uf: the LM head reads inject_uf instead of the final RMSNorm
 *    output (pass or decoding step). */
typedef struct dg_taps {
  void* qkv;                 /* [L][BN][(Hq+2Hkv)*hd] act */
  void* attn;                /* [L][BN][Hq*hd] act: attention output before Wo */
  void* x1;                  /* [L][BN][D] act */
  void* u2;                  /* [L][BN][D] act */
  float* router;             /* [L][BN][E] f32 (the logits routing used) */
  int32_t* ids;              /* [L][BN][k] */
  float* gates;              /* [L][BN][k] */
  int32_t* counts;           /* [L][E] */
  int32_t* offsets;          /* [L][E+1] */
  int32_t* perm;             /* [L][BN*k]: entries t*k+j sorted by (expert, t, j) */
  void* hmid;                /* [L][BN][k][F] act: SwiGLU output per slot */
  void* yexp;                /* [L][BN][k][D] act: expert output per slot */
  void* xout;                /* [L][BN][D] act: layer output (computed, not injected) */
  void* uf;                  /* [BN][D] act: final RMSNorm output (pass or decoding step; computed) */
  float* logits;             /* [BN][V] f32 (pass or decoding step) */
  const float* inject_router;/* input [L][BN][E] f32 */
  const void* inject_x;      /* input [L][BN][D] act */
  const void* inject_uf;     /* input [BN][D] act (pass or decoding step) */
  void* const* stage_events; /* host array [L][DG_NSTAGES][2] of hipEvent_t: entry
                                [l][s][0] is recorded on `stream` just before the
                                launches of stage s of layer l, [l][s][1] just
                                after them (timing of one stage); NULL entries and
                                stages a call does not run are skipped */
} dg_taps;

/* Fill *m after validating cfg and the weight pointers.  No device work. */
dg_status dg_model_init(dg_model* m, const dg_config* cfg, const dg_weights* w);

/* Bytes of workspace a call needs for up to max_rows token rows (B*N of a
 * pass or B*T of a prefill) and up to max_keys keys per request (prefix +
 * rows of that request; 0 = not known: room for the most key splits).
 * max_keys sizes the partial results of the attention's key splits; a call
 * whose requests hold more keys still runs, with fewer splits.  0 when cfg
 * is invalid.  Host arithmetic only. */
size_t dg_workspace_bytes(const dg_config* cfg, int32_t max_rows, int32_t max_keys);

/* Causal prefill ("Prefill mode"): appends T tokens per request (device
 * tokens [B][T] int32 in [0, V)) to every layer's cache at positions
 * [len[b], len[b]+T) and, on success, advances kv->len[b] by T (host).  Query
 * i sees keys 0 .. len[b]+i.  The last layer stops after its cache write.
 * Token ids are not checked on the host (they live in device memory): an id
 * outside [0, V) is clamped into that range by the embedding kernel, with no
 * error reported; the same holds for the canvas of a pass.
 * Errors: INVALID, CAPACITY (len[b]+T > cap), UNSUPPORTED, WORKSPACE, HIP. */
dg_status dg_kv_prefill(const dg_model* m, dg_kv* kv, const int32_t* tokens, int32_t B, int32_t T,
                        const dg_taps* taps, void* ws, size_t ws_bytes, void* stream);

/* One autoregressive decoding step, the baseline a canvas pass is weighed
 * against (course page "Module 12. Diffusion Language Models", break-even
 * solution: autoregressive decoding emits one token per pass over the
 * weights).  Appends one token per request (device tokens [B] int32) at
 * position len[b] as dg_kv_prefill with T = 1 does, runs every layer in full
 * on that row (query len[b] sees keys 0 .. len[b]) and the LM head, and writes
 * the next token (lowest index of the maximum logit) and its softmax
 * probability to device argmax [B] int32 and conf [B] f32.  Advances
 * kv->len[b] by 1 on success.  Taps as for a prefill; inject_uf, uf and
 * logits apply to the head.  Errors: those of dg_kv_prefill, INVALID for a
 * null argmax or conf. */
dg_status dg_decode_step(const dg_model* m, dg_kv* kv, const int32_t* tokens, int32_t B,
                         int32_t* argmax, float* conf, const dg_taps* taps, void* ws, size_t ws_bytes,
                         void* stream);

/* One denoising pass ("Denoising mode") over device canvases [B][N] int32.
 * Request b's canvas queries see its whole cached prefix kv->len[b] and its
 * whole canvas (bidirectional).  The cache is only read.  Outputs device
 * argmax [B][N] int32 and conf [B][N] f32.  The per-layer expert counts of
 * this pass stay in the workspace for dg_expert_coverage until the workspace
 * is used again. */
dg_status dg_denoise_pass(const dg_model* m, const dg_kv* kv, const int32_t* canvas, int32_t B,
                          int32_t N, int32_t* argmax, float* conf, const dg_taps* taps, void* ws,
                          size_t ws_bytes, void* stream);

/* Uniform-state re-noise of device canvases [B][N] in place.  conf == NULL
 * noises every slot (canvas initialisation; argmax may be NULL).  Otherwise
 * slot i of request b keeps argmax[b][i] when conf[b][i] >= tau and else takes
 * a uniform token floor(r * V / 2^64), r = word 0 of Philox4x64-10 with
 * counter (pos0[b] + i, pass_tag, req_id[b], 0) and key (seed, 0) (Salmon et
 * al., "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11).  A NaN conf is
 * noised.  pos0: host [B] absolute position of slot 0; req_id: host [B] or
 * NULL for b.  B <= DG_MAX_BATCH. */
dg_status dg_renoise(int32_t* canvas, const int32_t* argmax, const float* conf, float tau,
                     uint64_t seed, uint32_t pass_tag, const int32_t* pos0,
                     const uint32_t* req_id, int32_t B, int32_t N, int32_t V, void* stream);

/* Samplers of the between-pass update. */
#define DG_SAMPLER_UNIFORM 0  /* uniform-state noise (explainer "DiffusionGemma", "Uniform
                                 State Diffusion"): slots below tau take a fresh random token */
#define DG_SAMPLER_MASKED 1   /* masked ("absorbing") diffusion (same page, "First attempt:
                                 masked diffusion"): a [MASK] slot takes the prediction once its
                                 confidence reaches tau and is then locked in */

/* Parameters of the update between two passes of a canvas.  tau, seed,
 * pass_tag, pos0 (host [B]) and req_id (host [B] or NULL for b) are the
 * arguments of dg_renoise.  mode: DG_SAMPLER_UNIFORM (what dg_renoise does)
 * or DG_SAMPLER_MASKED: a slot holding mask_id takes the pass's argmax when its
 * conf >= tau, or in any case when final_pass is set (the canvas's last
 * pass); any other slot keeps its token.  changed and masked_left: device [B]
 * int32 or NULL, receive per request the number of slots whose token changed
 * and (masked mode) the number still holding mask_id afterwards -- the canvas
 * has converged when nothing changed (uniform) or nothing is masked (masked;
 * explainer, "Uniform State Diffusion": after several passes the canvas
 * converges).
 * Two flags let consecutive passes of one canvas skip the canvas embedding
 * (both are read by dg_denoise_pass_next only; 0 = off):
 *  - embed_next: the pass's last kernel also writes the first layer's input
 *    of the updated canvas (its embedding rows and their RMSNorm) into the
 *    workspace;
 *  - input_embedded: this pass does not embed `canvas`; it reads the first
 *    layer's input from the workspace.  Set it only when the previous call on
 *    this workspace (and stream) was a dg_denoise_pass_next with embed_next
 *    for this canvas, B and N, and the canvas has not changed since: the
 *    library cannot check this, and any other use gives the pass the wrong
 *    input.  For dg_denoise_pass_next_noalloc the workspace is the GPU's
 *    scratch, so the previous call is the previous one on that GPU. */
typedef struct dg_renoise_args {
  float tau;
  uint64_t seed;
  uint32_t pass_tag;
  const int32_t* pos0;
  const uint32_t* req_id;
  int32_t mode;
  int32_t mask_id;
  int32_t final_pass;
  int32_t* changed;
  int32_t* masked_left;
  int32_t embed_next;
  int32_t input_embedded;
} dg_renoise_args;

/* The between-pass update of device canvases [B][N] in place as its own call:
 * from this pass's device argmax [B][N] and conf [B][N] under a->mode, with
 * the counts of a->changed / a->masked_left.  conf == NULL initialises a
 * canvas: uniform noise (pass tag a->pass_tag, as dg_renoise with conf NULL)
 * or mask_id in every slot.  Errors: INVALID (null canvas or a, null pos0 in
 * uniform mode, a negative pos0[b], conf without argmax, a bad mode, B
 * outside [1, DG_MAX_BATCH], N or V < 1), HIP. */
dg_status dg_canvas_update(int32_t* canvas, const int32_t* argmax, const float* conf,
                           const dg_renoise_args* a, int32_t B, int32_t N, int32_t V, void* stream);

/* A denoising pass (arguments and results as dg_denoise_pass) whose last
 * kernel also does the work that follows a pass inside a canvas ("Uniform
 * State Diffusion": every pass but the last re-noises the low-confidence
 * slots; newsletter comment: the expert coverage per step), so a canvas of S
 * passes launches no separate kernels for it:
 *  - touched: device [L] int32, or NULL; receives what dg_expert_coverage
 *    would write after this pass (the counts stay in the workspace as well);
 *  - next: or NULL; the canvas (device [B][N], read by this pass) is then
 *    updated in place from this pass's argmax and conf, with the same tokens
 *    and counts dg_canvas_update(canvas, argmax, conf, next, B, N, V) gives
 *    after the pass (uniform mode: those of dg_renoise).
 * With both NULL this is dg_denoise_pass.  Errors: those of dg_denoise_pass;
 * INVALID also for a bad next->mode, a null next->pos0 in uniform mode, a
 * negative next->pos0[b], or a canvas that aliases argmax or conf. */
dg_status dg_denoise_pass_next(const dg_model* m, const dg_kv* kv, int32_t* canvas, int32_t B,
                               int32_t N, int32_t* argmax, float* conf, int32_t* touched,
                               const dg_renoise_args* next, const dg_taps* taps, void* ws,
                               size_t ws_bytes, void* stream);

/* Bytes of the device scratch of dg_denoise_pass_next_noalloc (one per GPU). */
#define DG_NOALLOC_SCRATCH_BYTES (64 << 20)

/* dg_denoise_pass_next without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Arguments, results and errors are those
 * of dg_denoise_pass_next; the call allocates nothing.  Its workspace is a
 * static device array of DG_NOALLOC_SCRATCH_BYTES that the library holds on
 * each GPU it runs on until the process ends (looked up once per device on the
 * first call there).  Limit: the pass's fixed workspace (every buffer but the
 * attention split partials, which take the room that is left and so bound the
 * number of key splits) must fit the scratch, about 256 canvas rows of a
 * model with 2048-wide layers and a 32768-token vocabulary; larger calls
 * return DG_ERR_WORKSPACE before any device work.  Every call on one GPU
 * shares that GPU's scratch: calls that overlap on one GPU (different streams
 * or host threads without ordering) race; calls on one stream are ordered.
 * The expert counts of the pass stay in the scratch only until the next call
 * on that GPU, so read the coverage through `touched`. */
dg_status dg_denoise_pass_next_noalloc(const dg_model* m, const dg_kv* kv, int32_t* canvas, int32_t B,
                                       int32_t N, int32_t* argmax, float* conf, int32_t* touched,
                                       const dg_renoise_args* next, const dg_taps* taps, void* stream);

/* Experts touched per layer by the last pass run with this workspace: device
 * touched [L] int32 = #{e : count[l][e] > 0} (the union over the batch), and
 * optionally device counts [L][E] int32. */
dg_status dg_expert_coverage(const dg_model* m, const void* ws, size_t ws_bytes, int32_t* touched,
                             int32_t* counts, void* stream);

/* Bytes of a packed weight matrix: ceil(rows/16)*16 * cols * element bytes;
 * 0 when rows or cols < 1, dtype is not a storage type or the row bytes are
 * not a multiple of 128.  Host arithmetic only. */
size_t dg_packed_bytes(int32_t rows, int32_t cols, int32_t dtype);

/* Write the packed layout of the row-major device matrix src [rows][cols]
 * (dtype) to device dst (dg_packed_bytes(rows, cols, dtype) bytes, not
 * overlapping src).  Enqueued on stream; a one-time step when a model is
 * loaded.  Errors: INVALID (null or equal pointers, a shape dg_packed_bytes
 * rejects), UNSUPPORTED, HIP. */
dg_status dg_pack_weight(const void* src, void* dst, int32_t rows, int32_t cols, int32_t dtype,
                         void* stream);

/* Bytes of the packed MXFP4 scales of a [rows][cols] matrix (cols a multiple
 * of 256): ceil(rows/16)*16 * cols/32; 0 otherwise.  Host arithmetic only. */
size_t dg_packed_mx_scale_bytes(int32_t rows, int32_t cols);

/* Write the packed layout of the row-major device E8M0 scales src
 * [rows][cols/32] of an MXFP4 matrix [rows][cols] to device dst
 * (dg_packed_mx_scale_bytes bytes, not overlapping src); rows past the matrix
 * get scale 1 (code 127).  Errors: INVALID, HIP. */
dg_status dg_pack_mx_scales(const void* src, void* dst, int32_t rows, int32_t cols, void* stream);

const char* dg_status_str(dg_status s);

#ifdef __cplusplus
}
#endif
#endif
