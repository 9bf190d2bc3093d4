// launch.h -- host-side launchers of the libdgpass kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dgpass.h"

namespace dg {

// activation storage selector
enum Act { ACT_F32 = 0, ACT_BF16 = 1 };

struct Lens {
  int32_t v[DG_MAX_BATCH];
};
struct ReqIds {
  uint32_t v[DG_MAX_BATCH];
};

// ---- elementwise / reductions (kern_elem.hip) ----
void launch_embed_norm(int act, const int32_t* tok, const void* emb, const float* g, int rows, int D,
                       int V, float eps, void* x, void* u, hipStream_t s);
void launch_rmsnorm(int act, const void* x, const float* g, int rows, int D, float eps, void* u,
                    hipStream_t s);
void launch_combine_norm(int act, const void* x1, const void* Y, const float* gates,
                         const int32_t* inv, int rows, int k, int D, const float* gnext, float eps,
                         void* x, void* u, hipStream_t s, int32_t* zero0 = nullptr,
                         int32_t* zero1 = nullptr, int nzero = 0);   // zero0/1: [nzero <= 256]
                                                                    // ints cleared by block 0
void launch_renoise(int32_t* canvas, const int32_t* argmax, const float* conf, float tau,
                    uint64_t seed, uint32_t tag, const Lens& pos0, const ReqIds& req, int B, int N,
                    int V, hipStream_t s);
void launch_coverage(const int32_t* counts, int L, int E, int32_t* touched, int32_t* counts_out,
                     hipStream_t s);
void launch_unpermute(int act, const void* src, const int32_t* inv, int slots, int C, void* dst,
                      hipStream_t s);
// work a pass's last kernel can take over from the calls that follow it:
// rn.canvas != nullptr re-noises the canvas for the next pass (argmax and
// conf are this merge's outputs), touched != nullptr writes the expert
// coverage from counts [L][E]
struct RenoiseArgs {
  int32_t* canvas;
  const int32_t* argmax;
  const float* conf;
  float tau;
  uint64_t seed;
  uint32_t tag;
  int B, N;
  uint32_t V;
  Lens pos0;
  ReqIds req;
  int mode;              // DG_SAMPLER_UNIFORM or DG_SAMPLER_MASKED
  int32_t mask_id;       // masked sampler: the [MASK] token
  int final_pass;        // masked sampler: fill every masked slot
  int32_t* changed;      // optional [B]: slots whose token changed
  int32_t* masked_left;  // optional [B]: slots holding mask_id afterwards
};
// the between-pass update of either sampler as its own launch (one block per
// request, so the counts need no atomics); a.conf == nullptr initialises
void launch_canvas_update(const RenoiseArgs& a, hipStream_t s);
struct MergeNext {
  RenoiseArgs rn;
  const int32_t* counts;
  int L, E;
  int32_t* touched;
  // with ex set (and rn.canvas): each row block also writes the first layer's
  // input of its updated slot, x = emb[token] and u = its RMSNorm with g1
  int act;
  const void* emb;
  const float* g1;
  int D;
  float eps;
  void* ex;
  void* eu;
};
void launch_lm_merge(const float* pmax, const int32_t* pidx, const float* psum, int rows,
                     int ntiles, int32_t* argmax, float* conf, const MergeNext& nx, hipStream_t s);

// ---- MoE routing (kern_moe.hip) ----
// logits: nsplit (<= ROUTER_MAX_SPLIT) partial [rows][E] arrays (consecutive);
// with nsplit > 1 the summed logits are written back over the first one
constexpr int ROUTER_MAX_SPLIT = 16;
void launch_topk(float* logits, int nsplit, int rows, int E, int k, int32_t* ids, float* gates,
                 hipStream_t s);
// top-k that also takes the RMSNorm in front of the router: it writes
// u2 = round(x1 * rsqrt(mean(x1^2) + eps) * g2) for its row and, with
// scale set, multiplies the summed logits by the same rsqrt (the router GEMM
// then ran on round(x1 * g2)); with scale clear the logits are used as given
struct TopkNorm {
  const void* x1;
  const float* g2;
  int D;
  float eps;
  void* u2;
  int scale;
};
void launch_topk_norm(int act, float* logits, int nsplit, int rows, int E, int k, int32_t* ids,
                      float* gates, const TopkNorm& tn, hipStream_t s);
// fused RMSNorm + router logits + top-k (false if D does not fit the LDS tile)
struct RouteArgs {
  const void* x1;
  const float* g2;
  const void* wr;
  int rows, D, E, k;
  float eps;
  const float* inject;  // optional [rows][E] logits to route on
  void* u2;             // out [rows][D]
  float* logits;        // optional out [rows][E]
  int32_t* ids;
  float* gates;
};
bool launch_route(int act, const RouteArgs& a, hipStream_t s);
// counts/offsets/perm/inv + row tiles of at most tile_rows rows per expert
void launch_plan(const int32_t* ids, int rows, int k, int E, int tile_rows, int32_t* counts,
                 int32_t* offsets, int32_t* perm, int32_t* inv, int4* tiles, int32_t* ntiles,
                 hipStream_t s);

struct MoeW {
  const void* wg;
  const void* wu;
  const void* wd;
  const float* escale;  // [E][3] or null
  int wdt;              // DG_F32 / DG_BF16 / DG_FP8E4M3
};

// ---- LDS-tiled MFMA GEMMs (kern_gemm.hip) ----
enum GemmMode { GEMM_STORE = 0, GEMM_RESID = 1, GEMM_F32 = 2, GEMM_QKV_CACHE = 3 };
struct CacheDst {
  void* k;
  void* v;
  int cap, T, QD, KD, hd, Hkv;
  Lens len;
};
// C[M][N] = A[M][K] . B^T where B rows n come from up to three stacked matrices
// (rows [0,n1) from B0, [n1,n1+n2) from B1, the rest from B2).
void launch_gemm(int act, int mode, const void* A, int M, int K, const void* B0, int n1,
                 const void* B1, int n2, const void* B2, int N, void* C, int ldc, const void* R,
                 const CacheDst* cache, hipStream_t s);
// rows of an expert tile of the LDS-tiled grouped GEMMs (the tile plan's tile
// height when they run)
int group_tile_rows(int act);
void launch_gateup_lds(int act, const void* u2, const int32_t* perm, int k, const MoeW& w,
                       const int4* tiles, const int32_t* ntiles, int max_tiles, int D, int F,
                       void* H, hipStream_t s);
void launch_down_lds(int act, const void* H, const MoeW& w, const int4* tiles,
                     const int32_t* ntiles, int max_tiles, int D, int F, void* Y, hipStream_t s);
// LM head: per-row partial (max, argmax, sum exp) over vocabulary tiles of 128
// row-major [rows][rowbytes] -> packed weight layout (rowbytes % 128 == 0,
// rows padded to a multiple of 16 with zeros)
void launch_pack(const void* src, void* dst, int rows, int rowbytes, hipStream_t s);
// MXFP4 scales [rows][nblk] (nblk a multiple of 8) -> the packed scale layout
void launch_pack_mx_scales(const void* src, void* dst, int rows, int nblk, hipStream_t s);

// returns the number of per-row partials written (one per vocabulary tile)
int launch_lmhead(int act, const void* uf, int M, int D, const void* lm, int V, float* pmax,
                  int32_t* pidx, float* psum, float* logits, hipStream_t s);

// ---- weight-streaming MFMA GEMM for few rows (kern_stream.hip) ----
enum StreamMode { SG_STORE = 0, SG_RESID = 1, SG_F32 = 2, SG_QKV_CACHE = 3, SG_GATEUP = 4,
                  SG_DOWN = 5 };
struct StreamGemm {
  const void* A;          // activations [rows][K] (gate/up: gathered through perm)
  int M, K;
  const int32_t* perm;    // gate/up: slot -> token*k + j
  int k;
  const void* W0;         // packed weights: dense rows [0,n1) / gate / down
  const void* W1;         // dense rows [n1,n1+n2) / up
  const void* W2;         // dense rows [n1+n2,N)
  int n1, n2, N;          // dense / head output columns
  int NW;                 // grouped: rows per expert of W0
  const float* escale;    // grouped fp8: [E][3]
  const uint8_t* S0;      // grouped MXFP4: packed scales of W0 (gate / down)
  const uint8_t* S1;      //   and of W1 (up)
  const int4* tiles;      // grouped: (expert, first row, rows)
  const int32_t* ntiles;
  int nchunks;            // 64-weight-row chunks per row tile (gate/up: F/32)
  int ksplit;             // SG_F32: contraction splits (0 or 1 = none); split s writes
                          // its partial sums to out + s * M * ldo
  const float* gs;        // SG_F32: optional [K] scale of the activations (each element
                          // multiplied, then rounded to the activation type, before the MFMAs)
  void* out;
  int ldo;
  const void* R;          // residual (SG_RESID)
  CacheDst cache;         // SG_QKV_CACHE
};
int stream_tile_rows(int act, int wdt);
void launch_stream_gemm(int act, int wdt, int mode, int kw, const StreamGemm& a, int ntiles_max,
                        hipStream_t s);

// ---- attention (kern_attn.hip) ----
struct AttnArgsHost {
  int act;
  const void* q;   // qkv buffer (q at column h*hd), row stride ldq
  int ldq;
  const void* kc;  // cache of this layer [B][Hkv][cap][hd]
  const void* vc;
  int cap;
  const void* kn;  // canvas k/v (mode 0): rows of the qkv buffer
  const void* vn;
  int B, T, Hq, Hkv, hd;
  int mode;        // 0 = canvas (bidirectional over cache + canvas), 1 = causal over cache
  Lens len;
  void* out;       // [B*T][Hq*hd]
  void* po;        // split partials O (activation type: bf16 or fp32)
  float* pml;
  long part_cap;   // capacity of the partial buffers in (row, head) entries
};
void launch_attention(const AttnArgsHost& a, hipStream_t s);
long attn_partial_entries(int rows, int Hq, int max_keys);

}  // namespace dg
