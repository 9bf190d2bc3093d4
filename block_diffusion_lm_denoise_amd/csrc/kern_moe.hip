// kern_moe.hip -- MoE routing (top-k, permutation) and the weight-streaming
// grouped expert GEMMs used when few rows route to each expert.
//
// Every canvas token goes through the router and selects k experts; a pass
// therefore reads the union of the selected experts (newsletter comment under
// "A Visual Guide to DiffusionGemma"; course page "Module 12. Diffusion
// Language Models", dense-8B exercise: different positions select different
// experts).
#include <math.h>

#include "common.h"
#include "launch.h"

namespace dg {

// ---------------------------------------------------------------------------
// top-k: one wave per token.  Experts are ranked by (logit descending, index
// ascending); gates are the softmax of the k selected logits.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool better(float v, int i, float w, int j) {
  return v > w || (v == w && i < j);
}

__global__ __launch_bounds__(256) void topk_k(const float* __restrict__ logits, int rows, int E, int k,
                                              int32_t* __restrict__ ids, float* __restrict__ gates) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  float v[4];
  bool taken[4];
#pragma unroll
  for (int c = 0; c < 4; c++) {
    const int e = lane + 64 * c;
    const float x = e < E ? logits[(size_t)row * E + e] : -INFINITY;
    v[c] = x != x ? -INFINITY : x;  // a NaN logit ranks last (ids stay in range)
    taken[c] = e >= E;
  }
  float sel_v[8];
  int sel_i[8];
  for (int j = 0; j < k; j++) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int c = 0; c < 4; c++)
      if (!taken[c] && better(v[c], lane + 64 * c, bv, bi)) {
        bv = v[c];
        bi = lane + 64 * c;
      }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    sel_v[j] = bv;
    sel_i[j] = bi;
#pragma unroll
    for (int c = 0; c < 4; c++)
      if (lane + 64 * c == bi) taken[c] = true;
  }
  if (lane == 0) {
    float den = 0.f;
    for (int j = 0; j < k; j++) den += expf(sel_v[j] - sel_v[0]);
    for (int j = 0; j < k; j++) {
      ids[(size_t)row * k + j] = sel_i[j];
      gates[(size_t)row * k + j] = expf(sel_v[j] - sel_v[0]) / den;
    }
  }
}

// ---------------------------------------------------------------------------
// plan: one block per expert.  Every block builds the expert histogram of all
// (token, slot) entries in LDS and scans it; block e then lists its entries in
// (token, slot) order -- ids of a token are distinct, so at most one slot per
// token -- and writes perm / inv and its row tiles.  Block 0 publishes counts,
// offsets and the tile count.  Integer work only: the result is exact.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void plan_k(const int32_t* __restrict__ ids, int rows, int k, int E,
                                              int tile_rows, int32_t* __restrict__ counts,
                                              int32_t* __restrict__ offsets,
                                              int32_t* __restrict__ perm, int32_t* __restrict__ inv,
                                              int4* __restrict__ tiles, int32_t* __restrict__ ntiles) {
  __shared__ int hist[256];
  __shared__ int off[257];
  __shared__ int tst[257];
  __shared__ int wsum[4];
  const int tid = threadIdx.x, e = blockIdx.x;
  hist[tid] = 0;
  __syncthreads();
  const int n = rows * k;
  for (int i = tid; i < n; i += 256) atomicAdd(&hist[ids[i]], 1);
  __syncthreads();
  // inclusive scans of counts and of tile counts (Hillis-Steele over 256 slots)
  int c = tid < E ? hist[tid] : 0;
  int t = (c + tile_rows - 1) / tile_rows;
  off[tid + 1] = c;
  tst[tid + 1] = t;
  if (tid == 0) {
    off[0] = 0;
    tst[0] = 0;
  }
  __syncthreads();
  for (int s = 1; s < 256; s <<= 1) {
    int a = tid + 1 - s >= 1 ? off[tid + 1 - s] : 0;
    int b = tid + 1 - s >= 1 ? tst[tid + 1 - s] : 0;
    __syncthreads();
    off[tid + 1] += a;
    tst[tid + 1] += b;
    __syncthreads();
  }
  if (e == 0) {
    if (tid < E) counts[tid] = hist[tid];
    if (tid <= E) offsets[tid] = off[tid];
    if (tid == 0) *ntiles = tst[E];
  }
  // stable listing of expert e's entries
  const int lane = tid & 63, w = tid >> 6;
  int base = off[e];
  for (int r0 = 0; r0 < rows; r0 += 256) {
    const int r = r0 + tid;
    int js = -1;
    if (r < rows)
      for (int j = 0; j < k; j++)
        if (ids[(size_t)r * k + j] == e) js = j;
    const uint64_t m = __ballot(js >= 0);
    const int pre = __popcll(m & ((1ull << lane) - 1ull));
    __syncthreads();
    if (lane == 0) wsum[w] = __popcll(m);
    __syncthreads();
    int wpre = 0;
    for (int q = 0; q < w; q++) wpre += wsum[q];
    if (js >= 0) {
      const int pos = base + wpre + pre;
      perm[pos] = r * k + js;
      inv[(size_t)r * k + js] = pos;
    }
    base += wsum[0] + wsum[1] + wsum[2] + wsum[3];
  }
  const int ce = hist[e], nt = (ce + tile_rows - 1) / tile_rows;
  for (int i = tid; i < nt; i += 256)
    tiles[tst[e] + i] = make_int4(e, off[e] + i * tile_rows, min(tile_rows, ce - i * tile_rows), 0);
}

// ---------------------------------------------------------------------------
// Weight-streaming grouped GEMM.  One block = one row tile (<= 32 rows routed
// to one expert) x 64 weight rows.  The four waves split the contraction in
// 64-element chunks (wave w takes chunks w, w+4, ...), load A and B fragments
// straight from memory (no LDS for the weights: each weight byte is used by
// one block only), and reduce their partial tiles through LDS at the end.
//   gate/up: weight rows = [gate f0..f0+15, up f0.., gate f0+16.., up f0+16..]
//            for 32 SwiGLU outputs; A rows gathered through perm.
//   down:    64 output columns; A rows are the permuted SwiGLU rows.
// ---------------------------------------------------------------------------
template <typename TA, typename TW>
__device__ __forceinline__ void load_wfrag(typename FragOf<TA>::type& f, const TW* p);
template <>
__device__ __forceinline__ void load_wfrag<uint16_t, uint16_t>(FragBF& f, const uint16_t* p) {
  load_frag(f, p);
}
template <>
__device__ __forceinline__ void load_wfrag<uint16_t, uint8_t>(FragBF& f, const uint8_t* p) {
  load_frag_fp8(f, p);
}
template <>
__device__ __forceinline__ void load_wfrag<float, float>(FragF32& f, const float* p) {
  load_frag(f, p);
}

struct StreamArgs {
  const void* A;          // gate/up: u2 [tokens][D]; down: H [slots][F]
  const int32_t* perm;    // gate/up only
  int k;
  const void* W1;         // gate/up: wg; down: wd
  const void* W2;         // gate/up: wu
  const float* escale;
  const int4* tiles;
  const int32_t* ntiles;
  int K;                  // contraction length (D or F)
  int NW;                 // rows per expert of W1 (F for gate/up, D for down)
  int ldo;                // output row length (F or D)
  void* out;
};

template <typename TA, typename TW, bool GATEUP>
__global__ __launch_bounds__(256) void moe_stream_k(StreamArgs a) {
  typedef typename FragOf<TA>::type Frag;
  __shared__ float red[4][8][64][4];  // [wave][rt*4+ct][lane][i]  32 KB
  const int tile_id = blockIdx.x;
  if (tile_id >= *a.ntiles) return;
  const int4 tl = a.tiles[tile_id];
  const int e = tl.x, row0 = tl.y, nrows = tl.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int K = a.K;

  // A row pointers (2 row tiles) and weight row pointers (4 column tiles)
  const TA* arow[2];
#pragma unroll
  for (int rt = 0; rt < 2; rt++) {
    const int r = rt * 16 + l16;
    if (r < nrows) {
      const int slot = row0 + r;
      const size_t src = GATEUP ? (size_t)(a.perm[slot] / a.k) : (size_t)slot;
      arow[rt] = (const TA*)a.A + src * K;
    } else {
      arow[rt] = nullptr;
    }
  }
  const TW* wrow[4];
  int f0 = 0;
  if (GATEUP) {
    f0 = blockIdx.y * 32;
#pragma unroll
    for (int ct = 0; ct < 4; ct++) {
      const int f = f0 + 16 * (ct >> 1) + l16;
      const TW* base = (const TW*)((ct & 1) ? a.W2 : a.W1);
      wrow[ct] = base + ((size_t)e * a.NW + f) * K;
    }
  } else {
    f0 = blockIdx.y * 64;
#pragma unroll
    for (int ct = 0; ct < 4; ct++)
      wrow[ct] = (const TW*)a.W1 + ((size_t)e * a.NW + f0 + 16 * ct + l16) * K;
  }

  f32x4_t acc[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; rt++)
#pragma unroll
    for (int ct = 0; ct < 4; ct++) acc[rt][ct] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  const int nch = K / 64;

  for (int ch = w; ch < nch; ch += 4) {
#pragma unroll
    for (int s = 0; s < 2; s++) {
      const int kk = ch * 64 + s * 32 + 8 * g;
      Frag af[2], bf[4];
#pragma unroll
      for (int ct = 0; ct < 4; ct++) load_wfrag<TA, TW>(bf[ct], wrow[ct] + kk);
#pragma unroll
      for (int rt = 0; rt < 2; rt++) {
        if (arow[rt]) load_frag(af[rt], arow[rt] + kk);
        else zero_frag(af[rt]);
      }
#pragma unroll
      for (int rt = 0; rt < 2; rt++)
#pragma unroll
        for (int ct = 0; ct < 4; ct++) mma(acc[rt][ct], af[rt], bf[ct]);
    }
  }

#pragma unroll
  for (int rt = 0; rt < 2; rt++)
#pragma unroll
    for (int ct = 0; ct < 4; ct++)
#pragma unroll
      for (int i = 0; i < 4; i++) red[w][rt * 4 + ct][lane][i] = acc[rt][ct][i];
  __syncthreads();

  TA* out = (TA*)a.out;
  if (GATEUP) {
    // thread -> (row tile, f half); combines gate tile 2*fh and up tile 2*fh+1
    const int combo = threadIdx.x >> 6, rt = combo >> 1, fh = combo & 1;
    float sg = 1.f, su = 1.f;
    if (a.escale) {
      sg = a.escale[e * 3 + 0];
      su = a.escale[e * 3 + 1];
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
      float gv = 0.f, uv = 0.f;
#pragma unroll
      for (int q = 0; q < 4; q++) {
        gv += red[q][rt * 4 + 2 * fh][lane][i];
        uv += red[q][rt * 4 + 2 * fh + 1][lane][i];
      }
      const int r = rt * 16 + 4 * g + i;
      if (r < nrows) {
        gv *= sg;
        uv *= su;
        const float h = gv / (1.f + expf(-gv)) * uv;
        stx(out, (size_t)(row0 + r) * a.ldo + f0 + 16 * fh + l16, h);
      }
    }
  } else {
    const float sd = a.escale ? a.escale[e * 3 + 2] : 1.f;
#pragma unroll
    for (int pass = 0; pass < 2; pass++) {
      const int combo = pass * 4 + (threadIdx.x >> 6), rt = combo >> 2, ct = combo & 3;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        float v = 0.f;
#pragma unroll
        for (int q = 0; q < 4; q++) v += red[q][rt * 4 + ct][lane][i];
        const int r = rt * 16 + 4 * g + i;
        if (r < nrows) stx(out, (size_t)(row0 + r) * a.ldo + f0 + 16 * ct + l16, v * sd);
      }
    }
  }
}

// ---------------------------------------------------------------------------
void launch_topk(const float* logits, int rows, int E, int k, int32_t* ids, float* gates,
                 hipStream_t s) {
  topk_k<<<(rows + 3) / 4, 256, 0, s>>>(logits, rows, E, k, ids, gates);
}

void launch_plan(const int32_t* ids, int rows, int k, int E, int tile_rows, int32_t* counts,
                 int32_t* offsets, int32_t* perm, int32_t* inv, int4* tiles, int32_t* ntiles,
                 hipStream_t s) {
  plan_k<<<E, 256, 0, s>>>(ids, rows, k, E, tile_rows, counts, offsets, perm, inv, tiles, ntiles);
}

template <bool GATEUP>
static void stream_dispatch(int act, int wdt, const StreamArgs& a, dim3 grid, hipStream_t s) {
  if (act == ACT_F32)
    moe_stream_k<float, float, GATEUP><<<grid, 256, 0, s>>>(a);
  else if (wdt == DG_FP8E4M3)
    moe_stream_k<uint16_t, uint8_t, GATEUP><<<grid, 256, 0, s>>>(a);
  else
    moe_stream_k<uint16_t, uint16_t, GATEUP><<<grid, 256, 0, s>>>(a);
}

void launch_gateup_stream(int act, const void* u2, const int32_t* perm, int k, const MoeW& w,
                          const int4* tiles, const int32_t* ntiles, int max_tiles, int D, int F,
                          void* H, hipStream_t s) {
  StreamArgs a{u2, perm, k, w.wg, w.wu, w.escale, tiles, ntiles, D, F, F, H};
  stream_dispatch<true>(act, w.wdt, a, dim3(max_tiles, F / 32), s);
}

void launch_down_stream(int act, const void* H, const MoeW& w, const int4* tiles,
                        const int32_t* ntiles, int max_tiles, int D, int F, void* Y, hipStream_t s) {
  StreamArgs a{H, nullptr, 0, w.wd, nullptr, w.escale, tiles, ntiles, F, D, D, Y};
  stream_dispatch<false>(act, w.wdt, a, dim3(max_tiles, D / 64), s);
}

}  // namespace dg
