// kern_moe.hip -- MoE routing: top-k selection with gates, and the permutation
// that groups the (token, slot) entries by expert into row tiles.
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
// ascending).  That order is the order of one 64-bit key per expert (the
// logit's bits mapped to an order-preserving unsigned integer, then the
// complemented index), so each of the k rounds takes the wave maximum of the
// keys not yet selected (DPP reductions, no LDS round trips).  Gates are the
// softmax of the k selected logits.  The logits may arrive as nsplit partial
// sums (contraction splits), added in split order.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t rank_key(float v, int e) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);   // order-preserving
  return ((uint64_t)ord << 32) | (uint32_t)~e;
}
__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t ord = (uint32_t)(key >> 32);
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord);
}

// the k best of one token's logits v[c] (expert lane + 64 c, c < 4; experts past
// E hold key 0, below every real key); writes ids/gates from lanes < k
__device__ __forceinline__ void select_topk(const float (&v)[4], int E, int k, int32_t* ids, float* gates) {
  const int lane = threadIdx.x & 63;
  uint64_t key[4];
#pragma unroll
  for (int c = 0; c < 4; c++) key[c] = lane + 64 * c < E ? rank_key(v[c], lane + 64 * c) : 0;
  float myv = 0.f;
  int myi = 0;
  for (int j = 0; j < k; j++) {
    uint64_t best = umax64(umax64(key[0], key[1]), umax64(key[2], key[3]));
    best = wave_max_u64(best);
    const int e = (int)~(uint32_t)best;
    if (lane == j) {
      myv = key_value(best);
      myi = e;
    }
#pragma unroll
    for (int c = 0; c < 4; c++) key[c] = lane + 64 * c == e ? 0 : key[c];
  }
  const float m0 = __shfl(myv, 0, 64);
  float den = 0.f;
  for (int j = 0; j < k; j++) den += expf(__shfl(myv, j, 64) - m0);
  if (lane < k) {
    ids[lane] = myi;
    gates[lane] = expf(myv - m0) / den;
  }
}

__global__ __launch_bounds__(64) void topk_k(float* __restrict__ logits, int nsplit, int rows, int E,
                                             int k, int32_t* __restrict__ ids, float* __restrict__ gates) {
  const int lane = threadIdx.x;
  const int row = blockIdx.x;
  const size_t stride = (size_t)rows * E;
  float v[4];
#pragma unroll
  for (int c = 0; c < 4; c++) {
    const int e = lane + 64 * c;
    const size_t o = (size_t)row * E + (e < E ? e : 0);
    // all partials in flight at once, then added in split order
    float p[ROUTER_MAX_SPLIT];
#pragma unroll
    for (int sp = 0; sp < ROUTER_MAX_SPLIT; sp++) p[sp] = sp < nsplit ? logits[sp * stride + o] : 0.f;
    float x = p[0];
#pragma unroll
    for (int sp = 1; sp < ROUTER_MAX_SPLIT; sp++) x = sp < nsplit ? x + p[sp] : x;
    if (e < E && nsplit > 1) logits[o] = x;   // the logits routing used
    v[c] = x != x ? -INFINITY : x;  // a NaN logit ranks with -inf (ids stay in range)
  }
  select_topk(v, E, k, ids + (size_t)row * k, gates + (size_t)row * k);
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
  // thread tid reads the k ids of rows tid, tid + 256, ...: all k loads of a
  // row are issued together (k <= 8), and the listing below reads the same rows
  auto load_row = [&](int r, int (&v)[8]) {
#pragma unroll
    for (int j = 0; j < 8; j++) v[j] = r < rows && j < k ? ids[(size_t)r * k + j] : -1;
  };
  hist[tid] = 0;
  __syncthreads();
  for (int r0 = 0; r0 < rows; r0 += 256) {
    int v[8];
    load_row(r0 + tid, v);
#pragma unroll
    for (int j = 0; j < 8; j++)
      if (v[j] >= 0) atomicAdd(&hist[v[j]], 1);
  }
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
    int v[8];
    load_row(r, v);
    int js = -1;
#pragma unroll
    for (int j = 0; j < 8; j++) js = v[j] == e ? j : js;
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
// route_k (bf16): RMSNorm of x1, router logits and top-k in one kernel for a
// tile of 16 tokens.  The normalised rows (rounded to bf16, also written out
// as u2) stay in LDS as the A operand of the router MFMAs; the waves split the
// experts in 16-column tiles (NT tiles each) and stream the packed W_r pieces
// through an NB-deep register ring; the logits go to LDS and each wave ranks 4
// of the tokens with the selection of topk_k.
// ---------------------------------------------------------------------------
template <int NT, int NB>
__global__ __launch_bounds__(256) void route_k(RouteArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  const int D = a.D, E = a.E;
  const int LDA = D + 8;                                          // padded A row (elements)
  uint16_t* sa = reinterpret_cast<uint16_t*>(smem_raw);          // [16][LDA]
  float* sl = reinterpret_cast<float*>(smem_raw + (size_t)16 * LDA * 2);   // [16][E]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l16 = lane & 15, g = lane >> 4;
  const int row0 = blockIdx.x * 16;
  const int nrows = min(16, a.rows - row0);

  // ---- RMSNorm (same arithmetic as rmsnorm_k): wave w takes rows w, w+4, .. ----
  for (int rr = w; rr < 16; rr += 4) {
    uint16_t* dst = sa + rr * LDA;
    if (rr >= nrows) {
      for (int d = lane * 8; d < D; d += 512) *reinterpret_cast<uint4*>(dst + d) = make_uint4(0, 0, 0, 0);
      continue;
    }
    const uint16_t* src = (const uint16_t*)a.x1 + (size_t)(row0 + rr) * D;
    float ss = 0.f;
    for (int d = lane * 8; d < D; d += 512) {
      float v[8];
      ld8(src + d, v);
#pragma unroll
      for (int i = 0; i < 8; i++) ss += v[i] * v[i];
    }
    ss = wave_sum(ss);
    const float r = rsqrtf(ss / (float)D + a.eps);
    for (int d = lane * 8; d < D; d += 512) {
      float v[8];
      ld8(src + d, v);
#pragma unroll
      for (int i = 0; i < 8; i++) v[i] = v[i] * r * a.g2[d + i];
      st8(dst + d, v);
      st8((uint16_t*)a.u2 + (size_t)(row0 + rr) * D + d, v);
    }
  }
  __syncthreads();

  // ---- router logits ----
  if (a.inject) {
    for (int i = threadIdx.x; i < 16 * E; i += 256) {
      const int rr = i / E, e = i % E;
      sl[i] = rr < nrows ? a.inject[(size_t)(row0 + rr) * E + e] : 0.f;
    }
  } else {
    const int nct = (E + 15) / 16;
    const int nkb = D / 64;   // packed pieces (128 bytes of bf16) per router row
    const char* wg[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) {
      const int ct = w + 4 * t;
      wg[t] = (const char*)a.wr + (size_t)(ct < nct ? ct : 0) * nkb * 2048 + 16 * lane;
    }
    f32x4_t acc[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) acc[t] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    u32x4 wv[NB][NT][2];
    auto load = [&](int b, int c) {
#pragma unroll
      for (int t = 0; t < NT; t++)
#pragma unroll
        for (int h = 0; h < 2; h++)
          wv[b][t][h] = *reinterpret_cast<const u32x4*>(wg[t] + (size_t)c * 2048 + h * 1024);
    };
    auto comp = [&](int b, int c) {
#pragma unroll
      for (int h = 0; h < 2; h++) {
        FragBF af;
        load_frag(af, sa + l16 * LDA + c * 64 + 32 * h + 8 * g);
#pragma unroll
        for (int t = 0; t < NT; t++) {
          FragBF bf;
          bf.v = __builtin_bit_cast(bf16x8_t, wv[b][t][h]);
          mma(acc[t], af, bf);
        }
      }
    };
#pragma unroll
    for (int b = 0; b < NB; b++) load(b, b);
    int c0 = 0;
    for (; c0 + NB < nkb; c0 += NB) {   // nkb is a multiple of NB
#pragma unroll
      for (int b = 0; b < NB; b++) {
        __builtin_amdgcn_sched_barrier(0);
        comp(b, c0 + b);
        __builtin_amdgcn_sched_barrier(0);
        load(b, c0 + NB + b);
      }
    }
#pragma unroll
    for (int b = 0; b < NB; b++) {
      __builtin_amdgcn_sched_barrier(0);
      comp(b, c0 + b);
    }
#pragma unroll
    for (int t = 0; t < NT; t++) {
      const int e = (w + 4 * t) * 16 + l16;
#pragma unroll
      for (int i = 0; i < 4; i++)
        if (w + 4 * t < nct && e < E) sl[(4 * g + i) * E + e] = acc[t][i];
    }
  }
  __syncthreads();
  if (a.logits)
    for (int i = threadIdx.x; i < nrows * E; i += 256) a.logits[(size_t)row0 * E + i] = sl[i];

  // ---- top-k: wave w ranks rows w, w+4, w+8, w+12 (same selection as topk_k) ----
  for (int rr = w; rr < nrows; rr += 4) {
    float v[4];
#pragma unroll
    for (int c = 0; c < 4; c++) {
      const int e = lane + 64 * c;
      const float x = e < E ? sl[rr * E + e] : -INFINITY;
      v[c] = x != x ? -INFINITY : x;
    }
    select_topk(v, E, a.k, a.ids + (size_t)(row0 + rr) * a.k, a.gates + (size_t)(row0 + rr) * a.k);
  }
}

size_t route_smem_bytes(int D, int E) {
  return (size_t)16 * (D + 8) * 2 + (size_t)16 * E * 4;
}

template <int NT>
static void launch_route_nt(const RouteArgs& a, size_t smem, hipStream_t s) {
  const int blocks = (a.rows + 15) / 16;
  const int nkb = a.D / 64;
  if (nkb % 8 == 0) route_k<NT, 8><<<blocks, 256, smem, s>>>(a);
  else if (nkb % 4 == 0) route_k<NT, 4><<<blocks, 256, smem, s>>>(a);
  else route_k<NT, 2><<<blocks, 256, smem, s>>>(a);
}

// bf16 activations only; false when the tile does not fit in LDS
bool launch_route(int act, const RouteArgs& a, hipStream_t s) {
  if (act != ACT_BF16) return false;
  constexpr size_t kMaxSmem = 160 * 1024;
  const size_t smem = route_smem_bytes(a.D, a.E);
  if (smem > kMaxSmem) return false;
  // allow more than the default 64 KiB of dynamic LDS (gfx950 has 160 KiB per CU)
  static const bool attr_set = [] {
    bool ok = true;
    const void* fns[] = {(const void*)&route_k<1, 2>, (const void*)&route_k<1, 4>, (const void*)&route_k<1, 8>,
                         (const void*)&route_k<2, 2>, (const void*)&route_k<2, 4>, (const void*)&route_k<2, 8>,
                         (const void*)&route_k<4, 2>, (const void*)&route_k<4, 4>, (const void*)&route_k<4, 8>};
    for (const void* f : fns)
      ok = ok && hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxSmem) == hipSuccess;
    return ok;
  }();
  if (!attr_set && smem > 64 * 1024) return false;
  const int nct = (a.E + 15) / 16;
  if (nct <= 4) launch_route_nt<1>(a, smem, s);
  else if (nct <= 8) launch_route_nt<2>(a, smem, s);
  else launch_route_nt<4>(a, smem, s);
  return true;
}

// ---------------------------------------------------------------------------
void launch_topk(float* logits, int nsplit, int rows, int E, int k, int32_t* ids, float* gates,
                 hipStream_t s) {
  topk_k<<<rows, 64, 0, s>>>(logits, nsplit, rows, E, k, ids, gates);
}

void launch_plan(const int32_t* ids, int rows, int k, int E, int tile_rows, int32_t* counts,
                 int32_t* offsets, int32_t* perm, int32_t* inv, int4* tiles, int32_t* ntiles,
                 hipStream_t s) {
  plan_k<<<E, 256, 0, s>>>(ids, rows, k, E, tile_rows, counts, offsets, perm, inv, tiles, ntiles);
}

}  // namespace dg
