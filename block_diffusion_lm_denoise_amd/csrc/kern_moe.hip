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

// the k best of the logits of R tokens at once (R independent selections, so
// their wave reductions overlap): v[r][c] is the logit of expert lane + 64 c
// (c < 4; experts past E hold key 0, below every real key).  Writes ids/gates
// of token r from lanes < k when valid[r].
template <int R>
__device__ __forceinline__ void select_topk(const float (&v)[R][4], const bool (&valid)[R], int E, int k,
                                            int32_t* const (&ids)[R], float* const (&gates)[R]) {
  const int lane = threadIdx.x & 63;
  uint64_t key[R][4];
#pragma unroll
  for (int r = 0; r < R; r++)
#pragma unroll
    for (int c = 0; c < 4; c++) key[r][c] = lane + 64 * c < E ? rank_key(v[r][c], lane + 64 * c) : 0;
  float myv[R];
  int myi[R];
#pragma unroll
  for (int r = 0; r < R; r++) {
    myv[r] = 0.f;
    myi[r] = 0;
  }
  for (int j = 0; j < k; j++) {
    uint64_t best[R];
#pragma unroll
    for (int r = 0; r < R; r++) best[r] = wave_max_u64(umax64(umax64(key[r][0], key[r][1]), umax64(key[r][2], key[r][3])));
#pragma unroll
    for (int r = 0; r < R; r++) {
      const int e = (int)~(uint32_t)best[r];
      if (lane == j) {
        myv[r] = key_value(best[r]);
        myi[r] = e;
      }
#pragma unroll
      for (int c = 0; c < 4; c++) key[r][c] = lane + 64 * c == e ? 0 : key[r][c];
    }
  }
#pragma unroll
  for (int r = 0; r < R; r++) {
    // lane j < k holds the j-th selected logit: read them as scalars
    const float m0 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(myv[r]), 0));
    float den = 0.f;
    for (int j = 0; j < k; j++) den += expf(__uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(myv[r]), j)) - m0);
    if (valid[r] && lane < k) {
      ids[r][lane] = myi[r];
      gates[r][lane] = expf(myv[r] - m0) / den;
    }
  }
}

__global__ __launch_bounds__(64) void topk_k(float* __restrict__ logits, int nsplit, int rows, int E,
                                             int k, int32_t* __restrict__ ids, float* __restrict__ gates) {
  const int lane = threadIdx.x;
  const int row = blockIdx.x;
  const size_t stride = (size_t)rows * E;
  float v[1][4];
#pragma unroll
  for (int c = 0; c < 4; c++) {
    const int e = lane + 64 * c;
    const size_t o = (size_t)row * E + (e < E ? e : 0);
    // all partials in flight at once, then added in split order
    float p[ROUTER_MAX_SPLIT];
#pragma unroll
    for (int sp = 0; sp < ROUTER_MAX_SPLIT; sp++)   // splits past nsplit re-read split 0 (not added): no branches
      p[sp] = logits[(sp < nsplit ? sp : 0) * stride + o];
    float x = p[0];
#pragma unroll
    for (int sp = 1; sp < ROUTER_MAX_SPLIT; sp++) x = sp < nsplit ? x + p[sp] : x;
    if (e < E && nsplit > 1) logits[o] = x;   // the logits routing used
    v[0][c] = x != x ? -INFINITY : x;  // a NaN logit ranks with -inf (ids stay in range)
  }
  const bool valid[1] = {true};
  int32_t* const idp[1] = {ids + (size_t)row * k};
  float* const gp[1] = {gates + (size_t)row * k};
  select_topk<1>(v, valid, E, k, idp, gp);
}

// Top-k with the RMSNorm in front of the router folded in (one wave per
// row).  The row's x1 and g2 loads go out first, beside the router partials:
// none of them depends on the others.  The wave sums the squares of its row
// (8 consecutive elements per lane and 512-element chunk), writes
// u2 = round(x1 * r * g2) with r = rsqrt(mean(x1^2) + eps), and ranks the
// logits: the split sums times r when the router ran on round(x1 * g2)
// (scale set), else the logits as given (injected).
template <typename TA>
__global__ __launch_bounds__(64) void topk_norm_k(float* __restrict__ logits, int nsplit, int rows,
                                                  int E, int k, int32_t* __restrict__ ids,
                                                  float* __restrict__ gates, const TA* __restrict__ x1,
                                                  const float* __restrict__ g2, int D, float eps,
                                                  TA* __restrict__ u2, int scale) {
  constexpr int NC = 4;   // 512-element chunks held in registers (rows up to 2048)
  const int lane = threadIdx.x;
  const int row = blockIdx.x;
  const TA* xr = x1 + (size_t)row * D;
  float xv[NC][8], gv[NC][8];
#pragma unroll
  for (int c = 0; c < NC; c++) {   // chunks past the row re-read element 0 (never used): no branches
    const int i = lane * 8 + 512 * c, ii = i < D ? i : 0;
    ld8(xr + ii, xv[c]);
    ld8(g2 + ii, gv[c]);
  }
  const size_t stride = (size_t)rows * E;
  float p[4][ROUTER_MAX_SPLIT];
#pragma unroll
  for (int c = 0; c < 4; c++) {
    const int e = lane + 64 * c;
    const size_t o = (size_t)row * E + (e < E ? e : 0);
#pragma unroll
    for (int sp = 0; sp < ROUTER_MAX_SPLIT; sp++)
      p[c][sp] = logits[(sp < nsplit ? sp : 0) * stride + o];
  }
  __builtin_amdgcn_sched_barrier(0);   // every load above is issued before the first use
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < NC; c++)
    if (lane * 8 + 512 * c < D)
#pragma unroll
      for (int i = 0; i < 8; i++) ss += xv[c][i] * xv[c][i];
  for (int i0 = lane * 8 + 512 * NC; i0 < D; i0 += 512) {   // longer rows
    float w[8];
    ld8(xr + i0, w);
#pragma unroll
    for (int i = 0; i < 8; i++) ss += w[i] * w[i];
  }
  ss = wave_sum(ss);
  const float r = rsqrtf(ss / (float)D + eps);
  TA* ur = u2 + (size_t)row * D;
#pragma unroll
  for (int c = 0; c < NC; c++) {
    const int i0 = lane * 8 + 512 * c;
    if (i0 < D) {
#pragma unroll
      for (int i = 0; i < 8; i++) xv[c][i] = xv[c][i] * r * gv[c][i];
      st8(ur + i0, xv[c]);
    }
  }
  for (int i0 = lane * 8 + 512 * NC; i0 < D; i0 += 512) {
    float w[8], h[8];
    ld8(xr + i0, w);
    ld8(g2 + i0, h);
#pragma unroll
    for (int i = 0; i < 8; i++) w[i] = w[i] * r * h[i];
    st8(ur + i0, w);
  }
  float v[1][4];
#pragma unroll
  for (int c = 0; c < 4; c++) {
    const int e = lane + 64 * c;
    float x = p[c][0];
#pragma unroll
    for (int sp = 1; sp < ROUTER_MAX_SPLIT; sp++) x = sp < nsplit ? x + p[c][sp] : x;
    if (scale) x *= r;
    // the logits routing used (the router tap reads them back)
    if (e < E && (nsplit > 1 || scale)) logits[(size_t)row * E + e] = x;
    v[0][c] = x != x ? -INFINITY : x;  // a NaN logit ranks with -inf (ids stay in range)
  }
  const bool valid[1] = {true};
  int32_t* const idp[1] = {ids + (size_t)row * k};
  float* const gp[1] = {gates + (size_t)row * k};
  select_topk<1>(v, valid, E, k, idp, gp);
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
  auto load_row = [&](int r, int (&v)[8]) {   // clamped loads, then a select: no branches
    const bool rok = r < rows;
    const size_t base = (size_t)(rok ? r : 0) * k;
    if (k == 8) {   // uniform: a row's ids are 32 aligned bytes, two 16-byte loads
      const int4 lo = *reinterpret_cast<const int4*>(ids + base);
      const int4 hi = *reinterpret_cast<const int4*>(ids + base + 4);
      v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
      v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    } else {
#pragma unroll
      for (int j = 0; j < 8; j++) v[j] = ids[base + (j < k ? j : 0)];
    }
#pragma unroll
    for (int j = 0; j < 8; j++) v[j] = rok && j < k ? v[j] : -1;
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
// tile of 16 tokens, 8 waves.  The normalised rows (rounded to bf16, also
// written out as u2) stay in LDS (rows padded to a 32 mod 64 byte stride) as
// the A operand of the router MFMAs.  Wave w takes the expert column tiles of
// group w % 4 (NT 16-column tiles) over half w / 4 of the contraction and
// streams the packed W_r pieces through an NB-deep register ring; the two
// halves are added in LDS in a fixed order; each wave then ranks 2 tokens
// with the selection of topk_k.
// ---------------------------------------------------------------------------
constexpr int ROUTE_THREADS = 512;

template <int NT, int NB>
__global__ __launch_bounds__(ROUTE_THREADS) void route_k(RouteArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  const int D = a.D, E = a.E;
  const int LDA = D + 16;                                         // padded A row (elements)
  const int nct = (E + 15) / 16;
  uint16_t* sa = reinterpret_cast<uint16_t*>(smem_raw);          // [16][LDA]
  float* sl = reinterpret_cast<float*>(smem_raw + (size_t)16 * LDA * 2);   // [16][E]
  float* red = sl + 16 * E;                                       // [2][nct][16][16]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l16 = lane & 15, g = lane >> 4;
  const int row0 = blockIdx.x * 16;
  const int nrows = min(16, a.rows - row0);

  // ---- RMSNorm (same arithmetic as rmsnorm_k): wave w takes rows w, w + 8 ----
  if (D % 512 == 0 && D <= 2048) {
    // all loads of the wave's rows in flight at once; the values stay in
    // registers for the scaling pass
    const int nc = D / 512;
    u32x4 raw[2][4];
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int rr = w + 8 * j;
      const uint16_t* src = (const uint16_t*)a.x1 + (size_t)(row0 + (rr < nrows ? rr : 0)) * D;
#pragma unroll
      for (int i = 0; i < 4; i++)   // chunks past the row re-read chunk 0 (never used): no branches
        raw[j][i] = *reinterpret_cast<const u32x4*>(src + lane * 8 + 512 * (i < nc ? i : 0));
    }
    float gv[4][8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float4* gp4 = reinterpret_cast<const float4*>(a.g2 + lane * 8 + 512 * (i < nc ? i : 0));
      const float4 g0 = gp4[0], g1 = gp4[1];
      gv[i][0] = g0.x; gv[i][1] = g0.y; gv[i][2] = g0.z; gv[i][3] = g0.w;
      gv[i][4] = g1.x; gv[i][5] = g1.y; gv[i][6] = g1.z; gv[i][7] = g1.w;
    }
    __builtin_amdgcn_sched_barrier(0);   // every load above is issued before the first use
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int rr = w + 8 * j;
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const float lo = __uint_as_float(raw[j][i][q] << 16), hi = __uint_as_float(raw[j][i][q] & 0xffff0000u);
          ss += i < nc ? lo * lo : 0.f;
          ss += i < nc ? hi * hi : 0.f;
        }
      ss = row16_sum(ss);
      ss += lane_xor16(ss);
      ss += lane_xor32(ss);
      const float r = rsqrtf(ss / (float)D + a.eps);
      uint16_t* dst = sa + rr * LDA;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        if (i >= nc) continue;
        float v[8];
#pragma unroll
        for (int q = 0; q < 4; q++) {
          v[2 * q] = __uint_as_float(raw[j][i][q] << 16) * r * gv[i][2 * q];
          v[2 * q + 1] = __uint_as_float(raw[j][i][q] & 0xffff0000u) * r * gv[i][2 * q + 1];
        }
        if (rr >= nrows) {
#pragma unroll
          for (int q = 0; q < 8; q++) v[q] = 0.f;
        }
        st8(dst + lane * 8 + 512 * i, v);
        if (rr < nrows) st8((uint16_t*)a.u2 + (size_t)(row0 + rr) * D + lane * 8 + 512 * i, v);
      }
    }
  } else {
    for (int rr = w; rr < 16; rr += 8) {
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
  }
  __syncthreads();

  // ---- router logits ----
  if (a.inject) {
    for (int i = threadIdx.x; i < 16 * E; i += ROUTE_THREADS) {
      const int rr = i / E, e = i % E;
      sl[i] = rr < nrows ? a.inject[(size_t)(row0 + rr) * E + e] : 0.f;
    }
  } else {
    const int cgp = w & 3, kh = w >> 2;
    const int nkb = D / 64;           // packed pieces (128 bytes of bf16) per router row
    const int per = nkb / 2;          // pieces of this wave's contraction half (a multiple of NB)
    const int c0 = kh * per;
    const char* wg[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) {
      const int ct = cgp + 4 * t;
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
    for (int b = 0; b < NB; b++) load(b, c0 + b);
    int i0 = 0;
    for (; i0 + NB < per; i0 += NB) {
#pragma unroll
      for (int b = 0; b < NB; b++) {
        __builtin_amdgcn_sched_barrier(0);
        comp(b, c0 + i0 + b);
        __builtin_amdgcn_sched_barrier(0);
        load(b, c0 + i0 + NB + b);
      }
    }
#pragma unroll
    for (int b = 0; b < NB; b++) {
      __builtin_amdgcn_sched_barrier(0);
      comp(b, c0 + i0 + b);
    }
#pragma unroll
    for (int t = 0; t < NT; t++) {
      const int ct = cgp + 4 * t;
      if (ct < nct)
#pragma unroll
        for (int i = 0; i < 4; i++) red[((kh * nct + ct) * 16 + 4 * g + i) * 16 + l16] = acc[t][i];
    }
    __syncthreads();
    // the two contraction halves, added in a fixed order
    for (int i = threadIdx.x; i < 16 * E; i += ROUTE_THREADS) {
      const int rr = i / E, e = i % E, ct = e >> 4, col = e & 15;
      sl[i] = red[(ct * 16 + rr) * 16 + col] + red[((nct + ct) * 16 + rr) * 16 + col];
    }
  }
  __syncthreads();
  if (a.logits)
    for (int i = threadIdx.x; i < nrows * E; i += ROUTE_THREADS) a.logits[(size_t)row0 * E + i] = sl[i];

  // ---- top-k: wave w ranks rows w and w + 8 together (the selection of topk_k) ----
  float v[2][4];
  bool valid[2];
  int32_t* idp[2];
  float* gp[2];
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int rr = w + 8 * j;
    valid[j] = rr < nrows;
    idp[j] = a.ids + (size_t)(row0 + (valid[j] ? rr : 0)) * a.k;
    gp[j] = a.gates + (size_t)(row0 + (valid[j] ? rr : 0)) * a.k;
#pragma unroll
    for (int c = 0; c < 4; c++) {
      const int e = lane + 64 * c;
      const float x = e < E ? sl[rr * E + e] : -INFINITY;
      v[j][c] = x != x ? -INFINITY : x;
    }
  }
  select_topk<2>(v, valid, E, a.k, idp, gp);
}

size_t route_smem_bytes(int D, int E) {
  const size_t nct = (size_t)(E + 15) / 16;
  return (size_t)16 * (D + 16) * 2 + (size_t)16 * E * 4 + 2 * nct * 256 * 4;
}

template <int NT>
static void launch_route_nt(const RouteArgs& a, size_t smem, hipStream_t s) {
  const int blocks = (a.rows + 15) / 16;
  const int per = a.D / 128;   // pieces per contraction half
  if (NT < 4 && per % 8 == 0) route_k<NT, 8><<<blocks, ROUTE_THREADS, smem, s>>>(a);   // 4 tiles x 8 spills
  else if (per % 4 == 0) route_k<NT, 4><<<blocks, ROUTE_THREADS, smem, s>>>(a);
  else if (per % 2 == 0) route_k<NT, 2><<<blocks, ROUTE_THREADS, smem, s>>>(a);
  else route_k<NT, 1><<<blocks, ROUTE_THREADS, smem, s>>>(a);
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
    const void* fns[] = {(const void*)&route_k<1, 1>, (const void*)&route_k<1, 2>, (const void*)&route_k<1, 4>,
                         (const void*)&route_k<1, 8>, (const void*)&route_k<2, 1>, (const void*)&route_k<2, 2>,
                         (const void*)&route_k<2, 4>, (const void*)&route_k<2, 8>, (const void*)&route_k<4, 1>,
                         (const void*)&route_k<4, 2>, (const void*)&route_k<4, 4>};
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

void launch_topk_norm(int act, float* logits, int nsplit, int rows, int E, int k, int32_t* ids,
                      float* gates, const TopkNorm& tn, hipStream_t s) {
  if (act == ACT_BF16)
    topk_norm_k<uint16_t><<<rows, 64, 0, s>>>(logits, nsplit, rows, E, k, ids, gates,
                                               (const uint16_t*)tn.x1, tn.g2, tn.D, tn.eps,
                                               (uint16_t*)tn.u2, tn.scale);
  else
    topk_norm_k<float><<<rows, 64, 0, s>>>(logits, nsplit, rows, E, k, ids, gates,
                                            (const float*)tn.x1, tn.g2, tn.D, tn.eps, (float*)tn.u2,
                                            tn.scale);
}

void launch_plan(const int32_t* ids, int rows, int k, int E, int tile_rows, int32_t* counts,
                 int32_t* offsets, int32_t* perm, int32_t* inv, int4* tiles, int32_t* ntiles,
                 hipStream_t s) {
  plan_k<<<E, 256, 0, s>>>(ids, rows, k, E, tile_rows, counts, offsets, perm, inv, tiles, ntiles);
}

}  // namespace dg
