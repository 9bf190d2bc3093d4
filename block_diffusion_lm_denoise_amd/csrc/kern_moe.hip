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
// complemented index), a strict total order, so the ranks are a permutation:
// each lane counts, for its experts, the keys above theirs (all keys are read
// back from LDS as broadcasts); the experts of rank < k are the selection, in
// rank order.  Gates are the softmax of the k selected logits.  The logits
// arrive as nsplit partial sums (contraction splits), added in split order.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool better(float v, int i, float w, int j) {
  return (v > w) | ((v == w) & (i < j));   // bitwise: no short-circuit branches
}

__device__ __forceinline__ uint64_t rank_key(float v, int e) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);   // order-preserving
  return ((uint64_t)ord << 32) | (uint32_t)~e;
}

__global__ __launch_bounds__(64) void topk_k(float* __restrict__ logits, int nsplit, int rows, int E,
                                             int k, int32_t* __restrict__ ids, float* __restrict__ gates) {
  __shared__ __attribute__((aligned(16))) uint64_t sk[256];
  __shared__ float selv[8];
  __shared__ int seli[8];
  const int lane = threadIdx.x;
  const int row = blockIdx.x;
  const size_t stride = (size_t)rows * E;
  float v[4];
  uint64_t key[4];
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
    x = e < E ? x : -INFINITY;
    v[c] = x != x ? -INFINITY : x;  // a NaN logit ranks with -inf (ids stay in range)
    key[c] = rank_key(v[c], e);
    sk[e] = key[c];
  }
  __syncthreads();
  int rank[4] = {0, 0, 0, 0};
  const int nc = (E + 63) / 64;   // lanes' experts actually present
  // keys past E (set above) rank below every real key: counting them is harmless
  for (int e0 = 0; e0 < E; e0 += 8) {
    uint64_t kk[8];
#pragma unroll
    for (int j = 0; j < 8; j++) kk[j] = sk[e0 + j];
#pragma unroll
    for (int j = 0; j < 8; j++)
#pragma unroll
      for (int c = 0; c < 4; c++) rank[c] += c < nc ? (int)(kk[j] > key[c]) : 0;
  }
#pragma unroll
  for (int c = 0; c < 4; c++) {
    const int e = lane + 64 * c;
    if (e < E && rank[c] < k) {
      selv[rank[c]] = v[c];
      seli[rank[c]] = e;
    }
  }
  __syncthreads();
  if (lane < k) {
    float den = 0.f;
    for (int j = 0; j < k; j++) den += expf(selv[j] - selv[0]);
    ids[(size_t)row * k + lane] = seli[lane];
    gates[(size_t)row * k + lane] = expf(selv[lane] - selv[0]) / den;
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
// route_k: RMSNorm of x1, router logits and top-k in one kernel for a tile of
// 16 tokens.  The normalised rows stay in LDS as the A operand of the router
// MFMAs (waves split the experts in 16-column tiles, packed W_r fragments
// come from L2); the logits go to LDS and each wave then ranks 4 of the tokens.
// ---------------------------------------------------------------------------
template <typename TA>
__global__ __launch_bounds__(256) void route_k(RouteArgs a) {
  typedef typename FragOf<TA>::type Frag;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  const int D = a.D, E = a.E;
  const int LDA = D + 16 / (int)sizeof(TA);            // padded A row (elements)
  TA* sa = reinterpret_cast<TA*>(smem_raw);             // [16][LDA]
  float* sl = reinterpret_cast<float*>(smem_raw + (size_t)16 * LDA * sizeof(TA));  // [16][E]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l16 = lane & 15, g = lane >> 4;
  const int row0 = blockIdx.x * 16;
  const int nrows = min(16, a.rows - row0);

  // ---- RMSNorm: wave w normalises rows w, w+4, w+8, w+12 ----
  for (int rr = w; rr < 16; rr += 4) {
    TA* dst = sa + rr * LDA;
    if (rr >= nrows) {
      for (int d = lane; d < D; d += 64) dst[d] = 0;
      continue;
    }
    const TA* src = (const TA*)a.x1 + (size_t)(row0 + rr) * D;
    float ss = 0.f;
    for (int d = lane; d < D; d += 64) {
      const float v = ldx(src, d);
      ss += v * v;
    }
    ss = wave_sum(ss);
    const float r = rsqrtf(ss / (float)D + a.eps);
    for (int d = lane; d < D; d += 64) {
      const float v = ldx(src, d) * r * a.g2[d];
      stx(dst, d, v);
      stx((TA*)a.u2, (size_t)(row0 + rr) * D + d, v);
    }
  }
  __syncthreads();

  // ---- router logits: column tiles of 16 experts split over the waves ----
  if (a.inject) {
    for (int i = threadIdx.x; i < 16 * E; i += 256) {
      const int rr = i / E, e = i % E;
      sl[i] = rr < nrows ? a.inject[(size_t)(row0 + rr) * E + e] : 0.f;
    }
  } else {
    const int nct = (E + 15) / 16;
    const int nkb = D * (int)sizeof(TA) / 128;   // packed pieces per router row
    for (int ct = w; ct < nct; ct += 4) {
      const int e = ct * 16 + l16;
      // packed W_r: row group ct (rows past E are zero), this lane's 16 bytes
      const char* wg = (const char*)a.wr + (size_t)ct * nkb * 2048 + 16 * lane;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      for (int k0 = 0; k0 < D; k0 += 128) {   // D is a multiple of 128
        Frag af[4], bf[4];
#pragma unroll
        for (int u = 0; u < 4; u++) {
          if constexpr (sizeof(TA) == 2) {
            // piece of 64 elements; half u&1 holds elements 32(u&1) + 8g of it
            const int piece = k0 / 64 + (u >> 1);
            load_frag(af[u], sa + l16 * LDA + k0 + 32 * u + 8 * g);
            bf[u].v = __builtin_bit_cast(bf16x8_t,
                                         *reinterpret_cast<const uint4*>(wg + (size_t)piece * 2048 + (u & 1) * 1024));
          } else {
            // piece of 32 floats; lane g holds floats 4g.. and 16+4g.. of it
            const int piece = k0 / 32 + u;
            const float* ar = reinterpret_cast<const float*>(sa) + l16 * LDA + k0 + 32 * u + 4 * g;
            const float4 a0 = *reinterpret_cast<const float4*>(ar);
            const float4 a1 = *reinterpret_cast<const float4*>(ar + 16);
            const float4 w0 = *reinterpret_cast<const float4*>(wg + (size_t)piece * 2048);
            const float4 w1 = *reinterpret_cast<const float4*>(wg + (size_t)piece * 2048 + 1024);
            float* fa = reinterpret_cast<float*>(&af[u]);
            float* fb = reinterpret_cast<float*>(&bf[u]);
            fa[0] = a0.x; fa[1] = a0.y; fa[2] = a0.z; fa[3] = a0.w;
            fa[4] = a1.x; fa[5] = a1.y; fa[6] = a1.z; fa[7] = a1.w;
            fb[0] = w0.x; fb[1] = w0.y; fb[2] = w0.z; fb[3] = w0.w;
            fb[4] = w1.x; fb[5] = w1.y; fb[6] = w1.z; fb[7] = w1.w;
          }
        }
#pragma unroll
        for (int u = 0; u < 4; u++) mma(acc, af[u], bf[u]);
      }
#pragma unroll
      for (int i = 0; i < 4; i++)
        if (e < E) sl[(4 * g + i) * E + e] = acc[i];
    }
  }
  __syncthreads();
  if (a.logits)
    for (int i = threadIdx.x; i < nrows * E; i += 256)
      a.logits[(size_t)row0 * E + i] = sl[i];

  // ---- top-k: wave w ranks rows w, w+4, w+8, w+12 ----
  for (int rr = w; rr < nrows; rr += 4) {
    float v[4];
    bool taken[4];
#pragma unroll
    for (int c = 0; c < 4; c++) {
      const int e = lane + 64 * c;
      const float x = e < E ? sl[rr * E + e] : -INFINITY;
      v[c] = x != x ? -INFINITY : x;
      taken[c] = e >= E;
    }
    float sel_v[8];
    int sel_i[8];
    for (int j = 0; j < a.k; j++) {
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
      for (int j = 0; j < a.k; j++) den += expf(sel_v[j] - sel_v[0]);
      const size_t row = (size_t)(row0 + rr);
      for (int j = 0; j < a.k; j++) {
        a.ids[row * a.k + j] = sel_i[j];
        a.gates[row * a.k + j] = expf(sel_v[j] - sel_v[0]) / den;
      }
    }
  }
}

size_t route_smem_bytes(int act, int D, int E) {
  const size_t esz = act == ACT_BF16 ? 2 : 4;
  return (size_t)16 * (D + 16 / esz) * esz + (size_t)16 * E * 4;
}

bool launch_route(int act, const RouteArgs& a, hipStream_t s) {
  constexpr size_t kMaxSmem = 96 * 1024;
  const size_t smem = route_smem_bytes(act, a.D, a.E);
  if (smem > kMaxSmem) return false;
  // allow more than the default 64 KiB of dynamic LDS (gfx950 has 160 KiB per CU)
  static const bool attr_set = [] {
    hipError_t e1 = hipFuncSetAttribute(reinterpret_cast<const void*>(&route_k<uint16_t>),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxSmem);
    hipError_t e2 = hipFuncSetAttribute(reinterpret_cast<const void*>(&route_k<float>),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxSmem);
    return e1 == hipSuccess && e2 == hipSuccess;
  }();
  if (!attr_set && smem > 64 * 1024) return false;
  const int blocks = (a.rows + 15) / 16;
  if (act == ACT_BF16)
    route_k<uint16_t><<<blocks, 256, smem, s>>>(a);
  else
    route_k<float><<<blocks, 256, smem, s>>>(a);
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
