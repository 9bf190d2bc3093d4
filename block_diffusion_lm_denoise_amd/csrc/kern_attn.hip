// kern_attn.hip -- MFMA flash attention with the block mask of a denoising pass.
//
// Denoising mode (explainer "DiffusionGemma", "Two modes, one model"): each
// canvas query of request b attends to the whole cached prefix [0, len[b])
// and to every canvas key of b -- bidirectional.  Prefill mode: query i of the
// new tokens attends to cache keys 0 .. len[b] + i (causal); the new keys were
// written by the projection epilogue first.  Course page "Module 12. Diffusion
// Language Models", block-mask exercise, prints this mask for 3 + 4 tokens.
//
// Block = (query tile, request b, kv head g, key split).  A query tile holds 64
// rows = G query heads sharing kv head g x 64/G consecutive queries, so each
// staged K/V tile serves every head of the group.  Each wave owns 16 rows and
// computes S^T = K Q^T (keys on the MFMA row axis, queries on the column
// axis), so a lane's softmax statistics belong to one query row; then
// O^T += V^T P^T with V staged transposed in LDS (bf16: P as hi + lo bf16).
// Online softmax in fp32 (base-2 exponent with the scale folded in).  The
// next K/V tile is loaded into registers while the current one is used.
// Key splits write unnormalised partials (O, m, l) that a merge kernel
// combines in split order.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace dg {

constexpr int KT = 64;  // keys per staged tile

struct AttnArgs {
  const void* q;
  int ldq;
  const void* kc;
  const void* vc;
  int cap;
  const void* kn;
  const void* vn;
  int T, Hq, Hkv, G, QT;
  int mode;
  int split_len;  // keys per split (multiple of KT)
  int nsplit;
  Lens len;
  float scale_log2;
  void* out;
  float* po;      // [nsplit][rows*Hq][hd]
  float* pml;     // [nsplit][rows*Hq][2]
  int rows;       // B*T
  int nqt, groups;   // query tiles; (request, kv head, split) groups
};

template <typename TA, int HD>
__global__ __launch_bounds__(256) void attn_k(AttnArgs a) {
  typedef typename FragOf<TA>::type Frag;
  constexpr int ES = (int)sizeof(TA);
  constexpr int EPC = 16 / ES;                  // elements per 16-byte chunk
  constexpr int CPR = HD / EPC;                 // chunks per key row
  constexpr int KLD = HD + 16 * EPC / 8;        // padded row of the K tile (bf16: 288 B, conflict-free fragment reads)
  constexpr int VLD = KT + EPC;                 // padded row of the transposed V tile
  constexpr int KCH = KT * CPR / 256;           // K chunks staged per thread
  constexpr int NKG = KT / 4;                   // 4-key groups per tile
  constexpr int NVG = NKG * CPR;                // V groups (4 keys x 1 chunk); the
                                                // key group runs fastest over the
                                                // lanes, so the transposed stores
                                                // of a wave are contiguous in LDS
  constexpr int VCH = (NVG + 255) / 256;        // V groups per thread
  static_assert(KT * CPR % 256 == 0, "K staging");
  // two LDS buffers: tile t+1 is stored while tile t is read
  __shared__ __attribute__((aligned(16))) TA ks2[2][KT * KLD];
  __shared__ __attribute__((aligned(16))) TA vt2[2][HD * VLD];

  // 1-D grid: the query tiles that share one (request, kv head, key split)
  // -- and so read the same K/V -- have ids 8 apart and run on one XCD,
  // whose L2 then serves the K/V tiles after the first read
  const int id = blockIdx.x, nqt = a.nqt;
  const int g = (id / (8 * nqt)) * 8 + id % 8, qt = (id % (8 * nqt)) / 8;
  if (g >= a.groups) return;
  const int bh = g / a.nsplit, split = g % a.nsplit;
  const int b = bh / a.Hkv, gh = bh % a.Hkv;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, l16 = lane & 15, g4 = lane >> 4;
  const int P = a.len.v[b];

  // this lane's query row
  const int trow = 16 * w + l16;
  const int hh = trow / a.QT, qi = qt * a.QT + trow % a.QT;
  const bool qvalid = qi < a.T;
  const int head = gh * a.G + hh;

  // key range of this block
  const int nkeys = a.mode == 0 ? P + a.T : P + min((qt + 1) * a.QT, a.T);
  const int kbeg = split * a.split_len;
  const int kend = min(nkeys, kbeg + a.split_len);
  const int qlimit = a.mode == 0 ? 0x7fffffff : P + qi;  // last key this query may see

  Frag qf[HD / 32];
  {
    const TA* qp = (const TA*)a.q + (size_t)(b * a.T + (qvalid ? qi : 0)) * a.ldq + head * HD;
#pragma unroll
    for (int s = 0; s < HD / 32; s++) {
      if (qvalid) load_frag(qf[s], qp + 32 * s + 8 * g4);
      else zero_frag(qf[s]);
    }
  }
  f32x4_t o[HD / 16];
#pragma unroll
  for (int u = 0; u < HD / 16; u++) o[u] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  float mrow = -INFINITY, lsum = 0.f;

  // K/V of key kk: the cache, or in mode 0 the canvas rows of the qkv buffer
  // for kk >= P.  Keys past the split end read key kbeg (a valid key, so the
  // data is finite): their scores are masked to -inf, so they add nothing.
  // Straight-line selects keep the loads of the next tile in flight.
  const TA* const kc = (const TA*)a.kc + ((size_t)b * a.Hkv + gh) * a.cap * HD;
  const TA* const vc = (const TA*)a.vc + ((size_t)b * a.Hkv + gh) * a.cap * HD;
  const TA* const kn = a.mode == 0 ? (const TA*)a.kn + (size_t)b * a.T * a.ldq + gh * HD : kc;
  const TA* const vn = a.mode == 0 ? (const TA*)a.vn + (size_t)b * a.T * a.ldq + gh * HD : vc;
  const int fresh0 = a.mode == 0 ? P : 0x7fffffff;   // first key read from the qkv rows
  // last key every query of the block may see (the tile's first query in prefill mode)
  const int qlim_all = a.mode == 0 ? 0x7fffffff : P + qt * a.QT;
  const size_t ldq = (size_t)a.ldq;
  auto kptr = [&](int kk, const TA* cache, const TA* fresh) -> const TA* {
    const int k = kk < kend ? kk : kbeg;
    const bool f = k >= fresh0;
    return (f ? fresh : cache) + (size_t)(f ? k - fresh0 : k) * (f ? ldq : (size_t)HD);
  };
  // register ring of two tiles (K chunks and V 4-key groups): the loads of
  // the next two tiles are in flight while a tile is used
  u32x4 rk[2][KCH], rv[2][VCH][4];
  // A tile wholly inside the key range and wholly in the cache (or wholly in
  // the canvas rows) is addressed as a uniform base plus this thread's fixed
  // row offsets; other tiles take the per-key selects.
  auto gload = [&](int buf, int k0) {
    const bool in_range = k0 + KT <= kend;
    const bool all_cache = in_range && k0 + KT <= fresh0;
    const bool all_fresh = in_range && k0 >= fresh0;
    if (all_cache || all_fresh) {
      const size_t rs = all_cache ? (size_t)HD : ldq;
      const TA* kb = all_cache ? kc + (size_t)k0 * HD : kn + (size_t)(k0 - fresh0) * ldq;
      const TA* vb = all_cache ? vc + (size_t)k0 * HD : vn + (size_t)(k0 - fresh0) * ldq;
#pragma unroll
      for (int u = 0; u < KCH; u++) {
        const int id = t + 256 * u, j = id / CPR, q = id % CPR;
        rk[buf][u] = *reinterpret_cast<const u32x4*>(kb + j * rs + q * EPC);
      }
#pragma unroll
      for (int u = 0; u < VCH; u++) {
        const int id = t + 256 * u;
        const int jg = (id < NVG ? id : 0) % NKG, dq = (id < NVG ? id : 0) / NKG;
#pragma unroll
        for (int jj = 0; jj < 4; jj++)
          rv[buf][u][jj] = *reinterpret_cast<const u32x4*>(vb + (4 * jg + jj) * rs + dq * EPC);
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < KCH; u++) {
      const int id = t + 256 * u, j = id / CPR, q = id % CPR;
      rk[buf][u] = *reinterpret_cast<const u32x4*>(kptr(k0 + j, kc, kn) + q * EPC);
    }
#pragma unroll
    for (int u = 0; u < VCH; u++) {
      const int id = t + 256 * u;
      const int jg = (id < NVG ? id : 0) % NKG, dq = (id < NVG ? id : 0) / NKG;
#pragma unroll
      for (int jj = 0; jj < 4; jj++)
        rv[buf][u][jj] = *reinterpret_cast<const u32x4*>(kptr(k0 + 4 * jg + jj, vc, vn) + dq * EPC);
    }
  };
  auto word = [](u32x4 v, int k) -> uint32_t { return v[k]; };
  // LDS: K row-major; V transposed (vt[d][key]), 4 keys of one d per store
  auto sstore = [&](int buf, int lb) {
    TA* ks = ks2[lb];
    TA* vt = vt2[lb];
#pragma unroll
    for (int u = 0; u < KCH; u++) {
      const int id = t + 256 * u, j = id / CPR, q = id % CPR;
      *reinterpret_cast<u32x4*>(ks + j * KLD + q * EPC) = rk[buf][u];
    }
#pragma unroll
    for (int u = 0; u < VCH; u++) {
      const int id = t + 256 * u;
      if (NVG % 256 != 0 && id >= NVG) continue;
      const int jg = id % NKG, dq = id / NKG;
#pragma unroll
      for (int k = 0; k < 4; k++) {
        const uint32_t a0 = word(rv[buf][u][0], k), a1 = word(rv[buf][u][1], k);
        const uint32_t a2 = word(rv[buf][u][2], k), a3 = word(rv[buf][u][3], k);
        if constexpr (ES == 2) {
          // elements 2k (low halves) and 2k+1 (high halves) of the chunk
          const uint2 lo = make_uint2((a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16));
          const uint2 hi = make_uint2((a0 >> 16) | (a1 & 0xffff0000u), (a2 >> 16) | (a3 & 0xffff0000u));
          *reinterpret_cast<uint2*>(vt + (dq * EPC + 2 * k) * VLD + 4 * jg) = lo;
          *reinterpret_cast<uint2*>(vt + (dq * EPC + 2 * k + 1) * VLD + 4 * jg) = hi;
        } else {
          *reinterpret_cast<u32x4*>(vt + (dq * EPC + k) * VLD + 4 * jg) = (u32x4){a0, a1, a2, a3};
        }
      }
    }
  };

  // one key tile: S, online softmax, O update (K and V tiles in LDS buffer
  // lb).  MFMAs are issued so that consecutive ones use different
  // accumulators (a dependent one would wait for the previous result).
  auto compute = [&](int k0, int lb, bool full) {
    const TA* ks = ks2[lb];
    const TA* vt = vt2[lb];
    // ---- S^T = K Q^T: lane holds keys 16*mt + 4*g4 + i for query row l16 ----
    f32x4_t s[KT / 16];
#pragma unroll
    for (int mt = 0; mt < KT / 16; mt++) s[mt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ss = 0; ss < HD / 32; ss++) {
      Frag kf[KT / 16];
#pragma unroll
      for (int mt = 0; mt < KT / 16; mt++) load_frag(kf[mt], ks + (16 * mt + l16) * KLD + 32 * ss + 8 * g4);
#pragma unroll
      for (int mt = 0; mt < KT / 16; mt++) mma(s[mt], kf[mt], qf[ss]);
    }
    // full: every key of the tile is in range and visible to every query of
    // the block, so no masks; the row maximum is taken on the raw scores (the
    // scale is positive) and the scale folds into the exponent's FMA.  Rows
    // past the queries need no mask either: a lane's statistics are its own
    // row's, and those rows are never stored.
    float tmax = -INFINITY;
    if (full) {
      float x = max3_nn(s[0][0], s[0][1], s[0][2]);
#pragma unroll
      for (int mt = 0; mt < KT / 16; mt++)
#pragma unroll
        for (int i = (mt == 0 ? 3 : 0); i < 4; i += 2)
          x = i + 1 < 4 ? max3_nn(x, s[mt][i], s[mt][i + 1]) : max_nn(x, s[mt][i]);
      tmax = x * a.scale_log2;
    } else {
#pragma unroll
      for (int mt = 0; mt < KT / 16; mt++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int kk = k0 + 16 * mt + 4 * g4 + i;
          const bool ok = (kk < kend) & (kk <= qlimit) & qvalid;
          const float v = ok ? s[mt][i] * a.scale_log2 : -INFINITY;
          s[mt][i] = v;
          tmax = fmaxf(tmax, v);
        }
    }
    tmax = pair_max16(tmax);
    tmax = pair_max32(tmax);
    const float mnew = fmaxf(mrow, tmax);
    const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(mrow - mnew);
    float psum = 0.f;
    if (full) {
#pragma unroll
      for (int mt = 0; mt < KT / 16; mt++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][i], a.scale_log2, -mnew));
          s[mt][i] = p;
          psum += p;
        }
    } else {
#pragma unroll
      for (int mt = 0; mt < KT / 16; mt++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const float p = mnew == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s[mt][i] - mnew);
          s[mt][i] = p;
          psum += p;
        }
    }
    lsum = lsum * alpha + psum;
    mrow = mnew;
    if (__ballot(alpha != 1.f)) {   // no row's maximum moved: nothing to rescale
#pragma unroll
      for (int u = 0; u < HD / 16; u++) o[u] *= alpha;
    }

    // ---- O^T += V^T P^T: key slot 8*g4 + 4*t + i <-> key 32*c + 16*t + 4*g4 + i ----
    // bf16: P is split into hi + lo bf16 parts (two MFMAs), so the products
    // keep ~16 mantissa bits of P instead of bf16's 8.
#pragma unroll
    for (int c = 0; c < KT / 32; c++) {
      Frag pf, pl;
      if constexpr (ES == 2) {
        uint32_t ph[4], plo[4];
#pragma unroll
        for (int tt = 0; tt < 2; tt++)
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            const float p0 = s[2 * c + tt][i], p1 = s[2 * c + tt][i + 1];
            const uint32_t h = f2bf2(p0, p1);
            ph[2 * tt + i / 2] = h;
            plo[2 * tt + i / 2] = f2bf2(p0 - __uint_as_float(h << 16), p1 - __uint_as_float(h & 0xffff0000u));
          }
        pf.v = __builtin_bit_cast(bf16x8_t, make_uint4(ph[0], ph[1], ph[2], ph[3]));
        pl.v = __builtin_bit_cast(bf16x8_t, make_uint4(plo[0], plo[1], plo[2], plo[3]));
      } else {
#pragma unroll
        for (int tt = 0; tt < 2; tt++)
#pragma unroll
          for (int i = 0; i < 4; i++) pf.v[4 * tt + i] = s[2 * c + tt][i];
      }
      if constexpr (ES == 2) {
        // four head-dim tiles at a time: their hi products, then their lo products
#pragma unroll
        for (int h4 = 0; h4 < HD / 64; h4++) {
          Frag vf[4];
#pragma unroll
          for (int x = 0; x < 4; x++) {
            const TA* vrow = vt + (16 * (4 * h4 + x) + l16) * VLD + 32 * c + 4 * g4;
            const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
            const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16);
            vf[x].v = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
          }
#pragma unroll
          for (int x = 0; x < 4; x++) mma(o[4 * h4 + x], vf[x], pf);
#pragma unroll
          for (int x = 0; x < 4; x++) mma(o[4 * h4 + x], vf[x], pl);
        }
      } else {
#pragma unroll
        for (int ht = 0; ht < HD / 16; ht++) {
          const TA* vrow = vt + (16 * ht + l16) * VLD + 32 * c + 4 * g4;
          Frag vf;
          float4 lo = *reinterpret_cast<const float4*>(vrow);
          float4 hi = *reinterpret_cast<const float4*>(vrow + 16);
          vf.v[0] = lo.x; vf.v[1] = lo.y; vf.v[2] = lo.z; vf.v[3] = lo.w;
          vf.v[4] = hi.x; vf.v[5] = hi.y; vf.v[6] = hi.z; vf.v[7] = hi.w;
          mma(o[ht], vf, pf);
        }
      }
    }
  };

  // tiles past the split load key kbeg (clamped) and are never computed, so
  // every load is issued unconditionally and the ring indices are constants.
  // Iteration t stores tile t+1 (registers loaded two iterations earlier) in
  // the other LDS buffer, refills those registers with tile t+3 and computes
  // tile t; one barrier per tile makes tile t+1 visible and frees buffer t.
  const int ntile = kend > kbeg ? (kend - kbeg + KT - 1) / KT : 0;
  gload(0, kbeg);
  gload(1, kbeg + KT);
  sstore(0, 0);
  gload(0, kbeg + 2 * KT);
  __syncthreads();
  int it = 0;
  for (; it + 2 <= ntile; it += 2) {
#pragma unroll
    for (int buf = 0; buf < 2; buf++) {
      const int k0 = kbeg + (it + buf) * KT;
      const int nb = buf ^ 1;          // registers (and LDS buffer) of tile it+buf+1
      sstore(nb, nb);
      gload(nb, k0 + 3 * KT);
      compute(k0, buf, k0 + KT <= kend && k0 + KT - 1 <= qlim_all);
      __syncthreads();
    }
  }
  if (it < ntile) {
    const int k0 = kbeg + it * KT;
    compute(k0, 0, k0 + KT <= kend && k0 + KT - 1 <= qlim_all);
  }

  lsum += lane_xor16(lsum);
  lsum += lane_xor32(lsum);
  const size_t row = (size_t)b * a.T + (qvalid ? qi : 0);
  if (a.nsplit == 1) {
    if (!qvalid) return;
    const float inv = 1.f / lsum;
    TA* out = (TA*)a.out + row * (a.Hq * HD) + head * HD;
#pragma unroll
    for (int ht = 0; ht < HD / 16; ht++)
#pragma unroll
      for (int i = 0; i < 4; i++) stx(out, 16 * ht + 4 * g4 + i, o[ht][i] * inv);
    return;
  }

  // ---- key splits: unnormalised partials (O, m, l), merged by attn_merge_k ----
  if (!qvalid) return;
  const size_t e = split * (size_t)a.rows * a.Hq + row * a.Hq + head;
  float* po = a.po + e * HD;
#pragma unroll
  for (int ht = 0; ht < HD / 16; ht++)
#pragma unroll
    for (int i = 0; i < 4; i++) po[16 * ht + 4 * g4 + i] = o[ht][i];
  if (g4 == 0) {
    a.pml[2 * e] = mrow;
    a.pml[2 * e + 1] = lsum;
  }
}

// combine key splits in split order: o = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// A thread owns 8 consecutive head-dimension elements of one (row, head)
// entry; the partial loads of several splits are in flight together.
template <typename TA, int HD>
__global__ __launch_bounds__(256) void attn_merge_k(const float* __restrict__ po,
                                                    const float* __restrict__ pml, int nsplit,
                                                    int entries, TA* __restrict__ out) {
  constexpr int TPE = HD / 8;   // threads per entry
  const int gt = blockIdx.x * 256 + threadIdx.x;
  const int e = gt / TPE, d0 = (gt % TPE) * 8;
  if (e >= entries) return;
  float M = -INFINITY;
  for (int s0 = 0; s0 < nsplit; s0 += 8) {
    float m[8];
#pragma unroll
    for (int j = 0; j < 8; j++) m[j] = s0 + j < nsplit ? pml[2 * ((size_t)(s0 + j) * entries + e)] : -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; j++) M = fmaxf(M, m[j]);
  }
  float den = 0.f, num[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nsplit; s0 += 4) {
    float f[4], l[4];
    float4 v0[4], v1[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int sp = s0 + j < nsplit ? s0 + j : s0;
      const size_t ee = (size_t)sp * entries + e;
      const float mj = pml[2 * ee];
      f[j] = (s0 + j < nsplit && mj != -INFINITY) ? __builtin_amdgcn_exp2f(mj - M) : 0.f;
      l[j] = pml[2 * ee + 1];
      v0[j] = *reinterpret_cast<const float4*>(po + ee * HD + d0);
      v1[j] = *reinterpret_cast<const float4*>(po + ee * HD + d0 + 4);
    }
#pragma unroll
    for (int j = 0; j < 4; j++) {
      den += f[j] * l[j];
      num[0] += f[j] * v0[j].x;
      num[1] += f[j] * v0[j].y;
      num[2] += f[j] * v0[j].z;
      num[3] += f[j] * v0[j].w;
      num[4] += f[j] * v1[j].x;
      num[5] += f[j] * v1[j].y;
      num[6] += f[j] * v1[j].z;
      num[7] += f[j] * v1[j].w;
    }
  }
  const float inv = 1.f / den;
  float r[8];
#pragma unroll
  for (int i = 0; i < 8; i++) r[i] = num[i] * inv;
  st8(out + (size_t)e * HD + d0, r);
}

// ---------------------------------------------------------------------------
// key splits: enough blocks to fill the chip several times over (each block
// is a short latency chain), at least ATTN_MIN_SPLIT_KEYS keys per split
#ifndef ATTN_TARGET_BLOCKS
#define ATTN_TARGET_BLOCKS 512
#endif
#ifndef ATTN_MIN_SPLIT_KEYS
#define ATTN_MIN_SPLIT_KEYS 128
#endif

long attn_partial_entries(int rows, int Hq) {
  // bounded split buffer: at most 2^18 (row, head) entries across all splits
  long full = (long)rows * Hq * 16;
  return full < (1L << 18) ? full : (1L << 18);
}

void launch_attention(const AttnArgsHost& h, hipStream_t s) {
  AttnArgs a{};
  a.q = h.q;
  a.ldq = h.ldq;
  a.kc = h.kc;
  a.vc = h.vc;
  a.cap = h.cap;
  a.kn = h.kn;
  a.vn = h.vn;
  a.T = h.T;
  a.Hq = h.Hq;
  a.Hkv = h.Hkv;
  a.G = h.Hq / h.Hkv;
  a.QT = 64 / a.G;
  a.mode = h.mode;
  a.len = h.len;
  a.scale_log2 = 1.4426950408889634f / sqrtf((float)h.hd);
  a.out = h.out;
  a.po = h.po;
  a.pml = h.pml;
  a.rows = h.B * h.T;

  int maxkeys = 0;
  for (int b = 0; b < h.B; b++) maxkeys = maxkeys > h.len.v[b] + h.T ? maxkeys : h.len.v[b] + h.T;
  const int nqt = (h.T + a.QT - 1) / a.QT;
  const long base = (long)nqt * h.B * h.Hkv;
  int nsplit = 1;
  if (base < ATTN_TARGET_BLOCKS) {
    nsplit = (int)((ATTN_TARGET_BLOCKS + base - 1) / base);
    const int by_keys = (maxkeys + ATTN_MIN_SPLIT_KEYS - 1) / ATTN_MIN_SPLIT_KEYS;
    if (nsplit > by_keys) nsplit = by_keys;
    const long entries = (long)a.rows * h.Hq;
    while (nsplit > 1 && entries * nsplit > h.part_cap) nsplit--;
    if (nsplit < 1) nsplit = 1;
  }
  int split_len = (maxkeys + nsplit - 1) / nsplit;
  split_len = (split_len + KT - 1) / KT * KT;
  nsplit = (maxkeys + split_len - 1) / split_len;
  if (nsplit < 1) nsplit = 1;
  a.split_len = split_len;
  a.nsplit = nsplit;

  a.nqt = nqt;
  a.groups = h.B * h.Hkv * nsplit;
  const dim3 grid((unsigned)(((a.groups + 7) / 8) * 8 * nqt));
  if (h.act == ACT_BF16) {
    if (h.hd == 128) attn_k<uint16_t, 128><<<grid, 256, 0, s>>>(a);
    else attn_k<uint16_t, 64><<<grid, 256, 0, s>>>(a);
  } else {
    if (h.hd == 128) attn_k<float, 128><<<grid, 256, 0, s>>>(a);
    else attn_k<float, 64><<<grid, 256, 0, s>>>(a);
  }
  if (nsplit > 1) {
    const int entries = a.rows * h.Hq;
    const int blocks = (int)(((long)entries * (h.hd / 8) + 255) / 256);
    if (h.act == ACT_BF16) {
      if (h.hd == 128) attn_merge_k<uint16_t, 128><<<blocks, 256, 0, s>>>(h.po, h.pml, nsplit, entries, (uint16_t*)h.out);
      else attn_merge_k<uint16_t, 64><<<blocks, 256, 0, s>>>(h.po, h.pml, nsplit, entries, (uint16_t*)h.out);
    } else {
      if (h.hd == 128) attn_merge_k<float, 128><<<blocks, 256, 0, s>>>(h.po, h.pml, nsplit, entries, (float*)h.out);
      else attn_merge_k<float, 64><<<blocks, 256, 0, s>>>(h.po, h.pml, nsplit, entries, (float*)h.out);
    }
  }
}

}  // namespace dg
