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

#include <type_traits>

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
  void* po;       // [nsplit][rows*Hq][hd], elements of the activation type
  float* pml;     // [nsplit][rows*Hq][2]
  int rows;       // B*T
  int nqt, groups;   // query tiles; (request, kv head, split) groups
};

// Block id -> (request b, kv head gh, key split, query tile qt).  The query
// tiles that share one (request, kv head, key split) -- and so read the same
// K/V -- have ids 8 apart and run on one XCD, whose L2 then serves the K/V
// tiles after the first read.  False for the padding ids of the last group.
__host__ __device__ inline bool attn_block(int id, int nqt, int groups, int nsplit, int Hkv,
                                           int& b, int& gh, int& split, int& qt) {
  const int g = (id / (8 * nqt)) * 8 + id % 8;
  qt = (id % (8 * nqt)) / 8;
  if (g >= groups) return false;
  const int bh = g / nsplit;
  split = g % nsplit;
  b = bh / Hkv;
  gh = bh % Hkv;
  return true;
}

// The key a block addresses for key index kk of its staged tiles.  Keys of
// the split [kbeg, kend) are read as they are; the staged tiles run past the
// split end (the pipeline loads whole tiles, and two tiles ahead), and those
// slots read a key of the same request that holds data: kbeg when the split
// has keys, else key 0 (a request always has at least one key: T >= 1).
// Their scores are masked to -inf, so the data only has to be finite.
__host__ __device__ inline int attn_key_index(int kk, int kbeg, int kend) {
  return kk < kend ? kk : (kbeg < kend ? kbeg : 0);
}

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

  int b, gh, split, qt;
  if (!attn_block(blockIdx.x, a.nqt, a.groups, a.nsplit, a.Hkv, b, gh, split, qt)) return;
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
  // for kk >= P.  Slots past the split end read a key of this request
  // (attn_key_index): their scores are masked to -inf, so they add nothing.
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
    const int k = attn_key_index(kk, kbeg, kend);
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
      float x = fmax3(s[0][0], s[0][1], s[0][2]);
#pragma unroll
      for (int mt = 0; mt < KT / 16; mt++)
#pragma unroll
        for (int i = (mt == 0 ? 3 : 0); i < 4; i += 2)
          x = i + 1 < 4 ? fmax3(x, s[mt][i], s[mt][i + 1]) : __builtin_fmaxf(x, s[mt][i]);
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
  float* po = static_cast<float*>(a.po) + e * HD;
#pragma unroll
  for (int ht = 0; ht < HD / 16; ht++)
#pragma unroll
    for (int i = 0; i < 4; i++) po[16 * ht + 4 * g4 + i] = o[ht][i];
  if (g4 == 0) {
    a.pml[2 * e] = mrow;
    a.pml[2 * e + 1] = lsum;
  }
}

// ---------------------------------------------------------------------------
// bf16 attention (gfx950).  Block = NW waves x 32 rows = 32 NW (query, head)
// rows of one (request, kv head, key split): G query heads sharing the kv head
// x 32 NW / G consecutive queries.  K and V tiles of 64 keys go from memory
// straight into LDS (global_load_lds, 16 bytes per lane: a wave load fills
// 1 KB of LDS with 4 (hd 128) or 8 (hd 64) key rows); the 16-byte chunks of a
// key row are stored XOR-swizzled by the key index, so both the K fragment
// reads (16 keys x 64 bytes) and the transposing V reads (16 keys x 32 bytes)
// spread over all LDS banks.
//   S^T = K Q^T: keys on the MFMA row axis, queries on the column axis, so a
//   lane's softmax statistics belong to one query row (two per lane: the
//   wave's two 16-row tiles).
//   O^T += V^T P^T: the V^T operand comes from the row-major V tile through
//   the gfx950 transposing LDS read (ds_read_b64_tr_b16: 16 lanes read 4 key
//   rows x 16 dims and each lane receives one dim of the 4 keys), with the
//   key order of a lane's S^T accumulators, so P is used in place (one bf16
//   rounding of the probabilities).
// Software pipeline over key tiles, one barrier per tile: step t computes the
// scores S(t) on the matrix cores while the vector units turn S(t-1) into
// probabilities, then accumulates P(t-1) V(t-1) (and the row sums, as a
// product with an all-ones operand) while the vector units take the lane
// maxima of S(t).  The K tiles run one tile ahead of the V tiles: step t
// loads K(t+1) and V(t) (two buffers each), so a tile's loads have a whole
// step to land.
// Online softmax in fp32 (base-2 exponent with the scale folded in).  The
// running maximum is moved (and O and the sum rescaled) only when a tile's
// maximum exceeds it by more than 2^8: until then the probabilities of a
// tile are at most 256 times larger than with the exact maximum, which fp32
// sums and bf16 probabilities hold exactly as well, and the final division
// by the sum uses the same reference.
// ---------------------------------------------------------------------------
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr float ATTN_RESCALE_LOG2 = 8.f;   // move the running maximum past this margin

template <int HD, int NW, int KT, int J>
__global__ __launch_bounds__(NW * 64, 2) void attn_bf16_k(AttnArgs a) {
  // J 16-row tiles per wave, NW waves: 16 J NW (query, head) rows per block;
  // KT keys per tile
  constexpr int MT = KT / 16;            // 16-key tiles of S
  constexpr int NCH = KT / 32;           // 32-key chunks of P V
  constexpr int RBY = HD * 2;            // bytes of one key row
  constexpr int CPK = RBY / 16;          // 16-byte chunks per key row (16 or 8)
  constexpr int TB = KT * RBY;           // bytes of a K (or V) tile
  constexpr int KPI = 1024 / RBY;        // key rows per 1 KB wave load
  constexpr int NIW = TB / 1024 / NW;    // wave loads per wave per K (or V) tile
  constexpr int NSS = HD / 32;           // contraction steps of S
  constexpr int NHT = HD / 16;           // 16-dim tiles of O
  static_assert(NIW >= 1 && NIW * NW * 1024 == TB, "tile");
  // K tile buffers at 0 and TB, V tile buffers at 2 TB and 3 TB
  __shared__ __attribute__((aligned(1024))) char lds[4 * TB];

  int b, gh, split, qt;
  if (!attn_block(blockIdx.x, a.nqt, a.groups, a.nsplit, a.Hkv, b, gh, split, qt)) return;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, l16 = lane & 15, g4 = lane >> 4;
  const int P = a.len.v[b];

  // the wave's 16-row tiles; this lane's query row in each
  int qi[J], head[J], qlim[J];
  bool qv[J];
#pragma unroll
  for (int j = 0; j < J; j++) {
    const int r = 16 * J * w + 16 * j + l16;
    qi[j] = qt * a.QT + r % a.QT;
    qv[j] = qi[j] < a.T;
    head[j] = gh * a.G + r / a.QT;
    qlim[j] = a.mode == 0 ? 0x7fffffff : P + qi[j];   // last key the query may see
  }
  const int nkeys = a.mode == 0 ? P + a.T : P + min((qt + 1) * a.QT, a.T);
  const int kbeg = split * a.split_len;
  const int kend = min(nkeys, kbeg + a.split_len);
  // last key every query of the block may see (the tile's first query in prefill mode)
  const int qlim_all = a.mode == 0 ? 0x7fffffff : P + qt * a.QT;
  const float c2 = a.scale_log2, inv_c2 = 1.f / a.scale_log2;

  FragBF qf[J][NSS];
#pragma unroll
  for (int j = 0; j < J; j++) {
    const uint16_t* qp = (const uint16_t*)a.q + (size_t)(b * a.T + (qv[j] ? qi[j] : 0)) * a.ldq + head[j] * HD;
#pragma unroll
    for (int ss = 0; ss < NSS; ss++) {
      load_frag(qf[j][ss], qp + 32 * ss + 8 * g4);
      mask_frag(qf[j][ss], qv[j]);
    }
  }

  // key sources, uniform across the block (readfirstlane keeps them in
  // scalar registers, so uniform tiles load with a scalar base and a 32-bit
  // lane offset)
  const char* const kc = uniform_ptr((const uint16_t*)a.kc + ((size_t)b * a.Hkv + gh) * a.cap * HD);
  const char* const vc = uniform_ptr((const uint16_t*)a.vc + ((size_t)b * a.Hkv + gh) * a.cap * HD);
  const char* const kn = a.mode == 0 ? uniform_ptr((const uint16_t*)a.kn + (size_t)b * a.T * a.ldq + gh * HD) : kc;
  const char* const vn = a.mode == 0 ? uniform_ptr((const uint16_t*)a.vn + (size_t)b * a.T * a.ldq + gh * HD) : vc;
  const int fresh0 = a.mode == 0 ? P : 0x7fffffff;   // first key read from the qkv rows
  const uint32_t ldqb = (uint32_t)a.ldq * 2;         // bytes between two qkv rows

  // this lane's slot of each wave load: key row lkey[u] of the tile, global
  // chunk lq[u] (stored at slot lane % CPK = lq ^ (key % CPK)); its byte
  // offset from the tile's first key in the cache (coff) and in the qkv rows
  // (foff)
  int lkey[NIW], lq[NIW];
  uint32_t coff[NIW], foff[NIW];
#pragma unroll
  for (int u = 0; u < NIW; u++) {
    lkey[u] = (w * NIW + u) * KPI + lane / CPK;
    lq[u] = (lane % CPK) ^ (lkey[u] & (CPK - 1));
    coff[u] = (uint32_t)(lkey[u] * RBY + lq[u] * 16);
    foff[u] = (uint32_t)lkey[u] * ldqb + lq[u] * 16;
  }
  // K (KV = 0) or V (KV = 1) tile at key k0 into LDS buffer NB.  A tile
  // wholly inside the key range and wholly in the cache (or in the canvas
  // rows) is read from a uniform base plus the lane offsets; other tiles take
  // per-key sources (attn_key_index keeps the slots past the split end on
  // keys of this request).
  auto issue = [&](auto kvc, auto nbc, int k0) __attribute__((always_inline)) {
    constexpr int KV = decltype(kvc)::value, NB = decltype(nbc)::value;
    char* const dst = lds + (2 * KV + NB) * TB + w * NIW * 1024;
    const char* const cb = KV ? vc : kc;
    const char* const fb = KV ? vn : kn;
    const bool in_range = k0 + KT <= kend;
    if (in_range && k0 + KT <= fresh0) {
      const char* base = cb + (size_t)k0 * RBY;
#pragma unroll
      for (int u = 0; u < NIW; u++) lds_dma16(base + coff[u], dst + u * 1024);
    } else if (in_range && k0 >= fresh0) {
      const char* base = fb + (size_t)(k0 - fresh0) * ldqb;
#pragma unroll
      for (int u = 0; u < NIW; u++) lds_dma16(base + foff[u], dst + u * 1024);
    } else {
#pragma unroll
      for (int u = 0; u < NIW; u++) {
        // per-key source, as integer selects (a select between two pointers
        // is otherwise lowered to a table in private memory)
        const int k = attn_key_index(k0 + lkey[u], kbeg, kend);
        const bool f = k >= fresh0;
        const uint64_t off = f ? (uint64_t)(k - fresh0) * ldqb : (uint64_t)k * RBY;
        const uint64_t base = f ? (uint64_t)(uintptr_t)fb : (uint64_t)(uintptr_t)cb;
        lds_dma16((const char*)(uintptr_t)(base + off) + lq[u] * 16, dst + u * 1024);
      }
    }
  };

  f32x4_t o[J][NHT];
  float mrow[J];    // reference maximum of the row (log2 units); -inf before its first key
  float mneg[J];    // exponent offset -mrow (0 while mrow is -inf)
  float thr[J];     // raw score above which the reference moves: (mrow + margin) / c2
  f32x4_t ls[J];    // row sums of the probabilities (every element holds the sum)
#pragma unroll
  for (int j = 0; j < J; j++) {
#pragma unroll
    for (int u = 0; u < NHT; u++) o[j][u] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    mrow[j] = -INFINITY;
    mneg[j] = 0.f;
    thr[j] = -INFINITY;
    ls[j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  }
  FragBF ones;
  ones.v = __builtin_bit_cast(bf16x8_t, make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));
  f32x4_t sa[J][MT], sb[J][MT];   // raw scores of the even and of the odd tiles

  // LDS byte offsets of this lane's reads within a tile buffer.  K fragment
  // (16 mt + l16, chunk 4 ss + g4): koff[ss] + 16 mt RBY.  V^T operand (keys
  // 32 c + 16 h + 4 g4 + l16 / 4, dims 16 ht + 4 (l16 % 4)): voff[ht] +
  // (32 c + 16 h) RBY.  The swizzle depends on the key only modulo 16, so
  // the key-tile parts are constants the reads carry as immediate offsets.
  int koff[NSS], voff[NHT];
#pragma unroll
  for (int ss = 0; ss < NSS; ss++) koff[ss] = l16 * RBY + 16 * ((4 * ss + g4) ^ (l16 & (CPK - 1)));
#pragma unroll
  for (int ht = 0; ht < NHT; ht++) {
    const int r = 4 * g4 + (l16 >> 2);
    const int byte = 32 * ht + 8 * (l16 & 3);
    voff[ht] = r * RBY + 16 * ((byte >> 4) ^ (r & (CPK - 1))) + (byte & 15);
  }

  // S^T(t) = K(t) Q^T for the wave's row tiles (K tile in buffer PB)
  auto scores = [&](auto pbc, f32x4_t (&s)[J][MT]) __attribute__((always_inline)) {
    constexpr int PB = decltype(pbc)::value;
#pragma unroll
    for (int ss = 0; ss < NSS; ss++) {
      FragBF kf[MT];
#pragma unroll
      for (int mt = 0; mt < MT; mt++)
        kf[mt].v = *reinterpret_cast<const bf16x8_t*>(lds + PB * TB + mt * 16 * RBY + koff[ss]);
#pragma unroll
      for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int j = 0; j < J; j++) {
          if (ss == 0) s[j][mt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
          mma(s[j][mt], kf[mt], qf[j][ss]);
        }
    }
  };
  // scores of keys outside the split or past a query's causal limit -> -inf
  auto mask = [&](f32x4_t (&s)[J][MT], int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < J; j++)
#pragma unroll
      for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int kk = k0 + 16 * mt + 4 * g4 + i;
          const bool ok = (kk < kend) & (kk <= qlim[j]) & qv[j];
          s[j][mt][i] = ok ? s[j][mt][i] : -INFINITY;
        }
  };
  // probabilities 2^(c s - m) as bf16 B fragments of the 32-key chunks (a
  // row that has seen no key has m = -inf and all its scores -inf: offset 0
  // gives probabilities 0)
  auto probs = [&](const f32x4_t (&s)[J][MT], FragBF (&pf)[J][NCH]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < J; j++) {
      float p[MT][4];
#pragma unroll
      for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int i = 0; i < 4; i++) p[mt][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j][mt][i], c2, mneg[j]));
#pragma unroll
      for (int c = 0; c < NCH; c++)
        pf[j][c].v = __builtin_bit_cast(bf16x8_t, make_uint4(f2bf2(p[2 * c][0], p[2 * c][1]),
                                                             f2bf2(p[2 * c][2], p[2 * c][3]),
                                                             f2bf2(p[2 * c + 1][0], p[2 * c + 1][1]),
                                                             f2bf2(p[2 * c + 1][2], p[2 * c + 1][3])));
    }
  };
  // O^T += V^T P^T over the 32-key chunks of the tile (V tile in buffer PB),
  // and the row sums of the same bf16 probabilities on the matrix cores (an
  // all-ones A operand: every row of the product holds the column sums)
  auto pv = [&](auto pbc, const FragBF (&pf)[J][NCH]) __attribute__((always_inline)) {
    constexpr int PB = decltype(pbc)::value;
#pragma unroll
    for (int c = 0; c < NCH; c++) {
#pragma unroll
      for (int ht = 0; ht < NHT; ht++) {
        const char* vs = lds + (2 + PB) * TB + 32 * c * RBY + voff[ht];
        const s16x4_t r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vs));
        const s16x4_t r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vs + 16 * RBY));
        FragBF vf;
        vf.v = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int j = 0; j < J; j++) mma(o[j][ht], vf, pf[j][c]);
      }
#pragma unroll
      for (int j = 0; j < J; j++) mma(ls[j], ones, pf[j][c]);
    }
  };
  // this lane's maximum raw score of each row
  auto lanemax = [&](const f32x4_t (&s)[J][MT], float (&m)[J]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < J; j++) {
      float x[MT];
#pragma unroll
      for (int mt = 0; mt < MT; mt++) x[mt] = fmax3(s[j][mt][0], s[j][mt][1], __builtin_fmaxf(s[j][mt][2], s[j][mt][3]));
      float y = x[0];
#pragma unroll
      for (int mt = 1; mt + 1 < MT; mt += 2) y = fmax3(y, x[mt], x[mt + 1]);
      m[j] = MT % 2 == 0 ? __builtin_fmaxf(y, x[MT - 1]) : y;
    }
  };
  // move the reference past the margin: only when some lane of the wave
  // holds a score above its row's threshold does the wave take the row
  // maxima over the four lane groups (a row's first keys always move it:
  // the threshold starts at -inf)
  auto rescale = [&](const float (&m)[J]) __attribute__((always_inline)) {
    bool need = false;
#pragma unroll
    for (int j = 0; j < J; j++) need |= m[j] > thr[j];
    if (__ballot(need)) {
#pragma unroll
      for (int j = 0; j < J; j++) {
        const float tmax = pair_max32(pair_max16(m[j])) * c2;
        const bool move = tmax > mrow[j] + ATTN_RESCALE_LOG2;
        const float alpha = move ? __builtin_amdgcn_exp2f(mrow[j] - tmax) : 1.f;
        mrow[j] = move ? tmax : mrow[j];
        mneg[j] = mrow[j] == -INFINITY ? 0.f : -mrow[j];
        thr[j] = (mrow[j] + ATTN_RESCALE_LOG2) * inv_c2;
        ls[j] *= alpha;
#pragma unroll
        for (int u = 0; u < NHT; u++) o[j][u] *= alpha;
      }
    }
  };
  // instruction interleaving of the two phases (sched_group_barrier masks:
  // 0x008 MFMA, 0x100 LDS read, 0x402 VALU or transcendental)
  auto interleave_a = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < MT * NSS; i++) {
      __builtin_amdgcn_sched_group_barrier(0x008, J, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, 2 * J + 1, 0);
    }
  };
  auto interleave_b = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NCH * NHT; i++) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      __builtin_amdgcn_sched_group_barrier(0x008, J, 1);
      __builtin_amdgcn_sched_group_barrier(0x402, 1, 1);
    }
  };

  const int ntile = kend > kbeg ? (kend - kbeg + KT - 1) / KT : 0;
  auto full = [&](int k0) __attribute__((always_inline)) { return k0 + KT <= kend && k0 + KT - 1 <= qlim_all; };
  // Step tl (PB = tl & 1): scores of tile tl (CUR) and the probabilities and
  // P V product of tile tl - 1 (PREV).  K(tl) sits in K buffer PB and V(tl-1)
  // in V buffer PB ^ 1; after the barrier (every wave is done with step
  // tl - 1) the step loads K(tl+1) into K buffer PB ^ 1 and V(tl) into V
  // buffer PB, which both land before the next step's wait.
  auto step = [&](auto pbc, auto curc, auto prevc, int tl) __attribute__((always_inline)) {
    constexpr int PB = decltype(pbc)::value;
    constexpr bool CUR = decltype(curc)::value, PREV = decltype(prevc)::value;
    f32x4_t(&sc)[J][MT] = PB ? sb : sa;
    f32x4_t(&sp)[J][MT] = PB ? sa : sb;
    wait_vmcnt<0>();
    __syncthreads();
    const int k0 = kbeg + tl * KT;
    if (CUR) {
      if (tl + 1 < ntile) issue(std::integral_constant<int, 0>(), std::integral_constant<int, PB ^ 1>(), k0 + KT);
      issue(std::integral_constant<int, 1>(), std::integral_constant<int, PB>(), k0);
    }
    // phase A: S(t) on the matrix cores, the probabilities of t-1 on the
    // vector units (one basic block, interleaved)
    FragBF pf[J][NCH];
    if (PREV) probs(sp, pf);
    if (CUR) scores(pbc, sc);
    if (PREV && CUR) {
      // the probabilities are only used after the mask branch: an empty
      // statement that reads them keeps their computation in this block, so
      // that it overlaps the score MFMAs (it defines nothing, so the wait
      // states before the MFMAs that read them still follow the conversions)
#pragma unroll
      for (int j = 0; j < J; j++)
#pragma unroll
        for (int c = 0; c < NCH; c++) asm volatile("" ::"v"(pf[j][c].v));
      interleave_a();
    }
    if (CUR && !full(k0)) mask(sc, k0);
    // phase B: P(t-1) V(t-1) and the row sums on the matrix cores, the row
    // maxima of S(t) on the vector units
    float m[J];
    if (PREV) pv(std::integral_constant<int, PB ^ 1>(), pf);
    if (CUR) lanemax(sc, m);
    if (PREV && CUR) interleave_b();
    if (CUR) rescale(m);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using BT = std::integral_constant<bool, true>;
  using BF = std::integral_constant<bool, false>;
  if (ntile > 0) {
    issue(I0(), I0(), kbeg);
    step(I0(), BT(), BF(), 0);
    int tl = 1;
    for (; tl + 1 < ntile; tl += 2) {
      step(I1(), BT(), BT(), tl);
      step(I0(), BT(), BT(), tl + 1);
    }
    if (tl < ntile) {
      step(I1(), BT(), BT(), tl);
      step(I0(), BF(), BT(), tl + 1);
    } else {
      step(I1(), BF(), BT(), tl);
    }
  }

#pragma unroll
  for (int j = 0; j < J; j++) {
    // ls[j]: row 4 g4 + i of the column-sum product, i.e. query l16's sum in every element
    const float l = ls[j][0];
    const size_t row = (size_t)b * a.T + qi[j];
    if (!qv[j]) {
      // rows past the request's queries are not stored
    } else if (a.nsplit == 1) {
      const float inv = 1.f / l;
      uint16_t* out = (uint16_t*)a.out + row * (a.Hq * HD) + head[j] * HD + 4 * g4;
#pragma unroll
      for (int ht = 0; ht < NHT; ht++)
        *reinterpret_cast<uint2*>(out + 16 * ht) =
            make_uint2(f2bf2(o[j][ht][0] * inv, o[j][ht][1] * inv), f2bf2(o[j][ht][2] * inv, o[j][ht][3] * inv));
    } else {
      // key splits: unnormalised partials (O rounded to bf16, m, l in fp32),
      // merged by attn_merge_k
      const size_t e = split * (size_t)a.rows * a.Hq + row * a.Hq + head[j];
      uint16_t* po = static_cast<uint16_t*>(a.po) + e * HD + 4 * g4;
#pragma unroll
      for (int ht = 0; ht < NHT; ht++)
        *reinterpret_cast<uint2*>(po + 16 * ht) =
            make_uint2(f2bf2(o[j][ht][0], o[j][ht][1]), f2bf2(o[j][ht][2], o[j][ht][3]));
      if (g4 == 0) {
        a.pml[2 * e] = mrow[j];
        a.pml[2 * e + 1] = l;
      }
    }
  }
}

// combine key splits in split order: o = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// A thread owns 4 consecutive head-dimension elements of one (row, head)
// entry and has the loads of every split in flight at once (the merge is a
// short latency chain over 2 + nsplit loads).  The partial O_s are fp32 (fp32
// attention) or bf16 (bf16 attention: half the partial traffic; the rounding
// is one more bf16 step before the output's own, on a weighted average).
constexpr int ATTN_MAX_SPLIT = 16;
template <typename T> struct TypeTag { using type = T; };
__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4(const uint16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}
template <typename TA, int HD, int NS>
__global__ __launch_bounds__(256) void attn_merge_k(const TA* __restrict__ po,
                                                    const float* __restrict__ pml, int nsplit,
                                                    int entries, TA* __restrict__ out) {
  constexpr int TPE = HD / 4;   // threads per entry
  const int gt = blockIdx.x * 256 + threadIdx.x;
  const int e = gt / TPE, d0 = (gt % TPE) * 4;
  if (e >= entries) return;
  // NS >= nsplit: the loads of all splits at once (splits past nsplit re-read
  // split 0 and weigh nothing)
  float m[NS], l[NS];
  float4 v[NS];
#pragma unroll
  for (int j = 0; j < NS; j++) {
    const size_t ee = (size_t)(j < nsplit ? j : 0) * entries + e;
    m[j] = pml[2 * ee];
    l[j] = pml[2 * ee + 1];
    v[j] = load4(po + ee * HD + d0);
  }
  float M = -INFINITY;
#pragma unroll
  for (int j = 0; j < NS; j++) M = j < nsplit ? fmaxf(M, m[j]) : M;
  float den = 0.f, num[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NS; j++) {
    const float f = (j < nsplit && m[j] != -INFINITY) ? __builtin_amdgcn_exp2f(m[j] - M) : 0.f;
    den += f * l[j];
    num[0] += f * v[j].x;
    num[1] += f * v[j].y;
    num[2] += f * v[j].z;
    num[3] += f * v[j].w;
  }
  const float inv = 1.f / den;
  if constexpr (sizeof(TA) == 2)
    *reinterpret_cast<uint2*>(out + (size_t)e * HD + d0) =
        make_uint2(f2bf2(num[0] * inv, num[1] * inv), f2bf2(num[2] * inv, num[3] * inv));
  else
    *reinterpret_cast<float4*>(out + (size_t)e * HD + d0) =
        make_float4(num[0] * inv, num[1] * inv, num[2] * inv, num[3] * inv);
}

// ---------------------------------------------------------------------------
// key splits: enough blocks to fill the chip several times over (each block
// is a short latency chain), at least ATTN_MIN_SPLIT_KEYS keys per split
// About 512 blocks when requests hold many keys.  With few keys (up to 2048
// per request) 256: more splits then add partial traffic and merge work that
// outweigh the parallelism.  Measured for attention + merge: 20.8 against
// 23.9 us at 1280 keys; 256 blocks were slower at 2304 keys (batch 8: 89
// against 71 us) and at 8448 (47 against 42).
constexpr int ATTN_TARGET_BLOCKS = 512;
constexpr int ATTN_TARGET_BLOCKS_FEW_KEYS = 256;
constexpr int ATTN_FEW_KEYS = 2048;
constexpr int ATTN_MIN_SPLIT_KEYS = 128;
constexpr long ATTN_MAX_PART_ENTRIES = 1L << 18;

long attn_partial_entries(int rows, int Hq, int max_keys) {
  // bounded split buffer: at most 2^18 (row, head) entries across all splits;
  // no more splits than the key count allows (max_keys 0: not known)
  int splits = ATTN_MAX_SPLIT;
  if (max_keys > 0) {
    const int by_keys = (max_keys + ATTN_MIN_SPLIT_KEYS - 1) / ATTN_MIN_SPLIT_KEYS;
    splits = by_keys < splits ? by_keys : splits;
  }
  if (splits <= 1) return 0;
  const long full = (long)rows * Hq * splits;
  return full < ATTN_MAX_PART_ENTRIES ? full : ATTN_MAX_PART_ENTRIES;
}

struct AttnPlan {
  int G, QT, nqt, nsplit, split_len, groups;
  unsigned grid;
};

// bf16 kernel: 4 waves x 32 rows, K and V tiles of 32 keys in two buffers
// each (32 KB of LDS at hd 128, two blocks per CU)
constexpr int ATTN_ROWS = 128;   // (query, head) rows per bf16 attention block
constexpr int ATTN_KT = 32;   // keys per pipeline step of the bf16 kernel

// rows per block: 32 per wave for the bf16 kernel, 64 for the fp32 kernel
// (4 waves x 16 rows)
int attn_block_rows(int act) { return act == ACT_BF16 ? ATTN_ROWS : 64; }

AttnPlan plan_attention(int act, int B, int T, const Lens& len, int Hq, int Hkv, long part_cap) {
  AttnPlan p{};
  p.G = Hq / Hkv;
  p.QT = attn_block_rows(act) / p.G;
  int maxkeys = 0;
  for (int b = 0; b < B; b++) maxkeys = maxkeys > len.v[b] + T ? maxkeys : len.v[b] + T;
  p.nqt = (T + p.QT - 1) / p.QT;
  const long base = (long)p.nqt * B * Hkv;
  int nsplit = 1;
  const int target = maxkeys <= ATTN_FEW_KEYS ? ATTN_TARGET_BLOCKS_FEW_KEYS : ATTN_TARGET_BLOCKS;
  if (base < target) {
    nsplit = (int)((target + base - 1) / base);
    const int by_keys = (maxkeys + ATTN_MIN_SPLIT_KEYS - 1) / ATTN_MIN_SPLIT_KEYS;
    if (nsplit > by_keys) nsplit = by_keys;
    if (nsplit > ATTN_MAX_SPLIT) nsplit = ATTN_MAX_SPLIT;
    const long entries = (long)B * T * Hq;
    while (nsplit > 1 && entries * nsplit > part_cap) nsplit--;
    if (nsplit < 1) nsplit = 1;
  }
  int split_len = (maxkeys + nsplit - 1) / nsplit;
  split_len = (split_len + KT - 1) / KT * KT;
  nsplit = (maxkeys + split_len - 1) / split_len;
  if (nsplit < 1) nsplit = 1;
  p.split_len = split_len;
  p.nsplit = nsplit;
  p.groups = B * Hkv * nsplit;
  p.grid = (unsigned)(((p.groups + 7) / 8) * 8 * p.nqt);
  return p;
}

void launch_attention(const AttnArgsHost& h, hipStream_t s) {
  const AttnPlan p = plan_attention(h.act, h.B, h.T, h.len, h.Hq, h.Hkv, h.part_cap);
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
  a.G = p.G;
  a.QT = p.QT;
  a.mode = h.mode;
  a.len = h.len;
  a.scale_log2 = 1.4426950408889634f / sqrtf((float)h.hd);
  a.out = h.out;
  a.po = h.po;
  a.pml = h.pml;
  a.rows = h.B * h.T;
  a.split_len = p.split_len;
  a.nsplit = p.nsplit;
  a.nqt = p.nqt;
  a.groups = p.groups;
  const dim3 grid(p.grid);
  if (h.act == ACT_BF16) {
    // 4 waves of two 16-row tiles (each K and V fragment read from LDS
    // serves both tiles)
    static_assert(16 * 2 * 4 == ATTN_ROWS, "block rows");
    if (h.hd == 128) attn_bf16_k<128, 4, ATTN_KT, 2><<<grid, 4 * 64, 0, s>>>(a);
    else attn_bf16_k<64, 4, ATTN_KT, 2><<<grid, 4 * 64, 0, s>>>(a);
  } else {
    if (h.hd == 128) attn_k<float, 128><<<grid, 256, 0, s>>>(a);
    else attn_k<float, 64><<<grid, 256, 0, s>>>(a);
  }
  if (p.nsplit > 1) {
    const int entries = a.rows * h.Hq;
    const int blocks = (int)(((long)entries * (h.hd / 4) + 255) / 256);
    auto merge = [&](auto tac, auto nsc) {
      using TA = typename decltype(tac)::type;
      constexpr int NS = decltype(nsc)::value;
      const TA* po = static_cast<const TA*>(h.po);   // partials of the attention's own type
      if (h.hd == 128) attn_merge_k<TA, 128, NS><<<blocks, 256, 0, s>>>(po, h.pml, p.nsplit, entries, (TA*)h.out);
      else attn_merge_k<TA, 64, NS><<<blocks, 256, 0, s>>>(po, h.pml, p.nsplit, entries, (TA*)h.out);
    };
    auto by_splits = [&](auto tac) {
      if (p.nsplit <= 4) merge(tac, std::integral_constant<int, 4>());
      else if (p.nsplit <= 8) merge(tac, std::integral_constant<int, 8>());
      else merge(tac, std::integral_constant<int, ATTN_MAX_SPLIT>());
    };
    if (h.act == ACT_BF16) by_splits(TypeTag<uint16_t>());
    else by_splits(TypeTag<float>());
  }
}

// Host replica of every K/V address the attention kernels issue for one
// launch (the plan, the block decode and the key index of each staged slot,
// with each kernel's tile schedule: the bf16 kernel loads tiles 0 ..
// ntile-1 only; the fp32 kernel loads tiles 0, 1, 2 in its prologue, then tile
// i+3 while tile i is computed, so it stages tiles past the split end).
// Returns the number of addressed keys that are not keys of the block's own
// request: in mode 0 a cache row must lie in [0, len[b]) and a canvas row in
// [0, T); in mode 1 a cache row in [0, len[b] + T) (the new keys are written
// before the attention runs).  Also counts a launch whose partials would
// overflow part_cap.
long attn_check_addresses(int act, int B, int T, const Lens& len, int Hq, int Hkv, int mode,
                          long part_cap, long* nslots) {
  const AttnPlan p = plan_attention(act, B, T, len, Hq, Hkv, part_cap);
  long bad = 0, n = 0;
  if (p.nsplit > 1 && (long)B * T * Hq * p.nsplit > part_cap) bad++;
  for (unsigned id = 0; id < p.grid; id++) {
    int b, gh, split, qt;
    if (!attn_block((int)id, p.nqt, p.groups, p.nsplit, Hkv, b, gh, split, qt)) continue;
    const int P = len.v[b];
    const int nkeys = mode == 0 ? P + T : P + (((qt + 1) * p.QT) < T ? (qt + 1) * p.QT : T);
    const int kbeg = split * p.split_len;
    const int kend = nkeys < kbeg + p.split_len ? nkeys : kbeg + p.split_len;
    // the bf16 kernel loads exactly its ntile tiles of ATTN_KT keys; the
    // fp32 kernel stages 64-key tiles up to two ahead of the last one used
    const int kt = act == ACT_BF16 ? ATTN_KT : KT;
    const int ntile = kend > kbeg ? (kend - kbeg + kt - 1) / kt : 0;
    int last = ntile - 1;
    if (act != ACT_BF16) {
      last = 2;
      for (int it = 0; it + 2 <= ntile; it += 2) last = it + 1 + 3 > last ? it + 1 + 3 : last;
    }
    for (int tl = 0; tl <= last; tl++)
      for (int j = 0; j < kt; j++) {
        const int k = attn_key_index(kbeg + tl * kt + j, kbeg, kend);
        n++;
        bad += !(k >= 0 && k < P + T);
      }
  }
  if (nslots) *nslots = n;
  return bad;
}

}  // namespace dg

extern "C" long dg_check_attention_addresses(int act_dtype, int B, int T, const int32_t* lens, int Hq,
                                             int Hkv, int mode, long part_cap, long* nslots) {
  dg::Lens l{};
  if (B < 1 || B > DG_MAX_BATCH || T < 1 || Hkv < 1 || Hq % Hkv) return -1;
  if (act_dtype != DG_F32 && act_dtype != DG_BF16) return -1;
  for (int b = 0; b < B; b++) l.v[b] = lens[b];
  return dg::attn_check_addresses(act_dtype == DG_BF16 ? dg::ACT_BF16 : dg::ACT_F32, B, T, l, Hq,
                                  Hkv, mode, part_cap, nslots);
}
