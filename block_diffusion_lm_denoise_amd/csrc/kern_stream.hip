// kern_stream.hip -- weight-streaming MFMA GEMM for few rows against large
// weight matrices: the grouped expert GEMMs of a pass, the dense projections
// and the LM head.
//
// One block = (row tile of at most 32 rows, chunk of 64 weight rows).  The
// four waves split the contraction in 64-element pieces (wave w takes pieces
// w, w+4, ...), load MFMA fragments of A and W straight from memory with a
// register double buffer (the next piece is in flight while the current one
// is multiplied), and reduce their partial tiles through LDS one 16-row tile
// at a time.  Each weight byte is used by the row tiles of its rows only.
//
// Block ids run chunk-fastest (id = chunk + C * tile): blocks of one row tile
// are consecutive, and the row tiles that share a weight chunk are C ids
// apart.  With C a multiple of 8 they are dispatched to the same XCD (blocks
// go round-robin over the 8 XCDs), so a weight chunk read by several row
// tiles is served from that XCD's L2 after the first read.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace dg {

template <typename TA, typename TW>
__device__ __forceinline__ void load_w(typename FragOf<TA>::type& f, const TW* p);
template <>
__device__ __forceinline__ void load_w<uint16_t, uint16_t>(FragBF& f, const uint16_t* p) {
  load_frag(f, p);
}
template <>
__device__ __forceinline__ void load_w<uint16_t, uint8_t>(FragBF& f, const uint8_t* p) {
  load_frag_fp8(f, p);
}
template <>
__device__ __forceinline__ void load_w<float, float>(FragF32& f, const float* p) {
  load_frag(f, p);
}

__device__ __forceinline__ void mrg3(float& m, int& i, float& s, float m2, int i2, float s2) {
  if (m2 == -INFINITY) return;
  if (m2 > m || (m2 == m && i2 < i)) {
    s = s * __expf(m - m2) + s2;
    m = m2;
    i = i2;
  } else {
    s = s + s2 * __expf(m2 - m);
  }
}

// KW waves split the contraction; the 4/KW wave groups take different 64-row
// weight column groups (a block covers 64 * 4/KW weight rows).
template <typename TA, typename TW, int MODE, int KW>
__global__ __launch_bounds__(256) void wstream_k(StreamGemm a) {
  typedef typename FragOf<TA>::type Frag;
  constexpr int CWG = 4 / KW;          // column groups per block
  __shared__ float red[4][4][64][4];   // [wave][col tile][lane][i], one 16-row tile at a time
  __shared__ float hm[4][16], hs[4][16];
  __shared__ int hi[4][16];
  constexpr bool GROUPED = MODE == SG_GATEUP || MODE == SG_DOWN;
  const int C = a.nchunks;
  const int chunk = blockIdx.x % C, tile = blockIdx.x / C;
  int e = 0, row0, nrows;
  if (GROUPED) {
    if (tile >= *a.ntiles) return;
    const int4 t = a.tiles[tile];
    e = t.x;
    row0 = t.y;
    nrows = t.z;
  } else {
    row0 = tile * 32;
    if (row0 >= a.M) return;
    nrows = min(32, a.M - row0);
  }
  const int nrt = (nrows + 15) >> 4;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l16 = lane & 15, g = lane >> 4;
  const int kw = w % KW, cg = w / KW;  // contraction share, column group of this wave
  const int K = a.K;

  // A row pointers of this lane (row l16 of each 16-row tile).  Rows past the
  // tile read a valid row and are zeroed by a select, so the load path has no
  // branches and the next piece's loads stay in flight during the MFMAs.
  const TA* arow[2];
  bool aok[2];
#pragma unroll
  for (int rt = 0; rt < 2; rt++) {
    const int r = rt * 16 + l16;
    aok[rt] = r < nrows;
    const int slot = row0 + (aok[rt] ? r : 0);
    const size_t src = MODE == SG_GATEUP ? (size_t)(a.perm[slot] / a.k) : (size_t)slot;
    arow[rt] = (const TA*)a.A + src * K;
  }
  // W row pointers of this lane (row l16 of each 16-row column tile)
  const TW* wrow[4];
  bool wok[4];
  const int n0 = (chunk * CWG + cg) * 64;   // first weight row (dense/down) of this wave
#pragma unroll
  for (int ct = 0; ct < 4; ct++) {
    const TW* p;
    bool ok = true;
    if (MODE == SG_GATEUP) {
      // 32 SwiGLU outputs per column group: tiles [gate f, up f, gate f+16, up f+16]
      const int f = (chunk * CWG + cg) * 32 + 16 * (ct >> 1) + l16;
      p = (const TW*)((ct & 1) ? a.W1 : a.W0) + ((size_t)e * a.NW + f) * K;
    } else if (MODE == SG_DOWN) {
      p = (const TW*)a.W0 + ((size_t)e * a.NW + n0 + 16 * ct + l16) * K;
    } else {
      const int n = n0 + 16 * ct + l16;
      ok = n < a.N;
      const int nn = ok ? n : 0;
      if (nn < a.n1) p = (const TW*)a.W0 + (size_t)nn * K;
      else if (nn < a.n1 + a.n2) p = (const TW*)a.W1 + (size_t)(nn - a.n1) * K;
      else p = (const TW*)a.W2 + (size_t)(nn - a.n1 - a.n2) * K;
    }
    wrow[ct] = p;
    wok[ct] = ok;
  }

  f32x4_t acc[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; rt++)
#pragma unroll
    for (int ct = 0; ct < 4; ct++) acc[rt][ct] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  Frag wa[4][2], aa[2][2], wb[4][2], ab[2][2];
  auto load = [&](Frag(&wf)[4][2], Frag(&af)[2][2], int ch) {
#pragma unroll
    for (int s = 0; s < 2; s++) {
      const int kk = ch * 64 + 32 * s + 8 * g;
#pragma unroll
      for (int ct = 0; ct < 4; ct++) load_w<TA, TW>(wf[ct][s], wrow[ct] + kk);
#pragma unroll
      for (int rt = 0; rt < 2; rt++) load_frag(af[rt][s], arow[rt] + kk);
    }
  };
  // ok = false: the piece is past the contraction (clamped load), zero its A
  auto comp = [&](Frag(&wf)[4][2], Frag(&af)[2][2], bool ok) {
#pragma unroll
    for (int s = 0; s < 2; s++) {
#pragma unroll
      for (int ct = 0; ct < 4; ct++) mask_frag(wf[ct][s], wok[ct]);
#pragma unroll
      for (int rt = 0; rt < 2; rt++) mask_frag(af[rt][s], aok[rt] && ok);
#pragma unroll
      for (int rt = 0; rt < 2; rt++)
#pragma unroll
        for (int ct = 0; ct < 4; ct++) mma(acc[rt][ct], af[rt][s], wf[ct][s]);
    }
  };

  // wave takes pieces kw, kw+KW, ...; two register buffers, straight-line
  // code (indices past the end are clamped and masked) so that the waits
  // before each MFMA group cover only the older buffer's loads
  const int nch = K / 64;
  const int per = (nch + KW - 1) / KW;
  const int npairs = (per + 1) / 2;
  auto cidx = [&](int i) { const int c = kw + KW * i; return c < nch ? c : nch - 1; };
  auto cok = [&](int i) { return kw + KW * i < nch; };
  // sched_barrier pins each buffer's loads ahead of the other buffer's MFMAs
  // (otherwise the scheduler sinks them to save registers)
  load(wa, aa, cidx(0));
  int pi = 0;
  for (; pi + 1 < npairs; pi++) {
    load(wb, ab, cidx(2 * pi + 1));
    __builtin_amdgcn_sched_barrier(0);
    comp(wa, aa, cok(2 * pi));
    __builtin_amdgcn_sched_barrier(0);
    load(wa, aa, cidx(2 * pi + 2));
    __builtin_amdgcn_sched_barrier(0);
    comp(wb, ab, cok(2 * pi + 1));
    __builtin_amdgcn_sched_barrier(0);
  }
  load(wb, ab, cidx(2 * pi + 1));
  __builtin_amdgcn_sched_barrier(0);
  comp(wa, aa, cok(2 * pi));
  __builtin_amdgcn_sched_barrier(0);
  comp(wb, ab, cok(2 * pi + 1));

  // ---- reduce the four waves' partial tiles, one 16-row tile at a time ----
  float sg = 1.f, su = 1.f, sd = 1.f;
  if (GROUPED && a.escale) {
    sg = a.escale[e * 3 + 0];
    su = a.escale[e * 3 + 1];
    sd = a.escale[e * 3 + 2];
  }
  for (int rt = 0; rt < nrt; rt++) {
#pragma unroll
    for (int ct = 0; ct < 4; ct++)
#pragma unroll
      for (int i = 0; i < 4; i++) red[w][ct][lane][i] = acc[rt][ct][i];
    __syncthreads();
    // thread (q = wave index, lane) takes column tile q of column group cq
    // (KW == 4: the block's 4 tiles; KW == 2: tiles q of both groups, below)
    const int q = w;
    auto sumk = [&](int grp, int tile, int i) {
      float v = 0.f;
#pragma unroll
      for (int j = 0; j < KW; j++) v += red[grp * KW + j][tile][lane][i];
      return v;
    };
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; i++) v[i] = sumk(0, q, i);
    if (MODE == SG_GATEUP) {
      // thread q < 2*CWG owns SwiGLU pair (group q/2, gate tile 2*(q%2), up tile 2*(q%2)+1)
      if (q < 2 * CWG) {
        const int grp = q >> 1, pp = q & 1;
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const float gv = sumk(grp, 2 * pp, i) * sg;
          const float uv = sumk(grp, 2 * pp + 1, i) * su;
          const int r = rt * 16 + 4 * g + i;
          if (r < nrows)
            stx((TA*)a.out, (size_t)(row0 + r) * a.ldo + (chunk * CWG + grp) * 32 + 16 * pp + l16,
                gv / (1.f + expf(-gv)) * uv);
        }
      }
    } else if (MODE == SG_LMHEAD) {
      static_assert(MODE != SG_LMHEAD || KW == 4, "the head epilogue reduces one 64-column group");
      // per row: (max, lowest index attaining it, sum exp(l - max)) over the 64 columns
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int r = rt * 16 + 4 * g + i;
        const int n = n0 + 16 * q + l16;
        const float val = n < a.N ? v[i] : -INFINITY;
        if (a.logits && r < nrows && n < a.N) a.logits[(size_t)(row0 + r) * a.N + n] = val;
        float m = -INFINITY, s = 0.f;
        int idx = 0x7fffffff;
        mrg3(m, idx, s, val, n, 1.f);
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
          const int i2 = __shfl_xor(idx, o, 64);
          mrg3(m, idx, s, m2, i2, s2);
        }
        if (l16 == 0) {
          hm[q][4 * g + i] = m;
          hs[q][4 * g + i] = s;
          hi[q][4 * g + i] = idx;
        }
      }
      __syncthreads();
      if (threadIdx.x < 16) {
        const int rr = threadIdx.x;
        float m = hm[0][rr], s = hs[0][rr];
        int idx = hi[0][rr];
        for (int qq = 1; qq < 4; qq++) mrg3(m, idx, s, hm[qq][rr], hi[qq][rr], hs[qq][rr]);
        const int r = rt * 16 + rr;
        if (r < nrows) {
          const size_t o = (size_t)(row0 + r) * C + chunk;
          a.pmax[o] = m;
          a.pidx[o] = idx;
          a.psum[o] = s;
        }
      }
    } else {
#pragma unroll
      for (int grp = 0; grp < CWG; grp++) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int r = rt * 16 + 4 * g + i;
          const int n = (chunk * CWG + grp) * 64 + 16 * q + l16;
          if (r >= nrows || n >= a.N) continue;
          const size_t row = (size_t)(row0 + r);
          const size_t o = row * a.ldo + n;
          float val = grp == 0 ? v[i] : sumk(grp, q, i);
          if (MODE == SG_DOWN) {
            stx((TA*)a.out, o, val * sd);
          } else if (MODE == SG_F32) {
            ((float*)a.out)[o] = val;
          } else {
            if (MODE == SG_RESID) val += ldx((const TA*)a.R, o);
            stx((TA*)a.out, o, val);
            if (MODE == SG_QKV_CACHE && n >= a.cache.QD) {
              const int c = n - a.cache.QD;
              const bool isv = c >= a.cache.KD;
              const int cc = isv ? c - a.cache.KD : c;
              const int gh = cc / a.cache.hd, d = cc % a.cache.hd;
              const int b = (int)(row / a.cache.T), t = (int)(row % a.cache.T);
              const size_t co = (((size_t)b * a.cache.Hkv + gh) * a.cache.cap + a.cache.len.v[b] + t) *
                                    a.cache.hd + d;
              stx((TA*)(isv ? a.cache.v : a.cache.k), co, val);
            }
          }
        }
      }
    }
    __syncthreads();
  }
}

template <int MODE, int KW>
static void dispatch(int act, int wdt, const StreamGemm& a, int nblocks, hipStream_t s) {
  if (nblocks <= 0) return;
  if (act == ACT_F32)
    wstream_k<float, float, MODE, KW><<<nblocks, 256, 0, s>>>(a);
  else if (wdt == DG_FP8E4M3)
    wstream_k<uint16_t, uint8_t, MODE, KW><<<nblocks, 256, 0, s>>>(a);
  else
    wstream_k<uint16_t, uint16_t, MODE, KW><<<nblocks, 256, 0, s>>>(a);
}

// kw: waves splitting the contraction (4, or 2 when the block should cover 128
// weight rows, e.g. a short contraction); a.nchunks counts blocks per row tile
void launch_stream_gemm(int act, int wdt, int mode, int kw, const StreamGemm& a, int ntiles_max,
                        hipStream_t s) {
  const int nb = a.nchunks * ntiles_max;
  if (kw == 2) {
    switch (mode) {
      case SG_STORE: dispatch<SG_STORE, 2>(act, wdt, a, nb, s); break;
      case SG_RESID: dispatch<SG_RESID, 2>(act, wdt, a, nb, s); break;
      case SG_F32: dispatch<SG_F32, 2>(act, wdt, a, nb, s); break;
      case SG_QKV_CACHE: dispatch<SG_QKV_CACHE, 2>(act, wdt, a, nb, s); break;
      case SG_GATEUP: dispatch<SG_GATEUP, 2>(act, wdt, a, nb, s); break;
      case SG_DOWN: dispatch<SG_DOWN, 2>(act, wdt, a, nb, s); break;
      default: break;
    }
    return;
  }
  switch (mode) {
    case SG_STORE: dispatch<SG_STORE, 4>(act, wdt, a, nb, s); break;
    case SG_RESID: dispatch<SG_RESID, 4>(act, wdt, a, nb, s); break;
    case SG_F32: dispatch<SG_F32, 4>(act, wdt, a, nb, s); break;
    case SG_QKV_CACHE: dispatch<SG_QKV_CACHE, 4>(act, wdt, a, nb, s); break;
    case SG_GATEUP: dispatch<SG_GATEUP, 4>(act, wdt, a, nb, s); break;
    case SG_DOWN: dispatch<SG_DOWN, 4>(act, wdt, a, nb, s); break;
    case SG_LMHEAD: dispatch<SG_LMHEAD, 4>(act, wdt, a, nb, s); break;
  }
}

}  // namespace dg
