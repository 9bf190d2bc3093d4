// kern_stream.hip -- weight-streaming MFMA GEMM for few rows against large
// weight matrices: the grouped expert GEMMs of a pass and the dense
// projections.
//
// One block = (row tile of at most 32 rows, chunk of 64 weight rows).  The
// four waves split the contraction in pieces of 128 bytes per weight row
// (wave w takes pieces w, w+4, ...), load the weights from the packed layout
// (every wave load is 1 KB of contiguous memory: whole cache lines) and the
// activation fragments straight from memory, with a register double buffer
// (the next piece is in flight while the current one is multiplied), and
// reduce their partial tiles through LDS one 16-row tile at a time.  Each
// weight byte is used by the row tiles of its rows only.
//
// Block ids run chunk-fastest (id = chunk + C * tile): blocks of one row tile
// are consecutive, and the row tiles that share a weight chunk are C ids
// apart.  With C a multiple of 8 they are dispatched to the same XCD (blocks
// go round-robin over the 8 XCDs), so a weight chunk read by several row
// tiles is served from that XCD's L2 after the first read.  The down
// projection instead keeps each row tile on one XCD (its activation rows,
// just written by the gate/up launch, are then fetched into one L2).
#include <math.h>

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace dg {

// A piece is one 128-byte column block of the packed weights (16 rows x 128
// bytes, two 1 KB wave loads h = 0, 1; lane l gets row l%16, bytes
// 64h + 16(l/16)): 64 bf16, 128 fp8 or 32 fp32 contraction elements.  The
// activation fragments take the same elements in the same lane order, which
// is a consistent permutation of the contraction inside the piece.
template <typename TA, typename TW> struct Piece;
template <> struct Piece<uint16_t, uint16_t> {
  static constexpr int EP = 64, NA = 2;   // elements per piece, 16-byte A loads per row tile
  static __device__ __forceinline__ int a_off(int j, int g) { return 32 * j + 8 * g; }
};
template <> struct Piece<uint16_t, uint8_t> {
  static constexpr int EP = 128, NA = 4;
  static __device__ __forceinline__ int a_off(int j, int g) { return 64 * (j >> 1) + 16 * g + 8 * (j & 1); }
};
template <> struct Piece<uint16_t, mxfp4_t> {
  // MXFP4 works on half pieces: one 1 KB wave load of 64 code bytes per row =
  // 128 elements; lane g's 16 bytes are the 32 elements 32 g .. +31 (one MX
  // block), four MFMA groups of 8
  static constexpr int EP = 128, NA = 4;
  static __device__ __forceinline__ int a_off(int j, int g) { return 32 * g + 8 * j; }
};
template <> struct Piece<float, float> {
  static constexpr int EP = 32, NA = 2;
  static __device__ __forceinline__ int a_off(int j, int g) { return 16 * j + 4 * g; }
};

__device__ __forceinline__ void zero_unless(u32x4& u, bool ok) {
  u.x = ok ? u.x : 0u;
  u.y = ok ? u.y : 0u;
  u.z = ok ? u.z : 0u;
  u.w = ok ? u.w : 0u;
}

// acc[rt][ct] += A[rt] . W[ct] over one piece, from raw 16-byte registers.
// Row tiles rt >= 2 are multiplied only when the tile has rows there (nrt is
// uniform over the wave, so the test is a scalar branch).
template <int RT>
__device__ __forceinline__ void piece_mma(f32x4_t (&acc)[RT][4], const u32x4 (&wr)[4][2],
                                          const u32x4 (&ar)[RT][2], int nrt, uint16_t*, uint16_t*) {
#pragma unroll
  for (int j = 0; j < 2; j++)
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
      if (rt < 2 || rt < nrt)
#pragma unroll
        for (int ct = 0; ct < 4; ct++) {
          FragBF x, y;
          x.v = __builtin_bit_cast(bf16x8_t, ar[rt][j]);
          y.v = __builtin_bit_cast(bf16x8_t, wr[ct][j]);
          mma(acc[rt][ct], x, y);
        }
}
template <int RT>
__device__ __forceinline__ void piece_mma(f32x4_t (&acc)[RT][4], const u32x4 (&wr)[4][2],
                                          const u32x4 (&ar)[RT][4], int nrt, uint16_t*, uint8_t*) {
#pragma unroll
  for (int j = 0; j < 4; j++)
#pragma unroll
    for (int ct = 0; ct < 4; ct++) {
      const u32x4 u = wr[ct][j >> 1];
      FragBF y;
      y.v = __builtin_bit_cast(bf16x8_t, fp8x8_to_bf16x8((j & 1) ? make_uint2(u.z, u.w) : make_uint2(u.x, u.y)));
#pragma unroll
      for (int rt = 0; rt < RT; rt++)
        if (rt < 2 || rt < nrt) {
          FragBF x;
          x.v = __builtin_bit_cast(bf16x8_t, ar[rt][j]);
          mma(acc[rt][ct], x, y);
        }
    }
}
// MXFP4: each 16-byte weight load is one MX block of 32 codes with its scale
// byte sr[ct][h]; its four 8-code words decode (scaled, exactly) into the
// bf16 operands of four MFMA groups
template <int RT>
__device__ __forceinline__ void piece_mma_mx(f32x4_t (&acc)[RT][4], const u32x4 (&wr)[4][2],
                                             const u32x4 (&ar)[RT][4], const uint32_t (&sr)[4][2],
                                             int nrt) {
#pragma unroll
  for (int ks = 0; ks < 4; ks++)
#pragma unroll
    for (int ct = 0; ct < 4; ct++) {
      FragBF y;
      y.v = __builtin_bit_cast(bf16x8_t, fp4x8_to_bf16x8(wr[ct][0][ks], e8m0_to_f32(sr[ct][0])));
#pragma unroll
      for (int rt = 0; rt < RT; rt++)
        if (rt < 2 || rt < nrt) {
          FragBF x;
          x.v = __builtin_bit_cast(bf16x8_t, ar[rt][ks]);
          mma(acc[rt][ct], x, y);
        }
    }
}
template <int RT>
__device__ __forceinline__ void piece_mma(f32x4_t (&acc)[RT][4], const u32x4 (&wr)[4][2],
                                          const u32x4 (&ar)[RT][2], int nrt, float*, float*) {
#pragma unroll
  for (int rt = 0; rt < RT; rt++)
    if (rt < 2 || rt < nrt)
#pragma unroll
    for (int ct = 0; ct < 4; ct++) {
      FragF32 x, y;
#pragma unroll
      for (int j = 0; j < 2; j++) {
        const u32x4 ua = ar[rt][j], uw = wr[ct][j];
        x.v[4 * j + 0] = __uint_as_float(ua.x);
        x.v[4 * j + 1] = __uint_as_float(ua.y);
        x.v[4 * j + 2] = __uint_as_float(ua.z);
        x.v[4 * j + 3] = __uint_as_float(ua.w);
        y.v[4 * j + 0] = __uint_as_float(uw.x);
        y.v[4 * j + 1] = __uint_as_float(uw.y);
        y.v[4 * j + 2] = __uint_as_float(uw.z);
        y.v[4 * j + 3] = __uint_as_float(uw.w);
      }
      mma(acc[rt][ct], x, y);
    }
}

// expert weights are read once per expert tile: nontemporal loads (streamed,
// not kept); the dense projections' weights are shared by several row tiles
// (and read again every pass), so they are loaded normally
constexpr int STREAM_NT_DENSE = 0;
constexpr int STREAM_NT = 1;

// KW waves split the contraction; the 4/KW wave groups take different 64-row
// weight column groups (a block covers 64 * 4/KW weight rows).  A row tile
// holds up to 16 RT rows: RT = 4 for the grouped bf16 expert GEMMs, so an
// expert with up to 64 routed rows reads its weights once.
template <typename TA, typename TW, int MODE, int KW, int NB, int RT>
__global__ __launch_bounds__(256, 2) void wstream_k(StreamGemm a) {
  typedef Piece<TA, TW> PC;
  constexpr int NA = PC::NA;
  constexpr bool MX = std::is_same<TW, mxfp4_t>::value;
  constexpr int CWG = 4 / KW;          // column groups per block
  __shared__ float red[4][4][64][4];   // [wave][col tile][lane][i], one 16-row tile at a time
  constexpr bool GROUPED = MODE == SG_GATEUP || MODE == SG_DOWN;
  const int C = a.nchunks;
  // down projection: tile-major over the XCDs (blocks go round-robin over
  // the 8 XCDs, id % 8): the C column chunks of an expert tile run on one
  // XCD, so the tile's SwiGLU rows come into one L2 once (1024 prefix: pass
  // 301.6 -> 299.4 us).  Other modes: chunk-fastest (below).
  constexpr bool TILE_XCD = MODE == SG_DOWN;
  const int chunk = TILE_XCD ? (int)(blockIdx.x >> 3) % C : (int)blockIdx.x % C;
  int tile = TILE_XCD ? ((int)(blockIdx.x >> 3) / C) * 8 + (int)(blockIdx.x & 7) : (int)blockIdx.x / C;
  int split = 0;
  if (MODE == SG_F32 && a.ksplit > 1) {   // block id = chunk + C * (tile + T * split)
    const int T = (a.M + 16 * RT - 1) / (16 * RT);
    split = tile / T;
    tile -= split * T;
  }
  int e = 0, row0, nrows;
  if (GROUPED) {
    if (tile >= *a.ntiles) return;
    const int4 t = a.tiles[tile];
    e = t.x;
    row0 = t.y;
    nrows = t.z;
  } else {
    row0 = tile * 16 * RT;
    if (row0 >= a.M) return;
    nrows = min(16 * RT, a.M - row0);
  }
  const int nrt = (nrows + 15) >> 4;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l16 = lane & 15, g = lane >> 4;
  const int kw = w % KW, cg = w / KW;  // contraction share, column group of this wave
  const int K = a.K;
  const int nch_all = K / PC::EP;      // pieces (packed column blocks; MXFP4: halves) per weight row
  // bytes from one 16-row group of the packed weights to the next
  const size_t rg_bytes = (size_t)(MX ? K / 256 : nch_all) * 2048;
  // contraction split: this block takes pieces [pbeg, pbeg + nch)
  const int nsp = MODE == SG_F32 && a.ksplit > 1 ? a.ksplit : 1;
  const int nch = nch_all / nsp, pbeg = split * nch;

  // packed weight tiles of this wave's 4 column tiles: byte address of row
  // group rg, piece c, load h, this lane = base + (rg * nch_all + c) * 2048 + h * 1024 + 16 * lane
  const char* wtile[4];
  const uint8_t* stile[4];   // MXFP4: this lane's scale byte of the tile, piece 0, load 0
  const int n0 = (chunk * CWG + cg) * 64;   // first weight row (dense/down) of this wave
#pragma unroll
  for (int ct = 0; ct < 4; ct++) {
    const char* base;
    const uint8_t* sbase = nullptr;
    size_t row;   // first row of the 16-row group in its matrix
    if (MODE == SG_GATEUP) {
      // 32 SwiGLU outputs per column group: tiles [gate f, up f, gate f+16, up f+16]
      row = (size_t)e * a.NW + (chunk * CWG + cg) * 32 + 16 * (ct >> 1);
      base = (const char*)((ct & 1) ? a.W1 : a.W0);
      sbase = (ct & 1) ? a.S1 : a.S0;
    } else if (MODE == SG_DOWN) {
      row = (size_t)e * a.NW + n0 + 16 * ct;
      base = (const char*)a.W0;
      sbase = a.S0;
    } else {
      // groups past N read group 0: their output columns are never stored
      const int n = n0 + 16 * ct;
      const int nn = n < a.N ? n : 0;
      if (nn < a.n1) { base = (const char*)a.W0; row = nn; }
      else if (nn < a.n1 + a.n2) { base = (const char*)a.W1; row = nn - a.n1; }
      else { base = (const char*)a.W2; row = nn - a.n1 - a.n2; }
    }
    wtile[ct] = base + (row / 16) * rg_bytes + 16 * lane;
    stile[ct] = MX ? sbase + (row / 16) * (rg_bytes / 16) + lane : nullptr;
  }

  // residual values of this thread's outputs (stored by thread (w, lane) in
  // the epilogue: rows 16rt + 4g + i, column tile w of each column group),
  // loaded now so that their latency hides behind the main loop
  float res[MODE == SG_RESID ? RT : 1][MODE == SG_RESID ? CWG : 1][4];
  if (MODE == SG_RESID) {
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
#pragma unroll
      for (int grp = 0; grp < CWG; grp++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int r = rt * 16 + 4 * g + i;
          const int n = (chunk * CWG + grp) * 64 + 16 * w + l16;
          const bool ok = r < nrows && n < a.N;
          res[rt][grp][i] = ldx((const TA*)a.R, ok ? (size_t)(row0 + r) * a.ldo + n : 0);
        }
  }

  f32x4_t acc[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; rt++)
#pragma unroll
    for (int ct = 0; ct < 4; ct++) acc[rt][ct] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  // NB register buffers of one piece each: the loads of NB-1 later pieces are
  // in flight while a piece is multiplied
  u32x4 wbuf[NB][4][2], abuf[NB][RT][NA];
  uint32_t sbuf[NB][4][2];   // MXFP4 scale bytes of each buffer's weight loads
  auto load_w = [&](u32x4(&wr)[4][2], int c) {
#pragma unroll
    for (int h = 0; h < (MX ? 1 : 2); h++)
#pragma unroll
      for (int ct = 0; ct < 4; ct++) {
        // MXFP4 half piece c: load c % 2 of 128-byte piece c / 2
        const size_t off = MX ? (size_t)(c >> 1) * 2048 + (c & 1) * 1024 : (size_t)c * 2048 + h * 1024;
        wr[ct][h] = (GROUPED ? STREAM_NT : STREAM_NT_DENSE)
                        ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wtile[ct] + off))
                        : *reinterpret_cast<const u32x4*>(wtile[ct] + off);
      }
  };
  auto load_s = [&](uint32_t(&sr)[4][2], int c) {
    if constexpr (MX) {
#pragma unroll
      for (int ct = 0; ct < 4; ct++) sr[ct][0] = stile[ct][(size_t)(c >> 1) * 128 + (c & 1) * 64];
    }
  };
  const TA* arow[RT];
  auto load_a = [&](u32x4(&ar)[RT][NA], int c) {
#pragma unroll
    for (int j = 0; j < NA; j++)
#pragma unroll
      for (int rt = 0; rt < RT; rt++)
        ar[rt][j] = *reinterpret_cast<const u32x4*>(arow[rt] + c * PC::EP + PC::a_off(j, g));
  };
  // router (SG_F32) with a.gs: each activation element times gs[element],
  // rounded to the activation type, before the MFMAs (the RMSNorm weight in
  // front of the router; the row's rsqrt is applied to the summed logits).
  // A 16-byte register holds 16 / sizeof(TA) consecutive elements, whose
  // scales come in two 16-byte loads (one for fp32).
  constexpr bool GSC = MODE == SG_F32;
  const bool gsc = GSC && a.gs != nullptr;
  float4 gbuf[GSC ? NB : 1][GSC ? NA : 1][2];
  auto load_g = [&](int b, int c) {
    if constexpr (GSC) {
      if (gsc) {
#pragma unroll
        for (int j = 0; j < NA; j++) {
          const float* gp = a.gs + c * PC::EP + PC::a_off(j, g);
          gbuf[b][j][0] = *reinterpret_cast<const float4*>(gp);
          if constexpr (sizeof(TA) == 2) gbuf[b][j][1] = *reinterpret_cast<const float4*>(gp + 4);
        }
      }
    }
  };
  auto scale_a = [&](int b) {
    if constexpr (GSC) {
      if (gsc) {
#pragma unroll
        for (int j = 0; j < NA; j++) {
          const float gj[8] = {gbuf[b][j][0].x, gbuf[b][j][0].y, gbuf[b][j][0].z, gbuf[b][j][0].w,
                               gbuf[b][j][1].x, gbuf[b][j][1].y, gbuf[b][j][1].z, gbuf[b][j][1].w};
#pragma unroll
          for (int rt = 0; rt < RT; rt++) {
            u32x4 u = abuf[b][rt][j];
#pragma unroll
            for (int q = 0; q < 4; q++) {
              if constexpr (sizeof(TA) == 2)
                u[q] = f2bf2(__uint_as_float(u[q] << 16) * gj[2 * q],
                             __uint_as_float(u[q] & 0xffff0000u) * gj[2 * q + 1]);
              else
                u[q] = __float_as_uint(__uint_as_float(u[q]) * gj[q]);
            }
            abuf[b][rt][j] = u;
          }
        }
      }
    }
  };
  auto load = [&](int b, int c) {
    load_w(wbuf[b], c);
    load_s(sbuf[b], c);
    load_a(abuf[b], c);
    load_g(b, c);
  };
  auto comp = [&](int b) {
    scale_a(b);
    if constexpr (MX) piece_mma_mx<RT>(acc, wbuf[b], abuf[b], sbuf[b], nrt);
    else piece_mma<RT>(acc, wbuf[b], abuf[b], nrt, (TA*)nullptr, (TW*)nullptr);
  };
  // ok = false: the piece is past the contraction (a clamped load of the last
  // piece), so its A is zeroed
  auto comp_masked = [&](int b, bool ok) {
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
#pragma unroll
      for (int j = 0; j < NA; j++) zero_unless(abuf[b][rt][j], ok);
    comp(b);
  };

  // wave takes pieces kw, kw+KW, ...; indices past the end are clamped and
  // masked so the code is straight-line and the waits before each MFMA group
  // cover only that buffer's loads.  Every index past the end falls in the
  // last group (the count is rounded up to a multiple of NB), so only that
  // group is masked.  sched_barrier keeps each refill ahead of the next
  // buffers' MFMAs (otherwise the scheduler sinks the loads).
  const int per = (nch + KW - 1) / KW;
  const int nper = (per + NB - 1) / NB * NB;
  auto cidx = [&](int i) { const int c = kw + KW * i; return pbeg + (c < nch ? c : nch - 1); };
  auto cok = [&](int i) { return kw + KW * i < nch; };
  // A rows of this lane (row l16 of each 16-row tile).  Rows past the tile
  // read a valid row: an MFMA output row depends on its own A row only, and
  // those rows are never stored, so the load path needs no branches or masks
  // and the next piece's loads stay in flight during the MFMAs.  For the
  // gate/up GEMM the rows come through the permutation: those loads are
  // issued first and the first piece's weight loads right behind them, so
  // the wait for the permutation (an in-order counter) does not hold back
  // the weight stream.  Each buffer keeps its weight loads just ahead of its
  // A loads: a piece's MFMAs then wait for that buffer only.
  int src[RT];
#pragma unroll
  for (int rt = 0; rt < RT; rt++) {
    const int r = rt * 16 + l16;
    const int slot = row0 + (r < nrows ? r : 0);
    src[rt] = MODE == SG_GATEUP ? a.perm[slot] : slot;
  }
  __builtin_amdgcn_sched_barrier(0);
  load_w(wbuf[0], cidx(0));
  load_s(sbuf[0], cidx(0));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int rt = 0; rt < RT; rt++)
    arow[rt] = (const TA*)a.A + (size_t)(MODE == SG_GATEUP ? src[rt] / a.k : src[rt]) * K;
  load_a(abuf[0], cidx(0));
  load_g(0, cidx(0));
#pragma unroll
  for (int b = 1; b < NB; b++) load(b, cidx(b));
  int ib = 0;
  for (; ib + NB < nper; ib += NB) {
#pragma unroll
    for (int b = 0; b < NB; b++) {
      __builtin_amdgcn_sched_barrier(0);
      comp(b);
      __builtin_amdgcn_sched_barrier(0);
      load(b, cidx(ib + NB + b));
    }
  }
#pragma unroll
  for (int b = 0; b < NB; b++) {   // last group: nothing left to load
    __builtin_amdgcn_sched_barrier(0);
    comp_masked(b, cok(ib + b));
  }

  // ---- reduce the four waves' partial tiles, one 16-row tile at a time ----
  float sg = 1.f, su = 1.f, sd = 1.f;
  if (GROUPED && a.escale) {
    sg = a.escale[e * 3 + 0];
    su = a.escale[e * 3 + 1];
    sd = a.escale[e * 3 + 2];
  }
#pragma unroll
  for (int rt = 0; rt < RT; rt++) {   // constant register indices; tiles past nrt stop
    if (rt >= nrt) break;
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
                swiglu(gv, uv));
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
            ((float*)a.out)[o + (size_t)split * a.M * a.ldo] = val;
          } else {
            if (MODE == SG_RESID) val += res[MODE == SG_RESID ? rt : 0][MODE == SG_RESID ? grp : 0][i];
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

// register buffers (pieces in flight) per wave, chosen by measurement: bf16
// gate/up, bf16 down and dense projections, fp8 experts
constexpr int STREAM_NB_GATEUP = 2;
constexpr int STREAM_NB = 2;
constexpr int STREAM_NB_FP8 = 2;
// register buffers of the dense bf16 projections (64- and 32-row tiles)
constexpr int STREAM_NB_DENSE4 = 2;
constexpr int STREAM_NB_DENSE2 = 2;
// blocks a dense bf16 launch needs to take 64-row tiles
constexpr int STREAM_DENSE_RT4_BLOCKS = 256;
// 16-row tiles per expert tile of the bf16 grouped GEMMs
constexpr int STREAM_RT_BF16 = 4;

// rows per expert tile of the grouped modes (the plan cuts tiles this size)
int stream_tile_rows(int act, int wdt) {
  return act == ACT_BF16 && wdt == DG_BF16 ? 16 * STREAM_RT_BF16 : 32;
}


// row tiles a grouped launch covers: the down projection's grid is
// tile-major over the 8 XCDs, so its tile count is rounded up to 8 (the
// tiles past the plan's count exit at once)
template <int MODE>
constexpr int grouped_tiles(int ntiles_max) {
  return MODE == SG_DOWN ? (ntiles_max + 7) / 8 * 8 : ntiles_max;
}

// dense bf16 projections take 64-row tiles when that still gives at least
// one block per CU (fewer re-reads of each weight chunk), else 32-row tiles
template <int MODE, int KW>
static void dispatch(int act, int wdt, const StreamGemm& a, int ntiles_max, hipStream_t s) {
  constexpr bool GROUPED = MODE == SG_GATEUP || MODE == SG_DOWN;
  const int nsp = MODE == SG_F32 && a.ksplit > 1 ? a.ksplit : 1;
  if (act == ACT_F32) {
    const int nb = a.nchunks * (GROUPED ? grouped_tiles<MODE>(ntiles_max) : (a.M + 31) / 32) * nsp;
    if (nb > 0) wstream_k<float, float, MODE, KW, 2, 2><<<nb, 256, 0, s>>>(a);
  } else if (wdt == DG_FP8E4M3) {
    const int nb = a.nchunks * (GROUPED ? grouped_tiles<MODE>(ntiles_max) : (a.M + 31) / 32) * nsp;
    if (nb > 0) wstream_k<uint16_t, uint8_t, MODE, KW, STREAM_NB_FP8, 2><<<nb, 256, 0, s>>>(a);
  } else if (wdt == DG_MXFP4) {
    if constexpr (GROUPED) {
      const int nb = a.nchunks * grouped_tiles<MODE>(ntiles_max);
      if (nb > 0) wstream_k<uint16_t, mxfp4_t, MODE, KW, 2, 2><<<nb, 256, 0, s>>>(a);
    }
  } else if constexpr (GROUPED) {
    const int nb = a.nchunks * grouped_tiles<MODE>(ntiles_max);
    if (nb > 0)
      wstream_k<uint16_t, uint16_t, MODE, KW, MODE == SG_GATEUP ? STREAM_NB_GATEUP : STREAM_NB,
                STREAM_RT_BF16><<<nb, 256, 0, s>>>(a);
  } else {
    const int nb4 = a.nchunks * ((a.M + 63) / 64) * nsp, nb2 = a.nchunks * ((a.M + 31) / 32) * nsp;
    if (nb4 >= STREAM_DENSE_RT4_BLOCKS)
      wstream_k<uint16_t, uint16_t, MODE, KW, STREAM_NB_DENSE4, 4><<<nb4, 256, 0, s>>>(a);
    else if (nb2 > 0)
      wstream_k<uint16_t, uint16_t, MODE, KW, STREAM_NB_DENSE2, 2><<<nb2, 256, 0, s>>>(a);
  }
}

// kw: waves splitting the contraction (4, or 2 when the block should cover 128
// weight rows, e.g. a short contraction); a.nchunks counts blocks per row
// tile; ntiles_max bounds the expert row tiles of the grouped modes (the
// dense modes tile a.M rows themselves)
void launch_stream_gemm(int act, int wdt, int mode, int kw, const StreamGemm& a, int ntiles_max,
                        hipStream_t s) {
  const int nb = ntiles_max;
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
  }
}

}  // namespace dg
