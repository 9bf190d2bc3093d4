// kern_gemm.hip -- LDS-tiled MFMA GEMM C = A . B^T for the dense projections,
// the grouped expert GEMMs when many rows route to each expert, and the LM
// head with a fused per-row (max, argmax, sum exp) epilogue.
//
// Block: 256 threads = 4 waves in a 2 x 2 grid over a BM x BN output tile.
// Contraction tiles of 128 bytes per row (64 bf16 or 32 fp32 elements) are
// staged through LDS with a register prefetch of the next tile (double
// buffer); fp8 weights are decoded to bf16 on the way into LDS.  LDS rows are
// padded to 144 bytes so the 16 rows a fragment read touches fall in distinct
// banks.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace dg {

// byte address of row group (row / 16) of a packed matrix with nkb 128-byte
// pieces per row
__device__ __forceinline__ const char* packed_group(const void* base, size_t row, int nkb) {
  return (const char*)base + (row >> 4) * (size_t)nkb * 2048;
}

// contraction tiles in flight in registers in the LDS-tiled GEMMs (one more
// than the tile being stored, so a tile's loads have P - 1 steps to land)
constexpr int GEMM_P = 2;

template <typename TA, typename TW, int BM, int BN, int P = 1>
struct Mainloop {
  static constexpr int BK = 128 / (int)sizeof(TA);            // elements per staged row
  static constexpr int LDK = 160 / (int)sizeof(TA);           // padded LDS row: 160 B keeps fragment reads conflict-free
  static constexpr bool FP8 = sizeof(TW) == 1;
  static constexpr int A_LD = BM / 32;                         // 16-byte A chunks per thread
  static constexpr int B_ROWS_PER_PASS = FP8 ? 64 : 32;        // rows covered by 256 threads
  static constexpr int B_LD = BN / B_ROWS_PER_PASS;
  static constexpr int RT = BM / 32, CT = BN / 32;             // 16x16 tiles per wave
  static constexpr int SMEM = 2 * (BM + BN) * LDK;             // elements of TA
  static constexpr int NT = 256, WN = BN / 2, WM = BM / 2;
  static __device__ __forceinline__ int wave_m() { return threadIdx.x >> 7; }
  static __device__ __forceinline__ int wave_n() { return (threadIdx.x >> 6) & 1; }
  typedef typename FragOf<TA>::type Frag;

  // thread -> chunk assignment
  static __device__ __forceinline__ int a_row(int p) { return (threadIdx.x >> 3) + 32 * p; }
  static __device__ __forceinline__ int a_col() { return (threadIdx.x & 7) * (16 / (int)sizeof(TA)); }
  // B comes from the packed weight layout (tiles of 16 rows x 128 bytes, two
  // 1 KB halves; lane l of a half holds row l%16, bytes 64h + 16(l/16)): a
  // pass of the 256 threads stages 2 row groups x both halves (32 rows of one
  // 128-byte piece) or, for fp8, 4 row groups x the half that holds this
  // 64-element k-tile.  Each wave load is 1 KB of contiguous memory.
  static __device__ __forceinline__ int b_row(int p) {
    const int t = threadIdx.x;
    return FP8 ? 64 * p + 16 * (t >> 6) + (t & 15) : 32 * p + 16 * (t >> 7) + (t & 15);
  }
  static __device__ __forceinline__ int b_col() {   // TW elements into the k-tile
    const int t = threadIdx.x;
    return FP8 ? 16 * ((t & 63) >> 4) : (64 * ((t >> 6) & 1) + 16 * ((t & 63) >> 4)) / (int)sizeof(TW);
  }
  // byte offset of this thread's 16 bytes inside a row group's piece
  static __device__ __forceinline__ int b_lane() {
    const int t = threadIdx.x;
    return (FP8 ? 0 : ((t >> 6) & 1) * 1024) + (t & 63) * 16;
  }
  // byte offset of k-tile kt inside a row group's packed rows
  static __device__ __forceinline__ size_t b_koff(int kt) {
    return FP8 ? (size_t)(kt >> 1) * 2048 + (kt & 1) * 1024 : (size_t)kt * 2048;
  }

  // ap[p]: row pointers of the A rows this thread stages; bp[p]: byte address
  // of this thread's 16 bytes in k-tile 0 of its packed B row group (b_lane
  // included).  Rows with aok/bok false point at valid memory and are zeroed
  // by a select, so the load path has no branches.  P contraction tiles are in flight in registers
  // (a ring of P stages) while the MFMAs consume the LDS copy of an older
  // one; the tile count is padded to a multiple of P with zero tiles.
  static __device__ __forceinline__ void run(const TA* const (&ap)[A_LD], const bool (&aok)[A_LD],
                                             const char* const (&bp)[B_LD], const bool (&bok)[B_LD],
                                             int K, TA* smem, f32x4_t (&acc)[RT][CT]) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm = w >> 1, wn = w & 1, l16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
#pragma unroll
      for (int ct = 0; ct < CT; ct++) acc[rt][ct] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

    uint4 ra[P][A_LD], rb[P][B_LD];
    const int nk = K / BK;
    const int nkp = (nk + P - 1) / P * P;
    auto gload = [&](int st, int kt) {
      const int kc = kt < nk ? kt : nk - 1;   // clamped: always issued
      const int k0 = kc * BK;
#pragma unroll
      for (int p = 0; p < A_LD; p++) ra[st][p] = *reinterpret_cast<const uint4*>(ap[p] + k0 + a_col());
#pragma unroll
      for (int p = 0; p < B_LD; p++) rb[st][p] = *reinterpret_cast<const uint4*>(bp[p] + b_koff(kc));
    };
    auto zero_if = [](uint4& u, bool ok) {
      u.x = ok ? u.x : 0u;
      u.y = ok ? u.y : 0u;
      u.z = ok ? u.z : 0u;
      u.w = ok ? u.w : 0u;
    };
    auto sstore = [&](int st, int buf, bool ok) {
      TA* sa = smem + buf * (BM + BN) * LDK;
      TA* sb = sa + BM * LDK;
#pragma unroll
      for (int p = 0; p < A_LD; p++) zero_if(ra[st][p], aok[p] && ok);
#pragma unroll
      for (int p = 0; p < B_LD; p++) zero_if(rb[st][p], bok[p] && ok);
#pragma unroll
      for (int p = 0; p < A_LD; p++) *reinterpret_cast<uint4*>(sa + a_row(p) * LDK + a_col()) = ra[st][p];
#pragma unroll
      for (int p = 0; p < B_LD; p++) {
        if (FP8) {
          uint4 lo = fp8x8_to_bf16x8(make_uint2(rb[st][p].x, rb[st][p].y));
          uint4 hi = fp8x8_to_bf16x8(make_uint2(rb[st][p].z, rb[st][p].w));
          *reinterpret_cast<uint4*>(sb + b_row(p) * LDK + b_col()) = lo;
          *reinterpret_cast<uint4*>(sb + b_row(p) * LDK + b_col() + 8) = hi;
        } else {
          *reinterpret_cast<uint4*>(sb + b_row(p) * LDK + b_col()) = rb[st][p];
        }
      }
    };

    // fragments of one 32-wide contraction step, double-buffered so the LDS
    // reads of step ks+1 are in flight while the MFMAs of step ks run
    constexpr int KS = BK / 32;
    Frag af[2][RT], bf[2][CT];
    auto lload = [&](int buf, int ks, int fb) {
      const TA* sa = smem + buf * (BM + BN) * LDK;
      const TA* sb = sa + BM * LDK;
#pragma unroll
      for (int rt = 0; rt < RT; rt++)
        load_frag(af[fb][rt], sa + (wm * (BM / 2) + 16 * rt + l16) * LDK + 32 * ks + 8 * g);
#pragma unroll
      for (int ct = 0; ct < CT; ct++)
        load_frag(bf[fb][ct], sb + (wn * (BN / 2) + 16 * ct + l16) * LDK + 32 * ks + 8 * g);
    };
    auto mmas = [&](int fb) {
#pragma unroll
      for (int rt = 0; rt < RT; rt++)
#pragma unroll
        for (int ct = 0; ct < CT; ct++) mma(acc[rt][ct], af[fb][rt], bf[fb][ct]);
    };

#pragma unroll
    for (int st = 0; st < P; st++) gload(st, st);
    sstore(0, 0, true);
    __syncthreads();
    for (int kb = 0; kb < nkp; kb += P) {
#pragma unroll
      for (int st = 0; st < P; st++) {
        const int kt = kb + st;
        gload(st, kt + P);   // stage st was stored to LDS in the previous step
        __builtin_amdgcn_sched_barrier(0);
        lload(kt & 1, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
          if (ks + 1 < KS) lload(kt & 1, ks + 1, (ks + 1) & 1);
          __builtin_amdgcn_sched_barrier(0);
          mmas(ks & 1);
          __builtin_amdgcn_sched_barrier(0);
        }
        sstore((st + 1) % P, (kt + 1) & 1, kt + 1 < nk);
        __syncthreads();
      }
    }
  }
};

// Variant for bf16 activations whose weight operand goes straight from the
// packed layout into MFMA fragments: a 1 KB wave load is one 16 x 32 bf16
// fragment, or for fp8 weights two fragments decoded in registers (lane g
// then holds contraction elements 16g .. 16g+15 of the 64-element k-tile, so
// the activation fragments read the same elements: offset 16g + 8ks instead
// of 32ks + 8g -- one consistent permutation of the contraction).  Only the
// activation tile is staged through LDS, which halves the LDS traffic of the
// two-operand form.  Waves: NWM along the rows x BN/WN along the columns,
// each a (BM/NWM) x WN tile; a wider block reads each activation row fewer
// times from L2, and one wave along the rows reads each weight once per block
// (at twice the LDS reads of two).  Each k-tile ends at a block barrier
// after the next tile's activations are stored, which holds every wave until
// the slowest has stored its share; with one block per CU nothing fills the
// matrix cores meanwhile, so the grouped GEMMs keep a block under 128 VGPRs
// (two per CU).  Registers hold a ring of P k-tiles.
template <typename TW, int BM, int BN, int P, int NWM, int WN_>
struct MainloopD {
  typedef uint16_t TA;
  static constexpr int WN = WN_;            // columns per wave
  static constexpr int BK = 64, LDK = 80;   // 160-byte LDS rows (32 mod 64: conflict-free reads)
  static constexpr bool FP8 = sizeof(TW) == 1;
  static constexpr int NWN = BN / WN, NT = 64 * NWM * NWN;   // waves along the columns, threads
  static constexpr int WM = BM / NWM;       // rows per wave
  static constexpr int A_LD = BM * 8 / NT;  // 16-byte A chunks per thread
  static constexpr int RT = WM / 16, CT = WN / 16;
  static_assert(BM * 8 % NT == 0, "A staging");
  static constexpr int NB = FP8 ? 1 : 2;    // 16-byte weight loads per column tile and k-tile
  static constexpr int SMEM = 2 * BM * LDK;
  static_assert(P >= 2, "a step stores the next tile's activations from another stage");
  static __device__ __forceinline__ int a_row(int p) { return (threadIdx.x >> 3) + (NT / 8) * p; }
  static __device__ __forceinline__ int a_col() { return (threadIdx.x & 7) * 8; }
  static __device__ __forceinline__ int wave_m() { return (threadIdx.x >> 6) / NWN; }
  static __device__ __forceinline__ int wave_n() { return (threadIdx.x >> 6) % NWN; }

  // bq[ct]: byte address of this lane's 16 bytes of the wave's column tile ct
  // in contraction piece 0 (row group base + 16 * lane)
  static __device__ __forceinline__ void run(const TA* const (&ap)[A_LD], const bool (&aok)[A_LD],
                                             const char* const (&bq)[CT], int K, TA* smem,
                                             f32x4_t (&acc)[RT][CT]) {
    const int lane = threadIdx.x & 63;
    const int wm = wave_m(), l16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
#pragma unroll
      for (int ct = 0; ct < CT; ct++) acc[rt][ct] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    u32x4 ra[P][A_LD], rb[P][CT][NB];
    const int nk = K / BK;
    const int nkp = (nk + P - 1) / P * P;
    auto gload = [&](int st, int kt) {
      const int kc = kt < nk ? kt : nk - 1;   // clamped: always issued
#pragma unroll
      for (int ct = 0; ct < CT; ct++)
#pragma unroll
        for (int h = 0; h < NB; h++)
          rb[st][ct][h] = *reinterpret_cast<const u32x4*>(
              bq[ct] + (FP8 ? (size_t)(kc >> 1) * 2048 + (kc & 1) * 1024 : (size_t)kc * 2048 + h * 1024));
#pragma unroll
      for (int p = 0; p < A_LD; p++) ra[st][p] = *reinterpret_cast<const u32x4*>(ap[p] + kc * BK + a_col());
    };
    auto sstore = [&](int st, int buf, bool ok) {   // tiles past the end are stored as zeros
      TA* sa = smem + buf * BM * LDK;
#pragma unroll
      for (int p = 0; p < A_LD; p++) {
        u32x4 u = ra[st][p];
        const bool z = aok[p] && ok;
        u.x = z ? u.x : 0u;
        u.y = z ? u.y : 0u;
        u.z = z ? u.z : 0u;
        u.w = z ? u.w : 0u;
        *reinterpret_cast<u32x4*>(sa + a_row(p) * LDK + a_col()) = u;
      }
    };
    auto bfrag = [&](int st, int ct, int ks) {
      FragBF f;
      if constexpr (FP8) {
        const u32x4 u = rb[st][ct][0];
        f.v = __builtin_bit_cast(bf16x8_t, fp8x8_to_bf16x8(ks ? make_uint2(u.z, u.w) : make_uint2(u.x, u.y)));
      } else {
        f.v = __builtin_bit_cast(bf16x8_t, rb[st][ct][ks]);
      }
      return f;
    };
    const int aoff0 = FP8 ? 16 * g : 8 * g;   // A fragment column of ks = 0
    const int aoffs = FP8 ? 8 : 32;           // and the step to ks = 1

#pragma unroll
    for (int st = 0; st < P; st++) gload(st, st);
    sstore(0, 0, true);
    __syncthreads();
    for (int kb = 0; kb < nkp; kb += P) {
#pragma unroll
      for (int st = 0; st < P; st++) {
        const int kt = kb + st;
        const TA* sa = smem + (kt & 1) * BM * LDK;
        FragBF af[2][RT];
#pragma unroll
        for (int ks = 0; ks < 2; ks++)
#pragma unroll
          for (int rt = 0; rt < RT; rt++)
            load_frag(af[ks][rt], sa + (wm * WM + 16 * rt + l16) * LDK + aoff0 + aoffs * ks);
#pragma unroll
        for (int ks = 0; ks < 2; ks++)
#pragma unroll
          for (int ct = 0; ct < CT; ct++) {
            const FragBF bf = bfrag(st, ct, ks);
#pragma unroll
            for (int rt = 0; rt < RT; rt++) mma(acc[rt][ct], af[ks][rt], bf);
          }
        __builtin_amdgcn_sched_barrier(0);
        sstore((st + 1) % P, (kt + 1) & 1, kt + 1 < nk);   // A of tile kt+1 (loaded P-1 steps ago)
        gload(st, kt + P);                                  // stage st is consumed
        __syncthreads();
      }
    }
  }
};

// Main loop of the LDS-tiled GEMMs: bf16 activations take MainloopD with NWM
// waves along the rows (2: 64-column wave tiles from BN = 128 on; 1: waves of
// group_wn columns side by side), fp32 activations Mainloop (2 x 2 waves).
// Register rings: GROUP_P k-tiles for one wave along the rows, GEMM_P for
// two.  Expert tiles of 64 rows keep a block small enough that two or three
// blocks share a CU and one block's barrier waits are filled by the others'
// MFMAs (batch-8 fp8 gate/up: 176 us at 128-row tiles with one block per CU,
// 143 at 64).
constexpr int GROUP_P = 2;
constexpr int GROUP_BM = 64;   // rows of a bf16-activation expert tile
constexpr int DENSE_WIDE = 1;  // dense bf16 GEMMs from 1024 rows: 64-row tiles, waves side by side
// columns per wave with one wave along the rows: 64 for fp8 weights (each
// wave reads the block's activation tile from LDS once per 64 columns: batch-8
// gate/up 133 -> 127 us, down unchanged), 32 for bf16 weights (64 made the
// dense projections at 2048 rows ~10 us slower in all)
template <typename TW>
constexpr int group_wn() { return sizeof(TW) == 1 ? 64 : 32; }
template <typename TA, typename TW, int BM, int BN, int NWM>
using GemmML = typename std::conditional<
    sizeof(TA) == 2,
    typename std::conditional<NWM == 1, MainloopD<TW, BM, BN, GROUP_P, 1, group_wn<TW>()>,
                              MainloopD<TW, BM, BN, GEMM_P, 2, (BN >= 128 ? 64 : BN / 2)>>::type,
    Mainloop<TA, TW, BM, BN, GEMM_P>>::type;
template <typename TA, typename TW, int BM, int BN, int NWM>
constexpr int gemm_threads() {
  return GemmML<TA, TW, BM, BN, NWM>::NT;
}

// ---------------------------------------------------------------------------
// dense GEMM with epilogues
// ---------------------------------------------------------------------------
struct DenseArgs {
  const void* A;
  int M, K;
  const void* B0;
  int n1;
  const void* B1;
  int n2;
  const void* B2;
  int N;
  void* C;
  int ldc;
  const void* R;
  int mode;
  CacheDst cache;
};

template <typename TA, int BM, int BN, int NWM>
__global__ __launch_bounds__((gemm_threads<TA, TA, BM, BN, NWM>())) void gemm_dense_k(DenseArgs a) {
  // bf16: weights straight into fragments; fp32: both operands through LDS
  typedef GemmML<TA, TA, BM, BN, NWM> ML;
  __shared__ __attribute__((aligned(16))) TA smem[ML::SMEM];
  const int m0 = blockIdx.x * BM, n0 = blockIdx.y * BN;
  const TA* ap[ML::A_LD];
  bool aok[ML::A_LD];
  const int nkb = a.K * (int)sizeof(TA) / 128;
#pragma unroll
  for (int p = 0; p < ML::A_LD; p++) {
    const int r = m0 + ML::a_row(p);
    aok[p] = r < a.M;
    ap[p] = (const TA*)a.A + (size_t)(aok[p] ? r : 0) * a.K;
  }
  // weight row n: from B0, B1 or B2 by range; rows past N read row 0 (never stored)
  auto wrow = [&](int n) -> const char* {
    const int nn = n < a.N ? n : 0;
    if (nn < a.n1) return packed_group(a.B0, nn, nkb);
    if (nn < a.n1 + a.n2) return packed_group(a.B1, nn - a.n1, nkb);
    return packed_group(a.B2, nn - a.n1 - a.n2, nkb);
  };
  f32x4_t acc[ML::RT][ML::CT];
  if constexpr (sizeof(TA) == 2) {
    const int wn = ML::wave_n(), lane = threadIdx.x & 63;
    const char* bq[ML::CT];
#pragma unroll
    for (int ct = 0; ct < ML::CT; ct++) bq[ct] = wrow(n0 + wn * ML::WN + 16 * ct) + 16 * lane;
    ML::run(ap, aok, bq, a.K, smem, acc);
  } else {
    const char* bp[ML::B_LD];
    bool bok[ML::B_LD];
#pragma unroll
    for (int p = 0; p < ML::B_LD; p++) {
      const int n = n0 + ML::b_row(p);
      bok[p] = n < a.N;
      bp[p] = wrow(n) + ML::b_lane();
    }
    ML::run(ap, aok, bp, bok, a.K, smem, acc);
  }

  const int lane = threadIdx.x & 63;
  const int wm = ML::wave_m(), wn = ML::wave_n(), l16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int rt = 0; rt < ML::RT; rt++)
#pragma unroll
    for (int ct = 0; ct < ML::CT; ct++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int r = m0 + wm * ML::WM + 16 * rt + 4 * g + i;
        const int n = n0 + wn * ML::WN + 16 * ct + l16;
        if (r >= a.M || n >= a.N) continue;
        float v = acc[rt][ct][i];
        const size_t o = (size_t)r * a.ldc + n;
        if (a.mode == GEMM_F32) {
          ((float*)a.C)[o] = v;
          continue;
        }
        if (a.mode == GEMM_RESID) v += ldx((const TA*)a.R, o);
        stx((TA*)a.C, o, v);
        if (a.mode == GEMM_QKV_CACHE && n >= a.cache.QD) {
          // new key / value of token (b, i) goes to cache position len[b] + i
          const int c = n - a.cache.QD;
          const bool isv = c >= a.cache.KD;
          const int cc = isv ? c - a.cache.KD : c;
          const int gh = cc / a.cache.hd, d = cc % a.cache.hd;
          const int b = r / a.cache.T, t = r % a.cache.T;
          const size_t co = (((size_t)b * a.cache.Hkv + gh) * a.cache.cap + a.cache.len.v[b] + t) *
                                a.cache.hd + d;
          stx((TA*)(isv ? a.cache.v : a.cache.k), co, v);
        }
      }
}

// ---------------------------------------------------------------------------
// grouped expert GEMMs over row tiles (expert, first permuted row, rows)
// ---------------------------------------------------------------------------
struct GroupArgs {
  const void* A;
  const int32_t* perm;
  int k;
  const void* W1;
  const void* W2;
  const float* escale;
  const int4* tiles;
  const int32_t* ntiles;
  int K, NW, ldo;
  void* out;
  int max_tiles, ncol;   // row tiles the grid was sized for; column blocks per row tile
};

// The grouped GEMMs run on a 1-D grid of 8 * ceil(max_tiles * ncol / 8) blocks.
// Work items (row tile, column block) are numbered row-tile-major, and the
// XCD that runs block b (b mod 8, the round-robin dispatch order) takes the
// contiguous range [x * per, (x + 1) * per) of the ntiles * ncol live items:
// the column blocks of one row tile, and the row tiles of one expert, run
// side by side on one XCD and share its L2 copy of the activation rows and of
// the expert's weights (a column-major grid spreads them over all 8 L2s).
__device__ __forceinline__ bool group_item(const GroupArgs& a, int& tile, int& col) {
  const int nt = min(*a.ntiles, a.max_tiles);
  const int total = nt * a.ncol, per = (total + 7) >> 3;
  const int j = blockIdx.x >> 3, w = (blockIdx.x & 7) * per + j;
  if (j >= per || w >= total) return false;
  tile = w / a.ncol;
  col = w - tile * a.ncol;
  return true;
}

// gate/up: BN weight rows = BN/2 SwiGLU outputs, rows ordered in 32-row
// groups [gate f..f+15, up f..f+15] so each wave holds matching gate and up tiles.
template <typename TA, typename TW, int BM, int BN, int NWM>
__global__ __launch_bounds__((gemm_threads<TA, TW, BM, BN, NWM>())) void gateup_lds_k(GroupArgs a) {
  typedef GemmML<TA, TW, BM, BN, NWM> ML;
  __shared__ __attribute__((aligned(16))) TA smem[ML::SMEM];
  int tile_id, col;
  if (!group_item(a, tile_id, col)) return;
  const int4 tl = a.tiles[tile_id];
  const int e = tl.x, row0 = tl.y, nrows = tl.z;
  const int f0 = col * (BN / 2);
  const TA* ap[ML::A_LD];
  bool aok[ML::A_LD];
  const int nkb = a.K * (int)sizeof(TW) / 128;
#pragma unroll
  for (int p = 0; p < ML::A_LD; p++) {
    const int r = ML::a_row(p);
    aok[p] = r < nrows;
    ap[p] = (const TA*)a.A + (size_t)(a.perm[row0 + (aok[p] ? r : 0)] / a.k) * a.K;
  }
  // tile row n (of BN): 32-row groups [gate f .. f+15, up f .. f+15]
  auto wrow = [&](int n) -> const char* {
    const int f = f0 + 16 * (n >> 5) + (n & 15);
    return packed_group(((n >> 4) & 1) ? a.W2 : a.W1, (size_t)e * a.NW + f, nkb);
  };
  f32x4_t acc[ML::RT][ML::CT];
  if constexpr (sizeof(TA) == 2) {
    const int wn = ML::wave_n(), lane = threadIdx.x & 63;
    const char* bq[ML::CT];
#pragma unroll
    for (int ct = 0; ct < ML::CT; ct++) bq[ct] = wrow(wn * ML::WN + 16 * ct) + 16 * lane;
    ML::run(ap, aok, bq, a.K, smem, acc);
  } else {
    const char* bp[ML::B_LD];
    bool bok[ML::B_LD];
#pragma unroll
    for (int p = 0; p < ML::B_LD; p++) {
      bp[p] = wrow(ML::b_row(p)) + ML::b_lane();
      bok[p] = true;
    }
    ML::run(ap, aok, bp, bok, a.K, smem, acc);
  }

  const int lane = threadIdx.x & 63;
  const int wm = ML::wave_m(), wn = ML::wave_n(), l16 = lane & 15, g = lane >> 4;
  float sg = 1.f, su = 1.f;
  if (a.escale) {
    sg = a.escale[e * 3 + 0];
    su = a.escale[e * 3 + 1];
  }
#pragma unroll
  for (int rt = 0; rt < ML::RT; rt++)
#pragma unroll
    for (int p = 0; p < ML::CT / 2; p++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int r = wm * ML::WM + 16 * rt + 4 * g + i;
        if (r >= nrows) continue;
        const float gv = acc[rt][2 * p][i] * sg, uv = acc[rt][2 * p + 1][i] * su;
        const int f = f0 + wn * (ML::WN / 2) + 16 * p + l16;
        stx((TA*)a.out, (size_t)(row0 + r) * a.ldo + f, swiglu(gv, uv));
      }
}

template <typename TA, typename TW, int BM, int BN, int NWM>
__global__ __launch_bounds__((gemm_threads<TA, TW, BM, BN, NWM>())) void down_lds_k(GroupArgs a) {
  typedef GemmML<TA, TW, BM, BN, NWM> ML;
  __shared__ __attribute__((aligned(16))) TA smem[ML::SMEM];
  int tile_id, col;
  if (!group_item(a, tile_id, col)) return;
  const int4 tl = a.tiles[tile_id];
  const int e = tl.x, row0 = tl.y, nrows = tl.z;
  const int n0 = col * BN;
  const TA* ap[ML::A_LD];
  bool aok[ML::A_LD];
  const int nkb = a.K * (int)sizeof(TW) / 128;
#pragma unroll
  for (int p = 0; p < ML::A_LD; p++) {
    const int r = ML::a_row(p);
    aok[p] = r < nrows;
    ap[p] = (const TA*)a.A + (size_t)(row0 + (aok[p] ? r : 0)) * a.K;
  }
  f32x4_t acc[ML::RT][ML::CT];
  if constexpr (sizeof(TA) == 2) {
    const int wn = ML::wave_n(), lane = threadIdx.x & 63;
    const char* bq[ML::CT];
#pragma unroll
    for (int ct = 0; ct < ML::CT; ct++)
      bq[ct] = packed_group(a.W1, (size_t)e * a.NW + n0 + wn * ML::WN + 16 * ct, nkb) + 16 * lane;
    ML::run(ap, aok, bq, a.K, smem, acc);
  } else {
    const char* bp[ML::B_LD];
    bool bok[ML::B_LD];
#pragma unroll
    for (int p = 0; p < ML::B_LD; p++) {
      bp[p] = packed_group(a.W1, (size_t)e * a.NW + n0 + ML::b_row(p), nkb) + ML::b_lane();
      bok[p] = true;
    }
    ML::run(ap, aok, bp, bok, a.K, smem, acc);
  }

  const int lane = threadIdx.x & 63;
  const int wm = ML::wave_m(), wn = ML::wave_n(), l16 = lane & 15, g = lane >> 4;
  const float sd = a.escale ? a.escale[e * 3 + 2] : 1.f;
#pragma unroll
  for (int rt = 0; rt < ML::RT; rt++)
#pragma unroll
    for (int ct = 0; ct < ML::CT; ct++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int r = wm * ML::WM + 16 * rt + 4 * g + i;
        if (r >= nrows) continue;
        const int n = n0 + wn * ML::WN + 16 * ct + l16;
        stx((TA*)a.out, (size_t)(row0 + r) * a.ldo + n, acc[rt][ct][i] * sd);
      }
}

// ---------------------------------------------------------------------------
// LM head for fp32 activations: logits tile [BM rows x 128 vocabulary],
// reduced per row to (max, lowest index attaining it, sum exp(l - max));
// logits never stored unless the debug tap asks for them.
// ---------------------------------------------------------------------------
struct HeadArgs {
  const void* A;
  int M, K;
  const void* B;
  int V;
  float* pmax;
  int32_t* pidx;
  float* psum;
  float* logits;
  int ntiles, mtiles;
};

__device__ __forceinline__ void mrg(float& m, int& i, float& s, float m2, int i2, float s2) {
  if (m2 == -INFINITY) return;
  if (m2 > m || (m2 == m && i2 < i)) {
    s = s * __expf(m - m2) + s2;
    m = m2;
    i = i2;
  } else {
    s = s + s2 * __expf(m2 - m);
  }
}

template <typename TA, int BM, int P>
__global__ __launch_bounds__(256) void lmhead_k(HeadArgs a) {
  constexpr int BN = 128;
  typedef Mainloop<TA, TA, BM, BN, P> ML;
  __shared__ __attribute__((aligned(16))) TA smem[ML::SMEM];
  __shared__ float xm[2][BM], xs[2][BM];
  __shared__ int xi[2][BM];
  // 1-D grid; the row tiles of one column tile are 8 block ids apart, so
  // they run on the same XCD and share its L2 copy of the weight tile
  const int b8 = blockIdx.x >> 3, mtiles = a.mtiles;
  const int nt = (b8 / mtiles) * 8 + (blockIdx.x & 7), mt = b8 % mtiles;
  if (nt >= a.ntiles) return;
  const int n0 = nt * BN, m0 = mt * BM;
  const TA* ap[ML::A_LD];
  const char* bp[ML::B_LD];
  bool aok[ML::A_LD], bok[ML::B_LD];
  const int nkb = a.K * (int)sizeof(TA) / 128;
#pragma unroll
  for (int p = 0; p < ML::A_LD; p++) {
    const int r = m0 + ML::a_row(p);
    aok[p] = r < a.M;
    ap[p] = (const TA*)a.A + (size_t)(aok[p] ? r : 0) * a.K;
  }
#pragma unroll
  for (int p = 0; p < ML::B_LD; p++) {
    const int n = n0 + ML::b_row(p);
    bok[p] = n < a.V;
    bp[p] = packed_group(a.B, bok[p] ? n : 0, nkb) + ML::b_lane();
  }
  f32x4_t acc[ML::RT][ML::CT];
  ML::run(ap, aok, bp, bok, a.K, smem, acc);

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1, l16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int rt = 0; rt < ML::RT; rt++)
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int rl = wm * (BM / 2) + 16 * rt + 4 * g + i;
      const int r = m0 + rl;
      float m = -INFINITY, s = 0.f;
      int idx = 0x7fffffff;
#pragma unroll
      for (int ct = 0; ct < ML::CT; ct++) {
        const int n = n0 + wn * (BN / 2) + 16 * ct + l16;
        const float v = n < a.V ? acc[rt][ct][i] : -INFINITY;
        if (a.logits && r < a.M && n < a.V) a.logits[(size_t)r * a.V + n] = v;
        mrg(m, idx, s, v, n, 1.f);
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
        const int i2 = __shfl_xor(idx, o, 64);
        mrg(m, idx, s, m2, i2, s2);
      }
      if (l16 == 0) {
        xm[wn][rl] = m;
        xs[wn][rl] = s;
        xi[wn][rl] = idx;
      }
    }
  __syncthreads();
  for (int rl = threadIdx.x; rl < BM; rl += 256) {
    const int r = m0 + rl;
    if (r >= a.M) continue;
    float m = xm[0][rl], s = xs[0][rl];
    int idx = xi[0][rl];
    mrg(m, idx, s, xm[1][rl], xi[1][rl], xs[1][rl]);
    const size_t o = (size_t)r * a.ntiles + nt;
    a.pmax[o] = m;
    a.pidx[o] = idx;
    a.psum[o] = s;
  }
}

// Epilogue of the LM head kernels.  acc[rt][ct] is the block's transposed
// logits tile: lane (l16, g) of wave w holds vocabulary rows
// n0 + WC w + 16 ct + 4 g + i (i = 0..3) of token m0 + 16 rt + l16, so a
// token's WC columns of this wave sit in 4 CT registers of 4 lanes (g = 0..3).
// Writes, per token of the tile, the maximum over the block's NW WC columns,
// the lowest column attaining it and sum exp(l - max) to the tile's partials.
template <int NW, int RT, int CT>
__device__ __forceinline__ void head_tile_epilogue(const f32x4_t (&acc)[RT][CT], const HeadArgs& a,
                                                   int n0, int m0, int nt, float (*xm)[16 * RT],
                                                   float (*xs)[16 * RT], int (*xi)[16 * RT]) {
  constexpr int WC = 16 * CT, BM = 16 * RT;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, l16 = lane & 15, g = lane >> 4;
  if (a.logits) {   // debug tap: raw logits, 4 consecutive columns per store
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
#pragma unroll
      for (int ct = 0; ct < CT; ct++) {
        const int r = m0 + 16 * rt + l16, n = n0 + WC * w + 16 * ct + 4 * g;
        if (r < a.M)
#pragma unroll
          for (int i = 0; i < 4; i++)
            if (n + i < a.V) a.logits[(size_t)r * a.V + n + i] = acc[rt][ct][i];
      }
  }
  // epilogue: per token (a row of the transposed tile) the maximum over this
  // wave's WC columns, the lowest column attaining it and sum exp(l - max).
  // Lane maxima (max3 chains), two exchanges for the wave maximum, then per value one
  // compare-select against it (columns visited in descending order, so the
  // last hit is the lowest; the select keeps a small column code) and one
  // fused exponent argument.  The RT row tiles step together (independent
  // chains).  Column tiles inside the vocabulary take the path without masks.
  float m[RT], s[RT];
  int idx[RT];
  auto epilogue = [&](auto full) {
    constexpr bool FULL = decltype(full)::value;
    const int nl = n0 + WC * w + 4 * g;   // column of value (ct, i) = nl + 16 ct + i
    bool ok[CT][4];
#pragma unroll
    for (int ct = 0; ct < CT; ct++)
#pragma unroll
      for (int i = 0; i < 4; i++) ok[ct][i] = FULL || nl + 16 * ct + i < a.V;
#pragma unroll
    for (int rt = 0; rt < RT; rt++) {   // 4 CT values: one max3 per two after the first
      float x[4 * CT];
#pragma unroll
      for (int ct = 0; ct < CT; ct++)
#pragma unroll
        for (int i = 0; i < 4; i++) x[4 * ct + i] = ok[ct][i] ? acc[rt][ct][i] : -INFINITY;
      float v = x[0];
#pragma unroll
      for (int j = 1; j + 1 < 4 * CT; j += 2) v = fmax3(v, x[j], x[j + 1]);
      m[rt] = __builtin_fmaxf(v, x[4 * CT - 1]);
    }
#pragma unroll
    for (int rt = 0; rt < RT; rt++) m[rt] = pair_max16(m[rt]);
#pragma unroll
    for (int rt = 0; rt < RT; rt++) m[rt] = pair_max32(m[rt]);
    int c[RT];   // code 4 ct + i of the lowest hit; 4 CT = none
#pragma unroll
    for (int rt = 0; rt < RT; rt++) c[rt] = 4 * CT;
#pragma unroll
    for (int ct = CT - 1; ct >= 0; ct--)
#pragma unroll
      for (int i = 3; i >= 0; i--)
#pragma unroll
        for (int rt = 0; rt < RT; rt++) c[rt] = ok[ct][i] && acc[rt][ct][i] == m[rt] ? 4 * ct + i : c[rt];
#pragma unroll
    for (int rt = 0; rt < RT; rt++) idx[rt] = c[rt] == 4 * CT ? 0x7fffffff : nl + 16 * (c[rt] >> 2) + (c[rt] & 3);
#pragma unroll
    for (int rt = 0; rt < RT; rt++) idx[rt] = pair_min16(idx[rt]);
#pragma unroll
    for (int rt = 0; rt < RT; rt++) idx[rt] = pair_min32(idx[rt]);
    constexpr float L2E = 1.4426950408889634f;
    float mb[RT];
#pragma unroll
    for (int rt = 0; rt < RT; rt++) {
      mb[rt] = m[rt] * L2E;
      s[rt] = 0.f;
    }
#pragma unroll
    for (int ct = 0; ct < CT; ct++)
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int rt = 0; rt < RT; rt++) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[rt][ct][i], L2E, -mb[rt]));
          s[rt] += ok[ct][i] ? e : 0.f;
        }
#pragma unroll
    for (int rt = 0; rt < RT; rt++) s[rt] = m[rt] == -INFINITY ? 0.f : s[rt];
  };
  if (n0 + WC * NW <= a.V) epilogue(std::integral_constant<bool, true>{});
  else epilogue(std::integral_constant<bool, false>{});
#pragma unroll
  for (int rt = 0; rt < RT; rt++) s[rt] = pair_sum16(s[rt]);
#pragma unroll
  for (int rt = 0; rt < RT; rt++) s[rt] = pair_sum32(s[rt]);
  if (g == 0) {
#pragma unroll
    for (int rt = 0; rt < RT; rt++) {
      const int rl = 16 * rt + l16;
      xm[w][rl] = m[rt];
      xs[w][rl] = s[rt];
      xi[w][rl] = idx[rt];
    }
  }
  __syncthreads();
  if (t < BM && m0 + t < a.M) {
    // the NW wave partials of token t at once: their maximum, then each sum
    // rescaled to it (independent exponentials), and the lowest column among
    // the partials that reach the maximum; an empty partial has max -inf
    float pm[NW], ps[NW];
    int pi[NW];
#pragma unroll
    for (int q = 0; q < NW; q++) {
      pm[q] = xm[q][t];
      ps[q] = xs[q][t];
      pi[q] = xi[q][t];
    }
    float M = pm[0];
#pragma unroll
    for (int q = 1; q < NW; q++) M = fmax_sel(M, pm[q]);
    constexpr float L2E = 1.4426950408889634f;
    float s = 0.f;
    int idx = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < NW; q++) {
      const float e = __builtin_amdgcn_exp2f((pm[q] - M) * L2E);
      s += pm[q] == -INFINITY ? 0.f : ps[q] * e;
      idx = pm[q] == M ? min(idx, pi[q]) : idx;
    }
    const size_t o = (size_t)(m0 + t) * a.ntiles + nt;
    a.pmax[o] = M;
    a.pidx[o] = idx;
    a.psum[o] = M == -INFINITY ? 0.f : s;
  }
}

// ---------------------------------------------------------------------------
// LM head for bf16 activations below 1024 rows.  Block tile: 128 rows x BN
// vocabulary entries; the NW waves sit side by side (128 x BN/NW each: 8
// waves of 32 columns).  Every weight byte is used by exactly one wave, so the
// weight rows stream from HBM straight into MFMA fragments (P contraction
// tiles in flight in registers); only the activation tile, which all waves
// share, goes through LDS (a 3-buffer ring, stored from registers loaded two
// steps earlier).  Staging both operands through LDS would make the LDS write
// port the bottleneck.
// ---------------------------------------------------------------------------
template <int P, int NW, int BN, int MINB>
__global__ __launch_bounds__(NW * 64, MINB) void lmhead_direct_k(HeadArgs a) {
  constexpr int NT = NW * 64;                 // threads
  constexpr int BM = 128, BK = 64, LDK = 80, RT = 8;   // 160-byte LDS rows: conflict-free fragment reads
  constexpr int WC = BN / NW, CT = WC / 16;   // vocabulary columns per wave
  constexpr int A_LD = BM * BK * 2 / 16 / NT;   // 16-byte A chunks staged per thread
  constexpr int A_RSTEP = NT / 8;             // rows between a thread's chunks
  // three LDS buffers: while tile kt is consumed, tile kt+1 is readable (its
  // first fragments are prefetched) and tile kt+2 is being written
  __shared__ __attribute__((aligned(16))) uint16_t sA[3][BM * LDK];
  __shared__ float xm[NW][BM], xs[NW][BM];
  __shared__ int xi[NW][BM];
  const int b8 = blockIdx.x >> 3, mtiles = a.mtiles;
  const int nt = (b8 / mtiles) * 8 + (blockIdx.x & 7), mt = b8 % mtiles;
  if (nt >= a.ntiles) return;
  const int n0 = nt * BN, m0 = mt * BM;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, l16 = lane & 15, g = lane >> 4;
  const uint16_t* A = (const uint16_t*)a.A;
  const uint16_t* W = (const uint16_t*)a.B;
  const int K = a.K, nk = K / BK, nkp = (nk + P - 1) / P * P;

  const uint16_t* ap[A_LD];
  bool aok[A_LD];
#pragma unroll
  for (int p = 0; p < A_LD; p++) {
    const int r = m0 + (t >> 3) + A_RSTEP * p;
    aok[p] = r < a.M;
    ap[p] = A + (size_t)(aok[p] ? r : 0) * K + (t & 7) * 8;
  }
  // packed weights: one 1 KB wave load per (column tile, k-tile, half)
  const char* bp[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ct++) {
    const int n = n0 + WC * w + 16 * ct;
    bp[ct] = packed_group(W, n < a.V ? n : 0, nk) + 16 * lane;   // groups past V: masked in the epilogue
  }

  f32x4_t acc[RT][CT];
#pragma unroll
  for (int rt = 0; rt < RT; rt++)
#pragma unroll
    for (int ct = 0; ct < CT; ct++) acc[rt][ct] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  uint4 ra[P][A_LD];
  FragBF rb[P][2][CT];
  auto gload = [&](int st, int kt) {
    const int k0 = (kt < nk ? kt : nk - 1) * BK;   // clamped: always issued
#pragma unroll
    for (int p = 0; p < A_LD; p++) ra[st][p] = *reinterpret_cast<const uint4*>(ap[p] + k0);
#pragma unroll
    for (int ks = 0; ks < 2; ks++)
#pragma unroll
      for (int ct = 0; ct < CT; ct++)
        rb[st][ks][ct].v = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(bp[ct] + (size_t)(k0 / BK) * 2048 + ks * 1024));
  };
  // tiles past the end are stored as zeros, so their MFMAs add nothing
  auto astore = [&](int st, int buf, bool ok) {
#pragma unroll
    for (int p = 0; p < A_LD; p++) {
      uint4 u = ra[st][p];
      const bool z = aok[p] && ok;
      u.x = z ? u.x : 0u;
      u.y = z ? u.y : 0u;
      u.z = z ? u.z : 0u;
      u.w = z ? u.w : 0u;
      *reinterpret_cast<uint4*>(&sA[buf][((t >> 3) + A_RSTEP * p) * LDK + (t & 7) * 8]) = u;
    }
  };
  FragBF af[2][RT];
  auto lload = [&](int buf, int ks) {
#pragma unroll
    for (int rt = 0; rt < RT; rt++) load_frag(af[ks][rt], &sA[buf][(16 * rt + l16) * LDK + 32 * ks + 8 * g]);
  };
  auto mmas = [&](int st, int ks) {
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
#pragma unroll
      for (int ct = 0; ct < CT; ct++) mma(acc[rt][ct], rb[st][ks][ct], af[ks][rt]);   // logits^T
  };

#pragma unroll
  for (int st = 0; st < P; st++) gload(st, st);
  astore(0, 0, true);
  astore(1 % P, 1, 1 < nk);
  __syncthreads();
  lload(0, 0);
  int cur = 0;   // LDS buffer of tile kt
  auto step = [&](int st, int kt, auto with_load) {
    const int nxt = cur == 2 ? 0 : cur + 1, nn = nxt == 2 ? 0 : nxt + 1;
    lload(cur, 1);
    __builtin_amdgcn_sched_barrier(0);
    mmas(st, 0);
    __builtin_amdgcn_sched_barrier(0);
    lload(nxt, 0);   // tile kt+1: written one step ago, behind the last barrier
    __builtin_amdgcn_sched_barrier(0);
    mmas(st, 1);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (decltype(with_load)::value) {
      gload(st, kt + P);   // stage st: its A tile is in LDS, its B fragments consumed
      __builtin_amdgcn_sched_barrier(0);
    }
    astore((st + 2) % P, nn, kt + 2 < nk);
    __syncthreads();
    cur = nxt;
  };
  int kb = 0;
  for (; kb + P < nkp; kb += P) {
#pragma unroll
    for (int st = 0; st < P; st++) step(st, kb + st, std::integral_constant<bool, true>{});
  }
  // last group: every tile it needs is already loaded, so it issues no loads
  // (loads past the end would only hold the epilogue's registers)
#pragma unroll
  for (int st = 0; st < P; st++) step(st, kb + st, std::integral_constant<bool, false>{});

  head_tile_epilogue<NW, RT, CT>(acc, a, n0, m0, nt, xm, xs, xi);
}

// ---------------------------------------------------------------------------
// LM head for bf16 activations and many rows (batched canvases).  Block tile
// 128 rows x BN vocabulary entries, NW waves side by side of 128 rows x 64
// columns each.  Every wave reads the whole activation tile from LDS each
// step, so twice the columns of lmhead_direct_k per wave halve the LDS
// fragment reads per MFMA (the LDS command queue is what fills up there).
// The 128 accumulators per lane leave room for one fragment register set and
// two register stages: a step reads its fragments while the other wave of
// the SIMD multiplies, and the activation tile of step kt + 1 is stored from
// registers loaded one step earlier.
// ---------------------------------------------------------------------------
template <int P, int NW, int BN>
__global__ __launch_bounds__(NW * 64, 1) void lmhead_wide_k(HeadArgs a) {
  constexpr int NT = NW * 64;                 // threads
  constexpr int BM = 128, BK = 64, LDK = 80, RT = 8;   // 160-byte LDS rows: conflict-free fragment reads
  constexpr int WC = BN / NW, CT = WC / 16;   // vocabulary columns per wave
  constexpr int A_LD = BM * BK * 2 / 16 / NT;   // 16-byte A chunks staged per thread
  constexpr int A_RSTEP = NT / 8;             // rows between a thread's chunks
  static_assert(A_LD >= 1 && A_LD * NT * 16 == BM * BK * 2, "activation staging");
  // two LDS buffers: tile kt is read while tile kt + 1 is written
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * LDK];
  __shared__ float xm[NW][BM], xs[NW][BM];
  __shared__ int xi[NW][BM];
  const int b8 = blockIdx.x >> 3, mtiles = a.mtiles;
  const int nt = (b8 / mtiles) * 8 + (blockIdx.x & 7), mt = b8 % mtiles;
  if (nt >= a.ntiles) return;
  const int n0 = nt * BN, m0 = mt * BM;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, l16 = lane & 15, g = lane >> 4;
  const uint16_t* A = (const uint16_t*)a.A;
  const uint16_t* W = (const uint16_t*)a.B;
  const int K = a.K, nk = K / BK, nkp = (nk + P - 1) / P * P;

  const uint16_t* ap[A_LD];
  bool aok[A_LD];
#pragma unroll
  for (int p = 0; p < A_LD; p++) {
    const int r = m0 + (t >> 3) + A_RSTEP * p;
    aok[p] = r < a.M;
    ap[p] = A + (size_t)(aok[p] ? r : 0) * K + (t & 7) * 8;
  }
  const char* bp[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ct++) {
    const int n = n0 + WC * w + 16 * ct;
    bp[ct] = packed_group(W, n < a.V ? n : 0, nk) + 16 * lane;   // groups past V: masked in the epilogue
  }

  f32x4_t acc[RT][CT];
#pragma unroll
  for (int rt = 0; rt < RT; rt++)
#pragma unroll
    for (int ct = 0; ct < CT; ct++) acc[rt][ct] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  uint4 ra[P][A_LD];
  FragBF rb[P][2][CT];
  auto gload = [&](int st, int kt) {
    const int k0 = (kt < nk ? kt : nk - 1) * BK;   // clamped: always issued
#pragma unroll
    for (int p = 0; p < A_LD; p++) ra[st][p] = *reinterpret_cast<const uint4*>(ap[p] + k0);
#pragma unroll
    for (int ks = 0; ks < 2; ks++)
#pragma unroll
      for (int ct = 0; ct < CT; ct++)
        rb[st][ks][ct].v = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(bp[ct] + (size_t)(k0 / BK) * 2048 + ks * 1024));
  };
  // tiles past the end are stored as zeros, so their MFMAs add nothing
  auto astore = [&](int st, int buf, bool ok) {
#pragma unroll
    for (int p = 0; p < A_LD; p++) {
      uint4 u = ra[st][p];
      const bool z = aok[p] && ok;
      u.x = z ? u.x : 0u;
      u.y = z ? u.y : 0u;
      u.z = z ? u.z : 0u;
      u.w = z ? u.w : 0u;
      *reinterpret_cast<uint4*>(&sA[buf][((t >> 3) + A_RSTEP * p) * LDK + (t & 7) * 8]) = u;
    }
  };
  FragBF af[RT];
  auto lload = [&](int buf, int ks) {
#pragma unroll
    for (int rt = 0; rt < RT; rt++) load_frag(af[rt], &sA[buf][(16 * rt + l16) * LDK + 32 * ks + 8 * g]);
  };
  auto mmas = [&](int st, int ks) {
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
#pragma unroll
      for (int ct = 0; ct < CT; ct++) mma(acc[rt][ct], rb[st][ks][ct], af[rt]);   // logits^T
  };

#pragma unroll
  for (int st = 0; st < P; st++) gload(st, st);
  astore(0, 0, true);
  __syncthreads();
  auto step = [&](int st, int kt, auto with_load) {
    const int cur = kt & 1;
    lload(cur, 0);
    __builtin_amdgcn_sched_barrier(0);
    mmas(st, 0);
    __builtin_amdgcn_sched_barrier(0);
    lload(cur, 1);
    __builtin_amdgcn_sched_barrier(0);
    mmas(st, 1);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (decltype(with_load)::value) {
      gload(st, kt + P);   // stage st: its A tile is in LDS, its B fragments consumed
      __builtin_amdgcn_sched_barrier(0);
    }
    astore((st + 1) % P, cur ^ 1, kt + 1 < nk);   // tile kt + 1 into the buffer of tile kt - 1
    __syncthreads();
  };
  int kb = 0;
  for (; kb + P < nkp; kb += P) {
#pragma unroll
    for (int st = 0; st < P; st++) step(st, kb + st, std::integral_constant<bool, true>{});
  }
#pragma unroll
  for (int st = 0; st < P; st++) step(st, kb + st, std::integral_constant<bool, false>{});

  head_tile_epilogue<NW, RT, CT>(acc, a, n0, m0, nt, xm, xs, xi);
}

// ---------------------------------------------------------------------------
void launch_gemm(int act, int mode, const void* A, int M, int K, const void* B0, int n1,
                 const void* B1, int n2, const void* B2, int N, void* C, int ldc, const void* R,
                 const CacheDst* cache, hipStream_t s) {
  DenseArgs a{A, M, K, B0, n1, B1, n2, B2, N, C, ldc, R, mode, CacheDst{}};
  if (cache) a.cache = *cache;
  if (act == ACT_BF16 && M > 1024 && DENSE_WIDE) {
    // 64-row tiles, waves of 32 columns side by side: 256 columns per block
    // when that still gives two blocks per CU, else 128
    constexpr int N8 = gemm_threads<uint16_t, uint16_t, 64, 256, 1>();
    constexpr int N4 = gemm_threads<uint16_t, uint16_t, 64, 128, 1>();
    const long b256 = (long)((M + 63) / 64) * ((N + 255) / 256);
    if (b256 >= 512) gemm_dense_k<uint16_t, 64, 256, 1><<<dim3((M + 63) / 64, (N + 255) / 256), N8, 0, s>>>(a);
    else gemm_dense_k<uint16_t, 64, 128, 1><<<dim3((M + 63) / 64, (N + 127) / 128), N4, 0, s>>>(a);
  } else if (M > 1024) {
    dim3 grid((M + 127) / 128, (N + 127) / 128);
    if (act == ACT_BF16) gemm_dense_k<uint16_t, 128, 128, 2><<<grid, gemm_threads<uint16_t, uint16_t, 128, 128, 2>(), 0, s>>>(a);
    else gemm_dense_k<float, 128, 128, 2><<<grid, 256, 0, s>>>(a);
  } else {
    dim3 grid((M + 63) / 64, (N + 63) / 64);
    if (act == ACT_BF16) gemm_dense_k<uint16_t, 64, 64, 2><<<grid, gemm_threads<uint16_t, uint16_t, 64, 64, 2>(), 0, s>>>(a);
    else gemm_dense_k<float, 64, 64, 2><<<grid, 256, 0, s>>>(a);
  }
}

int group_tile_rows(int act) { return act == ACT_F32 ? 128 : GROUP_BM; }

void launch_gateup_lds(int act, const void* u2, const int32_t* perm, int k, const MoeW& w,
                       const int4* tiles, const int32_t* ntiles, int max_tiles, int D, int F,
                       void* H, hipStream_t s) {
  GroupArgs a{u2, perm, k, w.wg, w.wu, w.escale, tiles, ntiles, D, F, F, H, max_tiles, 0};
  auto grid = [&](int ncol) {
    a.ncol = ncol;
    return dim3((unsigned)(((size_t)max_tiles * ncol + 7) / 8 * 8));
  };
  if (act == ACT_F32) {   // 128 weight rows = 64 SwiGLU outputs per block
    gateup_lds_k<float, float, 128, 128, 2><<<grid(F / 64), 256, 0, s>>>(a);
  } else if (F % 128 == 0) {   // 256 weight rows: each routed row is read F/128 times
    constexpr int N8 = gemm_threads<uint16_t, uint8_t, GROUP_BM, 256, 1>();
    constexpr int N16 = gemm_threads<uint16_t, uint16_t, GROUP_BM, 256, 1>();
    if (w.wdt == DG_FP8E4M3) gateup_lds_k<uint16_t, uint8_t, GROUP_BM, 256, 1><<<grid(F / 128), N8, 0, s>>>(a);
    else gateup_lds_k<uint16_t, uint16_t, GROUP_BM, 256, 1><<<grid(F / 128), N16, 0, s>>>(a);
  } else {
    constexpr int N8 = gemm_threads<uint16_t, uint8_t, GROUP_BM, 128, 2>();
    constexpr int N16 = gemm_threads<uint16_t, uint16_t, GROUP_BM, 128, 2>();
    if (w.wdt == DG_FP8E4M3) gateup_lds_k<uint16_t, uint8_t, GROUP_BM, 128, 2><<<grid(F / 64), N8, 0, s>>>(a);
    else gateup_lds_k<uint16_t, uint16_t, GROUP_BM, 128, 2><<<grid(F / 64), N16, 0, s>>>(a);
  }
}

void launch_down_lds(int act, const void* H, const MoeW& w, const int4* tiles,
                     const int32_t* ntiles, int max_tiles, int D, int F, void* Y, hipStream_t s) {
  GroupArgs a{H, nullptr, 0, w.wd, nullptr, w.escale, tiles, ntiles, F, D, D, Y, max_tiles, 0};
  auto grid = [&](int ncol) {
    a.ncol = ncol;
    return dim3((unsigned)(((size_t)max_tiles * ncol + 7) / 8 * 8));
  };
  if (act == ACT_F32) {
    down_lds_k<float, float, 128, 128, 2><<<grid(D / 128), 256, 0, s>>>(a);
  } else if (D % 256 == 0) {
    constexpr int N8 = gemm_threads<uint16_t, uint8_t, GROUP_BM, 256, 1>();
    constexpr int N16 = gemm_threads<uint16_t, uint16_t, GROUP_BM, 256, 1>();
    if (w.wdt == DG_FP8E4M3) down_lds_k<uint16_t, uint8_t, GROUP_BM, 256, 1><<<grid(D / 256), N8, 0, s>>>(a);
    else down_lds_k<uint16_t, uint16_t, GROUP_BM, 256, 1><<<grid(D / 256), N16, 0, s>>>(a);
  } else {
    constexpr int N8 = gemm_threads<uint16_t, uint8_t, GROUP_BM, 128, 2>();
    constexpr int N16 = gemm_threads<uint16_t, uint16_t, GROUP_BM, 128, 2>();
    if (w.wdt == DG_FP8E4M3) down_lds_k<uint16_t, uint8_t, GROUP_BM, 128, 2><<<grid(D / 128), N8, 0, s>>>(a);
    else down_lds_k<uint16_t, uint16_t, GROUP_BM, 128, 2><<<grid(D / 128), N16, 0, s>>>(a);
  }
}

// contraction tiles in flight in the bf16 LM head, and its waves per block
constexpr int LMHEAD_P = 4;
constexpr int LMHEAD_NW = 8;
constexpr int LMHEAD_BN = 256;
constexpr int LMHEAD_MINB = 1;
// up to this many rows: 4-wave blocks of 128 vocabulary entries
constexpr int LMHEAD_FEW_ROWS = 64;
constexpr int LMHEAD_FEW_BN = 128;
constexpr int LMHEAD_FEW_P = 3;
// from this many rows: 64 vocabulary columns per wave, 512 per block
constexpr int LMHEAD_WIDE_MIN_ROWS = 1024;
constexpr int LMHEAD_WIDE_P = 2;
constexpr int LMHEAD_WIDE_BN = 512;

int launch_lmhead(int act, const void* uf, int M, int D, const void* lm, int V, float* pmax,
                  int32_t* pidx, float* psum, float* logits, hipStream_t s) {
  if (act == ACT_BF16 && M >= LMHEAD_WIDE_MIN_ROWS) {
    const int nt = (V + LMHEAD_WIDE_BN - 1) / LMHEAD_WIDE_BN;
    HeadArgs a{uf, M, D, lm, V, pmax, pidx, psum, logits, nt, (M + 127) / 128};
    lmhead_wide_k<LMHEAD_WIDE_P, LMHEAD_NW, LMHEAD_WIDE_BN>
        <<<((nt + 7) / 8) * 8 * a.mtiles, LMHEAD_NW * 64, 0, s>>>(a);
    return nt;
  }
  if (act == ACT_BF16 && M <= LMHEAD_FEW_ROWS) {
    // a few rows (decoding steps): 128 vocabulary entries per block of 4
    // waves, so one row tile still makes a block per CU (one row: 94.6 against
    // 97.3 us per decoding step with 256-entry blocks, 104 with the LDS-tiled
    // head); 3 register stages keep it within 256 VGPRs
    const int nt = (V + LMHEAD_FEW_BN - 1) / LMHEAD_FEW_BN;
    HeadArgs a{uf, M, D, lm, V, pmax, pidx, psum, logits, nt, (M + 127) / 128};
    lmhead_direct_k<LMHEAD_FEW_P, 4, LMHEAD_FEW_BN, 2><<<((nt + 7) / 8) * 8 * a.mtiles, 4 * 64, 0, s>>>(a);
    return nt;
  }
  if (act == ACT_BF16) {   // rows past M are masked
    const int nt = (V + LMHEAD_BN - 1) / LMHEAD_BN;
    HeadArgs a{uf, M, D, lm, V, pmax, pidx, psum, logits, nt, (M + 127) / 128};
    lmhead_direct_k<LMHEAD_P, LMHEAD_NW, LMHEAD_BN, LMHEAD_MINB>
        <<<((nt + 7) / 8) * 8 * a.mtiles, LMHEAD_NW * 64, 0, s>>>(a);
    return nt;
  }
  // fp32 activations
  const int nt = (V + 127) / 128, bm = M > 64 ? 128 : 64;
  HeadArgs a{uf, M, D, lm, V, pmax, pidx, psum, logits, nt, (M + bm - 1) / bm};
  const dim3 grid(((nt + 7) / 8) * 8 * a.mtiles);
  if (bm == 128) lmhead_k<float, 128, 1><<<grid, 256, 0, s>>>(a);
  else lmhead_k<float, 64, 1><<<grid, 256, 0, s>>>(a);
  return nt;
}

}  // namespace dg
