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
// O^T += V^T P^T with V staged transposed in LDS (bf16: P as hi + lo bf16).  Online softmax in fp32
// (base-2 exponent with the scale folded in).  Key splits write unnormalised
// partials (O, m, l) that a merge kernel combines in split order.
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
};

template <typename TA, int HD>
__global__ __launch_bounds__(256) void attn_k(AttnArgs a) {
  typedef typename FragOf<TA>::type Frag;
  constexpr int KLD = HD + 16 / (int)sizeof(TA);   // padded row of the K tile
  constexpr int VLD = KT + 16 / (int)sizeof(TA);   // padded row of the transposed V tile
  __shared__ __attribute__((aligned(16))) TA ks[KT * KLD];
  __shared__ __attribute__((aligned(16))) TA vt[HD * VLD];

  const int qt = blockIdx.x, b = blockIdx.y / a.Hkv, gh = blockIdx.y % a.Hkv, split = blockIdx.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l16 = lane & 15, g4 = lane >> 4;
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
  for (int t = 0; t < HD / 16; t++) o[t] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  float mrow = -INFINITY, lsum = 0.f;

  for (int k0 = kbeg; k0 < kend; k0 += KT) {
    __syncthreads();
    // ---- stage K [KT][HD] ----
    constexpr int CPR = HD * (int)sizeof(TA) / 16;   // 16-byte chunks per key row
    for (int c = threadIdx.x; c < KT * CPR; c += 256) {
      const int j = c / CPR, q = c % CPR;
      const int kk = k0 + j;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (kk < kend) {
        const TA* src = (a.mode == 0 && kk >= P)
                            ? (const TA*)a.kn + (size_t)(b * a.T + kk - P) * a.ldq + gh * HD
                            : (const TA*)a.kc + (((size_t)b * a.Hkv + gh) * a.cap + kk) * HD;
        v = *reinterpret_cast<const uint4*>(src + q * (16 / (int)sizeof(TA)));
      }
      *reinterpret_cast<uint4*>(ks + j * KLD + q * (16 / (int)sizeof(TA))) = v;
    }
    // ---- stage V transposed: vt[d][j] ----
    constexpr int EPC = 16 / (int)sizeof(TA);        // elements per 16-byte chunk
    for (int c = threadIdx.x; c < (KT / 4) * (HD / EPC); c += 256) {
      const int jg = c / (HD / EPC), dq = c % (HD / EPC);
      TA vals[4][EPC];
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const int kk = k0 + 4 * jg + jj;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (kk < kend) {
          const TA* src = (a.mode == 0 && kk >= P)
                              ? (const TA*)a.vn + (size_t)(b * a.T + kk - P) * a.ldq + gh * HD
                              : (const TA*)a.vc + (((size_t)b * a.Hkv + gh) * a.cap + kk) * HD;
          v = *reinterpret_cast<const uint4*>(src + dq * EPC);
        }
        *reinterpret_cast<uint4*>(vals[jj]) = v;
      }
#pragma unroll
      for (int d = 0; d < EPC; d++) {
        TA* dst = vt + (dq * EPC + d) * VLD + 4 * jg;
#pragma unroll
        for (int jj = 0; jj < 4; jj++) dst[jj] = vals[jj][d];
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T: lane holds keys 16*mt + 4*g4 + i for query row l16 ----
    f32x4_t s[KT / 16];
#pragma unroll
    for (int mt = 0; mt < KT / 16; mt++) {
      s[mt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ss = 0; ss < HD / 32; ss++) {
        Frag kf;
        load_frag(kf, ks + (16 * mt + l16) * KLD + 32 * ss + 8 * g4);
        mma(s[mt], kf, qf[ss]);
      }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < KT / 16; mt++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int kk = k0 + 16 * mt + 4 * g4 + i;
        float v = s[mt][i] * a.scale_log2;
        if (kk >= kend || kk > qlimit || !qvalid) v = -INFINITY;
        s[mt][i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float mnew = fmaxf(mrow, tmax);
    const float alpha = mnew == -INFINITY ? 1.f : exp2f(mrow - mnew);
    float psum = 0.f;
#pragma unroll
    for (int mt = 0; mt < KT / 16; mt++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const float p = mnew == -INFINITY ? 0.f : exp2f(s[mt][i] - mnew);
        s[mt][i] = p;
        psum += p;
      }
    lsum = lsum * alpha + psum;
    mrow = mnew;
#pragma unroll
    for (int t = 0; t < HD / 16; t++) o[t] *= alpha;

    // ---- O^T += V^T P^T: key slot 8*g4 + 4*t + i <-> key 32*c + 16*t + 4*g4 + i ----
    // bf16: P is split into hi + lo bf16 parts (two MFMAs), so the products
    // keep ~16 mantissa bits of P instead of bf16's 8.
#pragma unroll
    for (int c = 0; c < KT / 32; c++) {
      Frag pf, pl;
      if constexpr (sizeof(TA) == 2) {
        uint16_t ph[8], plo[8];
#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const float p = s[2 * c + t][i];
            const uint16_t h = f2bf(p);
            ph[4 * t + i] = h;
            plo[4 * t + i] = f2bf(p - bf2f(h));
          }
        pf.v = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<uint4*>(ph));
        pl.v = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<uint4*>(plo));
      } else {
#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
          for (int i = 0; i < 4; i++) pf.v[4 * t + i] = s[2 * c + t][i];
      }
#pragma unroll
      for (int ht = 0; ht < HD / 16; ht++) {
        const TA* vrow = vt + (16 * ht + l16) * VLD + 32 * c + 4 * g4;
        Frag vf;
        if constexpr (sizeof(TA) == 2) {
          uint2 lo = *reinterpret_cast<const uint2*>(vrow);
          uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16);
          vf.v = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
          mma(o[ht], vf, pf);
          mma(o[ht], vf, pl);
        } else {
          float4 lo = *reinterpret_cast<const float4*>(vrow);
          float4 hi = *reinterpret_cast<const float4*>(vrow + 16);
          vf.v[0] = lo.x; vf.v[1] = lo.y; vf.v[2] = lo.z; vf.v[3] = lo.w;
          vf.v[4] = hi.x; vf.v[5] = hi.y; vf.v[6] = hi.z; vf.v[7] = hi.w;
          mma(o[ht], vf, pf);
        }
      }
    }
  }

  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (!qvalid) return;
  const size_t row = (size_t)b * a.T + qi;
  if (a.nsplit == 1) {
    const float inv = 1.f / lsum;
    TA* out = (TA*)a.out + row * (a.Hq * HD) + head * HD;
#pragma unroll
    for (int ht = 0; ht < HD / 16; ht++)
#pragma unroll
      for (int i = 0; i < 4; i++) stx(out, 16 * ht + 4 * g4 + i, o[ht][i] * inv);
  } else {
    const size_t e = ((size_t)split * a.rows + row) * a.Hq + head;
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
}

// combine key splits in split order: o = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s
template <typename TA>
__global__ __launch_bounds__(256) void attn_merge_k(const float* __restrict__ po,
                                                    const float* __restrict__ pml, int nsplit,
                                                    int entries, int hd, TA* __restrict__ out) {
  const int e = blockIdx.x * (256 / 64) + (threadIdx.x >> 6);   // (row, head) entry
  if (e >= entries) return;
  const int lane = threadIdx.x & 63;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; s++) M = fmaxf(M, pml[2 * ((size_t)s * entries + e)]);
  float den = 0.f;
  for (int s = 0; s < nsplit; s++) {
    const float m = pml[2 * ((size_t)s * entries + e)];
    if (m != -INFINITY) den += exp2f(m - M) * pml[2 * ((size_t)s * entries + e) + 1];
  }
  for (int d = lane; d < hd; d += 64) {
    float num = 0.f;
    for (int s = 0; s < nsplit; s++) {
      const float m = pml[2 * ((size_t)s * entries + e)];
      if (m != -INFINITY) num += exp2f(m - M) * po[((size_t)s * entries + e) * hd + d];
    }
    stx(out, (size_t)e * hd + d, num / den);
  }
}

// ---------------------------------------------------------------------------
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
  if (base < 512) {
    nsplit = (int)((512 + base - 1) / base);
    const int by_keys = (maxkeys + 127) / 128;
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

  dim3 grid(nqt, h.B * h.Hkv, nsplit);
  if (h.act == ACT_BF16) {
    if (h.hd == 128) attn_k<uint16_t, 128><<<grid, 256, 0, s>>>(a);
    else attn_k<uint16_t, 64><<<grid, 256, 0, s>>>(a);
  } else {
    if (h.hd == 128) attn_k<float, 128><<<grid, 256, 0, s>>>(a);
    else attn_k<float, 64><<<grid, 256, 0, s>>>(a);
  }
  if (nsplit > 1) {
    const int entries = a.rows * h.Hq;
    if (h.act == ACT_BF16)
      attn_merge_k<uint16_t><<<(entries + 3) / 4, 256, 0, s>>>(h.po, h.pml, nsplit, entries, h.hd,
                                                               (uint16_t*)h.out);
    else
      attn_merge_k<float><<<(entries + 3) / 4, 256, 0, s>>>(h.po, h.pml, nsplit, entries, h.hd,
                                                            (float*)h.out);
  }
}

}  // namespace dg
