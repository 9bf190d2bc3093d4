// kern_elem.hip -- embedding + RMSNorm, combine + RMSNorm, re-noise, coverage,
// tap un-permute and the LM-head partial merge.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace dg {

// Row kernels: one block of 256 threads per token row, 8 consecutive elements
// per thread and step (D is a multiple of 128).  A thread's chunks stay in
// registers between the sum of squares and the scaling (rows of up to
// 256 * 8 * ROWC elements); all loads of a phase are issued together.
constexpr int ROWC = 2;

// x[row] = emb[tk] (copied), u[row] = round(x * rsqrt(mean(x^2)+eps) * g) by
// the 256 threads of a block
template <typename TA>
__device__ __forceinline__ void embed_norm_row(int tk, const TA* __restrict__ emb,
                                               const float* __restrict__ g, int D, float eps,
                                               TA* __restrict__ x, TA* __restrict__ u, size_t row,
                                               float* red) {
  const TA* src = emb + (size_t)tk * D;
  float v[ROWC][8], gv[ROWC][8];
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < ROWC; q++) {
    const int c = threadIdx.x * 8 + 2048 * q, cc = c < D ? c : 0;   // clamped: no branch per load
    ld8(src + cc, v[q]);
    ld8(g + cc, gv[q]);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < ROWC; q++) {
    const int c = threadIdx.x * 8 + 2048 * q;
    if (c < D) {
      st8(x + row * D + c, v[q]);
#pragma unroll
      for (int i = 0; i < 8; i++) ss += v[q][i] * v[q][i];
    }
  }
  for (int c = threadIdx.x * 8 + 2048 * ROWC; c < D; c += 2048) {   // longer rows
    float w[8];
    ld8(src + c, w);
    st8(x + row * D + c, w);
#pragma unroll
    for (int i = 0; i < 8; i++) ss += w[i] * w[i];
  }
  ss = block_sum256(ss, red);
  const float r = rsqrtf(ss / (float)D + eps);
#pragma unroll
  for (int q = 0; q < ROWC; q++) {
    const int c = threadIdx.x * 8 + 2048 * q;
    if (c < D) {
#pragma unroll
      for (int i = 0; i < 8; i++) v[q][i] = v[q][i] * r * gv[q][i];
      st8(u + row * D + c, v[q]);
    }
  }
  for (int c = threadIdx.x * 8 + 2048 * ROWC; c < D; c += 2048) {
    float w[8];
    ld8(src + c, w);
#pragma unroll
    for (int i = 0; i < 8; i++) w[i] = w[i] * r * g[c + i];
    st8(u + row * D + c, w);
  }
}

// one block per token row (token ids outside [0, V) are clamped into range
// rather than read out of bounds)
template <typename TA>
__global__ __launch_bounds__(256) void embed_norm_k(const int32_t* __restrict__ tok,
                                                    const TA* __restrict__ emb,
                                                    const float* __restrict__ g, int D, int V,
                                                    float eps, TA* __restrict__ x,
                                                    TA* __restrict__ u) {
  __shared__ float red[4];
  const int tk = min(max(tok[blockIdx.x], 0), V - 1);
  embed_norm_row<TA>(tk, emb, g, D, eps, x, u, blockIdx.x, red);
}

template <typename TA>
__global__ __launch_bounds__(256) void rmsnorm_k(const TA* __restrict__ x, const float* __restrict__ g,
                                                 int D, float eps, TA* __restrict__ u) {
  __shared__ float red[4];
  const size_t row = blockIdx.x;
  float v[ROWC][8], gv[ROWC][8];
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < ROWC; q++) {
    const int c = threadIdx.x * 8 + 2048 * q, cc = c < D ? c : 0;
    ld8(x + row * D + cc, v[q]);
    ld8(g + cc, gv[q]);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < ROWC; q++)
    if (threadIdx.x * 8 + 2048 * q < D)
#pragma unroll
      for (int i = 0; i < 8; i++) ss += v[q][i] * v[q][i];
  for (int c = threadIdx.x * 8 + 2048 * ROWC; c < D; c += 2048) {
    float w[8];
    ld8(x + row * D + c, w);
#pragma unroll
    for (int i = 0; i < 8; i++) ss += w[i] * w[i];
  }
  ss = block_sum256(ss, red);
  const float r = rsqrtf(ss / (float)D + eps);
#pragma unroll
  for (int q = 0; q < ROWC; q++) {
    const int c = threadIdx.x * 8 + 2048 * q;
    if (c < D) {
#pragma unroll
      for (int i = 0; i < 8; i++) v[q][i] = v[q][i] * r * gv[q][i];
      st8(u + row * D + c, v[q]);
    }
  }
  for (int c = threadIdx.x * 8 + 2048 * ROWC; c < D; c += 2048) {
    float w[8];
    ld8(x + row * D + c, w);
#pragma unroll
    for (int i = 0; i < 8; i++) w[i] = w[i] * r * g[c + i];
    st8(u + row * D + c, w);
  }
}

// x = round(x1 + sum_j g_j y_j) in slot order j; u = round(rmsnorm(x) * gnext).
// The k gates and slot indices of the row are uniform loads; all k expert rows
// of a chunk are loaded before they are added (k <= 8).
template <typename TA>
__global__ __launch_bounds__(256) void combine_norm_k(const TA* __restrict__ x1,
                                                      const TA* __restrict__ Y,
                                                      const float* __restrict__ gates,
                                                      const int32_t* __restrict__ inv, int k, int D,
                                                      const float* __restrict__ gnext, float eps,
                                                      TA* __restrict__ x, TA* __restrict__ u,
                                                      int32_t* zero0, int32_t* zero1, int nzero) {
  __shared__ float red[4];
  const size_t row = blockIdx.x;
  // counters the pass's last kernel adds to start at zero: cleared here, by
  // the last layer's combine (the kernel before the head)
  if (row == 0 && (int)threadIdx.x < nzero) {
    if (zero0) zero0[threadIdx.x] = 0;
    if (zero1) zero1[threadIdx.x] = 0;
  }
  float gs[8];
  int32_t rs[8];
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const int jj = j < k ? j : 0;
    gs[j] = gates[row * k + jj];
    rs[j] = inv[row * k + jj];
  }
  float acc[ROWC][8], gv[ROWC][8];
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < ROWC; q++) {
    const int c = threadIdx.x * 8 + 2048 * q, cc = c < D ? c : 0;
    float y[8][8];
    ld8(x1 + row * D + cc, acc[q]);
    ld8(gnext + cc, gv[q]);
#pragma unroll
    for (int j = 0; j < 8; j++) ld8(Y + (size_t)rs[j] * D + cc, y[j]);
    __builtin_amdgcn_sched_barrier(0);   // every load above is issued before the first use
    float mix[8];
#pragma unroll
    for (int i = 0; i < 8; i++) mix[i] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; j++)   // slots past k select the unchanged sum (no branch)
#pragma unroll
      for (int i = 0; i < 8; i++) mix[i] = j < k ? mix[i] + gs[j] * y[j][i] : mix[i];
#pragma unroll
    for (int i = 0; i < 8; i++) acc[q][i] = rnd(acc[q][i] + mix[i], x);
    if (c < D) {
#pragma unroll
      for (int i = 0; i < 8; i++) ss += acc[q][i] * acc[q][i];
      st8(x + row * D + c, acc[q]);
    }
  }
  for (int c = threadIdx.x * 8 + 2048 * ROWC; c < D; c += 2048) {   // longer rows
    float a2[8], mix[8], y[8];
    ld8(x1 + row * D + c, a2);
#pragma unroll
    for (int i = 0; i < 8; i++) mix[i] = 0.f;
    for (int j = 0; j < k; j++) {
      ld8(Y + (size_t)rs[j] * D + c, y);
#pragma unroll
      for (int i = 0; i < 8; i++) mix[i] += gs[j] * y[i];
    }
#pragma unroll
    for (int i = 0; i < 8; i++) {
      a2[i] = rnd(a2[i] + mix[i], x);
      ss += a2[i] * a2[i];
    }
    st8(x + row * D + c, a2);
  }
  ss = block_sum256(ss, red);
  const float r = rsqrtf(ss / (float)D + eps);
#pragma unroll
  for (int q = 0; q < ROWC; q++) {
    const int c = threadIdx.x * 8 + 2048 * q;
    if (c < D) {
#pragma unroll
      for (int i = 0; i < 8; i++) acc[q][i] = acc[q][i] * r * gv[q][i];
      st8(u + row * D + c, acc[q]);
    }
  }
  for (int c = threadIdx.x * 8 + 2048 * ROWC; c < D; c += 2048) {
    float v[8];
    ld8(x + row * D + c, v);
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = v[i] * r * gnext[c + i];
    st8(u + row * D + c, v);
  }
}

// ---------------------------------------------------------------------------
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11): per round the counter
// words 0 and 2 are multiplied by the round constants; high halves are xored
// with the other words and the key, which is bumped by two Weyl constants.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; r++) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    const uint64_t hi0 = __umul64hi(M0, c[0]), lo0 = M0 * c[0];
    const uint64_t hi1 = __umul64hi(M1, c[2]), lo1 = M1 * c[2];
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

// the token of slot idx (request b, position i) after re-noise: argmax when
// kept, else a uniform draw floor(r * V / 2^64) from word 0 of Philox4x64-10
// with counter (pos0[b] + i, tag, req[b], 0) and key (seed, 0)
__device__ __forceinline__ int32_t renoise_token(const RenoiseArgs& a, int b, int i, bool keep,
                                                 int32_t am) {
  uint64_t c[4] = {(uint64_t)(int64_t)(a.pos0.v[b] + i), (uint64_t)a.tag, (uint64_t)a.req.v[b], 0};
  philox4x64_10(c, a.seed, 0);
  const int32_t noise = (int32_t)__umul64hi(c[0], (uint64_t)a.V);
  return keep ? am : noise;
}

// The token of slot (b, i) after the between-pass update, from its current
// token `old` and this pass's prediction (am, cf):
//  - uniform-state noise: the prediction where cf >= tau, else a fresh draw;
//  - masked ("absorbing") diffusion: a slot holding the [MASK] token takes the
//    prediction where cf >= tau (every masked slot on the last pass); any other
//    slot keeps its token (a filled slot is locked in).
__device__ __forceinline__ int32_t update_token(const RenoiseArgs& a, int b, int i, int32_t old,
                                                int32_t am, float cf) {
  if (a.mode == DG_SAMPLER_MASKED)
    return (old == a.mask_id && (a.final_pass || cf >= a.tau)) ? am : old;
  return renoise_token(a, b, i, cf >= a.tau, am);
}

// One block per request: every slot's update, then the request's counts.  No
// confidence: initialisation (uniform noise, or the [MASK] token everywhere).
__global__ __launch_bounds__(256) void canvas_update_k(RenoiseArgs a) {
  __shared__ int red[2][4];
  const int b = blockIdx.x;
  int nch = 0, nleft = 0;
  for (int i = threadIdx.x; i < a.N; i += 256) {
    const size_t idx = (size_t)b * a.N + i;
    const int32_t old = a.canvas[idx];
    int32_t t;
    if (!a.conf) t = a.mode == DG_SAMPLER_MASKED ? a.mask_id : renoise_token(a, b, i, false, 0);
    else t = update_token(a, b, i, old, a.argmax[idx], a.conf[idx]);
    a.canvas[idx] = t;
    nch += t != old;
    nleft += a.mode == DG_SAMPLER_MASKED && t == a.mask_id;
  }
  // counts of at most 2^24 slots: exact in fp32
  const float c0 = wave_sum((float)nch), c1 = wave_sum((float)nleft);
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = (int)c0;
    red[1][threadIdx.x >> 6] = (int)c1;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    if (a.changed) a.changed[b] = red[0][0] + red[0][1] + red[0][2] + red[0][3];
    if (a.masked_left) a.masked_left[b] = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  }
}

__global__ __launch_bounds__(256) void renoise_k(RenoiseArgs a) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= a.B * a.N) return;
  // confidence and argmax are loaded together (one memory round trip) and the
  // noise token is always drawn; the select keeps argmax where conf >= tau
  // (NaN compares false: noised)
  const bool keep = a.conf ? a.conf[idx] >= a.tau : false;
  const int32_t am = a.conf ? a.argmax[idx] : 0;
  a.canvas[idx] = renoise_token(a, idx / a.N, idx % a.N, keep, am);
}

// one block per layer l: touched[l] = #{e : counts[l][e] > 0}
__device__ __forceinline__ void coverage_block(const int32_t* __restrict__ counts, int E, int l,
                                               int32_t* __restrict__ touched,
                                               int32_t* __restrict__ counts_out, int* red) {
  int t = 0;
  for (int e = threadIdx.x; e < E; e += 256) {
    int c = counts[l * E + e];
    t += c > 0;
    if (counts_out) counts_out[l * E + e] = c;
  }
  t += lane_xor32(t);
  t += lane_xor16(t);
  t = (int)row16_sum((float)t);   // counts of at most 256 experts: exact in fp32
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = t;
  __syncthreads();
  if (threadIdx.x == 0) touched[l] = red[0] + red[1] + red[2] + red[3];
}

__global__ __launch_bounds__(256) void coverage_k(const int32_t* __restrict__ counts, int E,
                                                  int32_t* __restrict__ touched,
                                                  int32_t* __restrict__ counts_out) {
  __shared__ int red[4];
  coverage_block(counts, E, blockIdx.x, touched, counts_out, red);
}

// dst[slot][c] = src[inv[slot]][c]
template <typename TA>
__global__ __launch_bounds__(256) void unpermute_k(const TA* __restrict__ src,
                                                   const int32_t* __restrict__ inv, int C,
                                                   TA* __restrict__ dst) {
  const size_t slot = blockIdx.x;
  const size_t r = inv[slot];
  for (int c = threadIdx.x; c < C; c += 256) dst[slot * C + c] = src[r * C + c];
}

// Merge per-tile (max, argmax, sum exp(l - max)) in vocabulary order: the
// global maximum, the lowest index attaining it, conf = 1 / sum exp(l - max).
__device__ __forceinline__ void merge3(float& m, int& i, float& s, float m2, int i2, float s2) {
  if (m2 == -INFINITY) return;  // empty partial
  if (m2 > m || (m2 == m && i2 < i)) {
    s = s * __expf(m - m2) + s2;
    m = m2;
    i = i2;
  } else {
    s = s + s2 * __expf(m2 - m);
  }
}

// Blocks 0..rows-1 merge one row each; with nx.touched set, blocks rows..
// rows+L-1 write the expert coverage of the pass, and with nx.rn.canvas set
// each row's slot is re-noised for the next pass from the argmax and conf just
// computed (the same values renoise_k would read back).
__global__ __launch_bounds__(256) void lm_merge_k(const float* __restrict__ pmax,
                                                  const int32_t* __restrict__ pidx,
                                                  const float* __restrict__ psum, int ntiles,
                                                  int rows, int32_t* __restrict__ argmax,
                                                  float* __restrict__ conf, MergeNext nx) {
  __shared__ float sm[4], ss[4];
  __shared__ int si[4];
  __shared__ int stok;
  if ((int)blockIdx.x >= rows) {
    coverage_block(nx.counts, nx.E, blockIdx.x - rows, nx.touched, nullptr, si);
    return;
  }
  const size_t row = blockIdx.x;
  float m = -INFINITY, s = 0.f;
  int i = 0x7fffffff;
  for (int t = threadIdx.x; t < ntiles; t += 256)
    merge3(m, i, s, pmax[row * ntiles + t], pidx[row * ntiles + t], psum[row * ntiles + t]);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    int i2 = __shfl_xor(i, o, 64);
    merge3(m, i, s, m2, i2, s2);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sm[w] = m;
    ss[w] = s;
    si[w] = i;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    m = sm[0];
    s = ss[0];
    i = si[0];
    for (int q = 1; q < 4; q++) merge3(m, i, s, sm[q], si[q], ss[q]);
    const float cf = 1.f / s;
    argmax[row] = i;
    conf[row] = cf;
    if (nx.rn.canvas) {
      const int b = (int)row / nx.rn.N, p = (int)row % nx.rn.N;
      const int32_t old = nx.rn.canvas[row];
      const int32_t t = update_token(nx.rn, b, p, old, i, cf);
      nx.rn.canvas[row] = t;
      // the counters were cleared by the last layer's combine
      if (nx.rn.changed && t != old) atomicAdd(nx.rn.changed + b, 1);
      if (nx.rn.masked_left && nx.rn.mode == DG_SAMPLER_MASKED && t == nx.rn.mask_id)
        atomicAdd(nx.rn.masked_left + b, 1);
      stok = t;
    }
  }
  // the first layer's input of the updated slot for the next pass (what
  // embed_norm_k would write from the new canvas)
  if (nx.ex) {
    __syncthreads();
    const int tk = min(max(stok, 0), (int)nx.rn.V - 1);
    if (nx.act == ACT_BF16)
      embed_norm_row<uint16_t>(tk, (const uint16_t*)nx.emb, nx.g1, nx.D, nx.eps, (uint16_t*)nx.ex,
                               (uint16_t*)nx.eu, row, sm);
    else
      embed_norm_row<float>(tk, (const float*)nx.emb, nx.g1, nx.D, nx.eps, (float*)nx.ex,
                            (float*)nx.eu, row, sm);
  }
}

// ---------------------------------------------------------------------------
// weight packing: 16-byte chunk q of the packed matrix is tile q/128 (row
// group rg, 128-byte column block kb, tiles row-group-major), half h, lane l;
// it holds row 16 rg + l%16, bytes 128 kb + 64 h + 16 (l/16) of the row-major
// source; rows past the source are zero.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_k(const uint8_t* __restrict__ src, uint4* __restrict__ dst,
                                              int rows, int rowbytes, size_t nchunks) {
  const int nkb = rowbytes / 128;
  for (size_t q = (size_t)blockIdx.x * 256 + threadIdx.x; q < nchunks; q += (size_t)gridDim.x * 256) {
    const size_t tile = q >> 7;
    const int h = (int)(q >> 6) & 1, l = (int)q & 63;
    const size_t rg = tile / nkb;
    const int kb = (int)(tile % nkb);
    const size_t row = rg * 16 + (l & 15);
    const size_t col = (size_t)kb * 128 + 64 * h + 16 * (l >> 4);
    dst[q] = row < (size_t)rows ? *reinterpret_cast<const uint4*>(src + row * rowbytes + col)
                                : make_uint4(0, 0, 0, 0);
  }
}

// MXFP4 scale packing: byte q of the packed scales is tile q/128 (row group
// rg, code column block kb of 8 scale blocks), half h = (q/64) % 2, lane l =
// q % 64; it holds the scale of row 16 rg + l%16, block 8 kb + 4 h + l/16;
// rows past the source get scale 1 (code 127).
__global__ __launch_bounds__(256) void pack_mx_k(const uint8_t* __restrict__ src,
                                                 uint8_t* __restrict__ dst, int rows, int nblk,
                                                 size_t n) {
  const int nkb = nblk / 8;
  for (size_t q = (size_t)blockIdx.x * 256 + threadIdx.x; q < n; q += (size_t)gridDim.x * 256) {
    const size_t tile = q >> 7;
    const int h = (int)(q >> 6) & 1, l = (int)q & 63;
    const size_t rg = tile / nkb;
    const int kb = (int)(tile % nkb);
    const size_t row = rg * 16 + (l & 15);
    const int blk = 8 * kb + 4 * h + (l >> 4);
    dst[q] = row < (size_t)rows ? src[row * nblk + blk] : (uint8_t)127;
  }
}

// ---------------------------------------------------------------------------
void launch_embed_norm(int act, const int32_t* tok, const void* emb, const float* g, int rows, int D,
                       int V, float eps, void* x, void* u, hipStream_t s) {
  if (act == ACT_BF16)
    embed_norm_k<uint16_t><<<rows, 256, 0, s>>>(tok, (const uint16_t*)emb, g, D, V, eps,
                                                 (uint16_t*)x, (uint16_t*)u);
  else
    embed_norm_k<float><<<rows, 256, 0, s>>>(tok, (const float*)emb, g, D, V, eps, (float*)x,
                                              (float*)u);
}

void launch_rmsnorm(int act, const void* x, const float* g, int rows, int D, float eps, void* u,
                    hipStream_t s) {
  if (act == ACT_BF16)
    rmsnorm_k<uint16_t><<<rows, 256, 0, s>>>((const uint16_t*)x, g, D, eps, (uint16_t*)u);
  else
    rmsnorm_k<float><<<rows, 256, 0, s>>>((const float*)x, g, D, eps, (float*)u);
}

void launch_combine_norm(int act, const void* x1, const void* Y, const float* gates,
                         const int32_t* inv, int rows, int k, int D, const float* gnext, float eps,
                         void* x, void* u, hipStream_t s, int32_t* zero0, int32_t* zero1, int nzero) {
  if (act == ACT_BF16)
    combine_norm_k<uint16_t><<<rows, 256, 0, s>>>((const uint16_t*)x1, (const uint16_t*)Y, gates,
                                                   inv, k, D, gnext, eps, (uint16_t*)x, (uint16_t*)u,
                                                   zero0, zero1, nzero);
  else
    combine_norm_k<float><<<rows, 256, 0, s>>>((const float*)x1, (const float*)Y, gates, inv, k, D,
                                                gnext, eps, (float*)x, (float*)u, zero0, zero1, nzero);
}

void launch_renoise(int32_t* canvas, const int32_t* argmax, const float* conf, float tau,
                    uint64_t seed, uint32_t tag, const Lens& pos0, const ReqIds& req, int B, int N,
                    int V, hipStream_t s) {
  RenoiseArgs a{canvas, argmax, conf, tau, seed, tag, B, N, (uint32_t)V, pos0, req,
                DG_SAMPLER_UNIFORM, 0, 0, nullptr, nullptr};
  const int n = B * N;
  if (n == 0) return;
  renoise_k<<<(n + 255) / 256, 256, 0, s>>>(a);
}

void launch_canvas_update(const RenoiseArgs& a, hipStream_t s) {
  if (a.B > 0 && a.N > 0) canvas_update_k<<<a.B, 256, 0, s>>>(a);
}

void launch_coverage(const int32_t* counts, int L, int E, int32_t* touched, int32_t* counts_out,
                     hipStream_t s) {
  coverage_k<<<L, 256, 0, s>>>(counts, E, touched, counts_out);
}

void launch_unpermute(int act, const void* src, const int32_t* inv, int slots, int C, void* dst,
                      hipStream_t s) {
  if (act == ACT_BF16)
    unpermute_k<uint16_t><<<slots, 256, 0, s>>>((const uint16_t*)src, inv, C, (uint16_t*)dst);
  else
    unpermute_k<float><<<slots, 256, 0, s>>>((const float*)src, inv, C, (float*)dst);
}

void launch_lm_merge(const float* pmax, const int32_t* pidx, const float* psum, int rows,
                     int ntiles, int32_t* argmax, float* conf, const MergeNext& nx, hipStream_t s) {
  lm_merge_k<<<rows + (nx.touched ? nx.L : 0), 256, 0, s>>>(pmax, pidx, psum, ntiles, rows, argmax,
                                                            conf, nx);
}

void launch_pack_mx_scales(const void* src, void* dst, int rows, int nblk, hipStream_t s) {
  const size_t n = (size_t)((rows + 15) / 16) * 16 * nblk;
  const size_t blocks = (n + 255) / 256;
  pack_mx_k<<<(unsigned)(blocks < 65536 ? blocks : 65536), 256, 0, s>>>((const uint8_t*)src,
                                                                      (uint8_t*)dst, rows, nblk, n);
}

void launch_pack(const void* src, void* dst, int rows, int rowbytes, hipStream_t s) {
  const size_t nchunks = (size_t)((rows + 15) / 16) * 16 * rowbytes / 16;
  const size_t blocks = (nchunks + 255) / 256;
  pack_k<<<(unsigned)(blocks < 65536 ? blocks : 65536), 256, 0, s>>>((const uint8_t*)src, (uint4*)dst, rows,
                                                                  rowbytes, nchunks);
}

}  // namespace dg
