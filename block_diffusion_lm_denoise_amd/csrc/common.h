// common.h -- device helpers shared by the libdgpass kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
// 16 raw bytes in registers (a native vector: plain loads and stores, never
// a struct copy through private memory)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// scalar conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// round-to-nearest-even fp32 -> bf16 (NaN stays NaN): the gfx950 hardware
// conversion (v_cvt_pk_bf16_f32)
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// two values -> packed bf16 pair (lo = a, hi = b), one instruction
__device__ __forceinline__ uint32_t f2bf2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// activation storage: float or bf16 bit patterns
__device__ __forceinline__ float ldx(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float ldx(const uint16_t* p, size_t i) { return bf2f(p[i]); }
__device__ __forceinline__ void stx(float* p, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ void stx(uint16_t* p, size_t i, float v) { p[i] = f2bf(v); }
__device__ __forceinline__ float rnd(float v, const float*) { return v; }
__device__ __forceinline__ float rnd(float v, const uint16_t*) { return bf2f(f2bf(v)); }

// SwiGLU of one (gate, up) pair: silu(g) * u = g / (1 + e^-g) * u, with the
// hardware base-2 exponential and reciprocal (a few fp32 ulps, below the
// rounding of the stored result).  Very negative g: e^-g is +inf, its
// reciprocal 0, and the result a signed zero.
__device__ __forceinline__ float swiglu(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f)) * u;
}

// ---------------------------------------------------------------------------
// MFMA fragments.  A fragment is 8 consecutive contraction-dim elements of one
// matrix row held by one lane.  For a 16x16 output tile, lane l holds row
// (l % 16) and contraction chunk (l / 16); both operands use the same chunk
// assignment, so any consistent permutation of the contraction index is
// harmless.  bf16: one v_mfma_f32_16x16x32_bf16 per fragment pair; fp32: eight
// v_mfma_f32_16x16x4_f32, element j of each lane feeding the j-th.
// The accumulator (4 floats) of lane l holds rows 4*(l/16)+i, column l%16.
// ---------------------------------------------------------------------------
// tag type of MXFP4 weights (4-bit E2M1 codes, two per byte, with E8M0 block
// scales): selects the decoding code paths
struct mxfp4_t {
  uint8_t codes;
};

// E8M0 scale byte -> the fp32 power of two 2^(e - 127) (code 0: the fp32
// subnormal 2^-127)
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  return __uint_as_float(e ? (e << 23) : 0x00400000u);
}
// eight MXFP4 codes (one 32-bit word, element 2i in the low nibble of byte i)
// times their block scale -> eight bf16, exact (two significant bits times a
// power of two), four hardware conversions
__device__ __forceinline__ uint4 fp4x8_to_bf16x8(uint32_t w, float scale) {
  uint4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
  return r;
}

struct FragBF {
  bf16x8_t v;
};
struct FragF32 {
  float v[8];
};

template <typename T> struct FragOf;
template <> struct FragOf<uint16_t> { typedef FragBF type; };
template <> struct FragOf<float> { typedef FragF32 type; };

__device__ __forceinline__ void mma(f32x4_t& acc, const FragBF& a, const FragBF& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4_t& acc, const FragF32& a, const FragF32& b) {
#pragma unroll
  for (int j = 0; j < 8; j++) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], acc, 0, 0, 0);
}

// 8 elements from memory (global or LDS)
__device__ __forceinline__ void load_frag(FragBF& f, const uint16_t* p) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  f.v = __builtin_bit_cast(bf16x8_t, u);
}
__device__ __forceinline__ void load_frag(FragF32& f, const float* p) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}
__device__ __forceinline__ void zero_frag(FragBF& f) {
  f.v = __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0));
}
__device__ __forceinline__ void zero_frag(FragF32& f) {
#pragma unroll
  for (int j = 0; j < 8; j++) f.v[j] = 0.f;
}

// keep f when ok, else zero it, without a branch (a select per register)
__device__ __forceinline__ void mask_frag(FragBF& f, bool ok) {
  uint4 u = __builtin_bit_cast(uint4, f.v);
  u.x = ok ? u.x : 0u;
  u.y = ok ? u.y : 0u;
  u.z = ok ? u.z : 0u;
  u.w = ok ? u.w : 0u;
  f.v = __builtin_bit_cast(bf16x8_t, u);
}
__device__ __forceinline__ void mask_frag(FragF32& f, bool ok) {
#pragma unroll
  for (int j = 0; j < 8; j++) f.v[j] = ok ? f.v[j] : 0.f;
}

// OCP e4m3 byte pair (low or high half-word of w) -> packed bf16 pair in one
// hardware conversion (the scaled form with scale 1).  Every e4m3 value is
// exact in bf16 (4 significant bits, exponent range 2^-9 .. 448), so the
// conversion rounds nothing.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint2 u) {
  uint4 r;
  r.x = fp8x2_to_bf16x2<false>(u.x);
  r.y = fp8x2_to_bf16x2<true>(u.x);
  r.z = fp8x2_to_bf16x2<false>(u.y);
  r.w = fp8x2_to_bf16x2<true>(u.y);
  return r;
}
__device__ __forceinline__ void load_frag_fp8(FragBF& f, const uint8_t* p) {
  uint2 u = *reinterpret_cast<const uint2*>(p);
  f.v = __builtin_bit_cast(bf16x8_t, fp8x8_to_bf16x8(u));
}

// 8 consecutive activations <-> 8 floats (16 bytes bf16, 32 bytes fp32)
__device__ __forceinline__ void ld8(const uint16_t* p, float (&v)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void ld8(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void st8(uint16_t* p, const float (&v)[8]) {
  uint4 u;
  u.x = f2bf2(v[0], v[1]);
  u.y = f2bf2(v[2], v[3]);
  u.z = f2bf2(v[4], v[5]);
  u.w = f2bf2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = u;
}
__device__ __forceinline__ void st8(float* p, const float (&v)[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// ---------------------------------------------------------------------------
// the value of lane l ^ 16 / l ^ 32 of a wave.  The gfx950 permlane swaps
// exchange 16-lane rows between two registers in the VALU (no LDS round trip
// as with ds_bpermute): with both operands x, lanes of an even row receive
// the next row's x in the second result and lanes of an odd row the previous
// row's x in the first (permlane32: the same for the two halves of the wave).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t lane_xor16(uint32_t x) {
  const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return (threadIdx.x & 16) ? p[0] : p[1];
}
__device__ __forceinline__ uint32_t lane_xor32(uint32_t x) {
  const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return (threadIdx.x & 32) ? p[0] : p[1];
}
__device__ __forceinline__ float lane_xor16(float x) { return __uint_as_float(lane_xor16(__float_as_uint(x))); }
__device__ __forceinline__ float lane_xor32(float x) { return __uint_as_float(lane_xor32(__float_as_uint(x))); }
__device__ __forceinline__ int lane_xor16(int x) { return (int)lane_xor16((uint32_t)x); }
__device__ __forceinline__ int lane_xor32(int x) { return (int)lane_xor32((uint32_t)x); }
// Symmetric reductions over a lane and its partner 16 (32) lanes apart, the
// result in both: the swap of two copies of x leaves rows (0, 0, 2, 2) in one
// and rows (1, 1, 3, 3) in the other (for 32: (0, 1, 0, 1) and (2, 3, 2, 3)),
// so an operation on the pair needs no lane select.
// (max_nn and max3_nn are inline assembly: the compiler does not see which
// registers they read, so it inserts no wait states for a matrix-core result
// read too early -- never pass them an MFMA accumulator; fmax3 below is the
// compiler-visible form for those)
__device__ __forceinline__ float max_nn(float a, float b) {   // non-NaN operands, no quieting
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float pair_max16(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_nn(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float pair_max32(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_nn(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float pair_sum16(float x) {   // row r + row r^1, the lower row first
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float pair_sum32(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ int pair_min16(int x) {
  const auto p = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
  return min((int)p[0], (int)p[1]);
}
__device__ __forceinline__ int pair_min32(int x) {
  const auto p = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
  return min((int)p[0], (int)p[1]);
}

// ---------------------------------------------------------------------------
// wave / block reductions (wave64)
// ---------------------------------------------------------------------------

// reductions over the 16 lanes of a DPP row (lanes 16j .. 16j+15) with DPP
// moves: two quad permutations, then the half-row and row mirrors.  Max and
// min are exact; each lane's sum may round differently, so a sum is read from
// one lane only.
template <int CTRL> __device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
template <int CTRL> __device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}
constexpr int DPP_QUAD_1032 = 0xB1, DPP_QUAD_2301 = 0x4E, DPP_ROW_HALF_MIRROR = 0x141,
              DPP_ROW_MIRROR = 0x140;
__device__ __forceinline__ float fmax_sel(float a, float b) { return b > a ? b : a; }   // no NaN canonicalising
// maximum of three non-NaN floats in one VALU instruction (the builtin max
// quiets its inputs first; these operands are never NaN)
__device__ __forceinline__ float max3_nn(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// maximum of three floats, compiler-visible (one v_max3 for operands the
// compiler knows are canonical, e.g. matrix-core results), so the hazard
// recognizer orders it after the MFMAs that produce its operands
__device__ __forceinline__ float fmax3(float a, float b, float c) {
  return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmax_sel(v, dpp_f<DPP_QUAD_1032>(v));
  v = fmax_sel(v, dpp_f<DPP_QUAD_2301>(v));
  v = fmax_sel(v, dpp_f<DPP_ROW_HALF_MIRROR>(v));
  return fmax_sel(v, dpp_f<DPP_ROW_MIRROR>(v));
}
__device__ __forceinline__ int row16_min(int v) {
  v = min(v, dpp_i<DPP_QUAD_1032>(v));
  v = min(v, dpp_i<DPP_QUAD_2301>(v));
  v = min(v, dpp_i<DPP_ROW_HALF_MIRROR>(v));
  return min(v, dpp_i<DPP_ROW_MIRROR>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<DPP_QUAD_1032>(v);
  v += dpp_f<DPP_QUAD_2301>(v);
  v += dpp_f<DPP_ROW_HALF_MIRROR>(v);
  return v + dpp_f<DPP_ROW_MIRROR>(v);
}

// sums / maxima over the wave (every lane gets the result): DPP within the
// 16-lane rows, then the permlane swaps across rows and wave halves
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  v += lane_xor16(v);
  return v + lane_xor32(v);
}
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  v = fmax_sel(v, lane_xor16(v));
  return fmax_sel(v, lane_xor32(v));
}

// max of a 64-bit value over the wave (every lane gets it): DPP within the
// 16-lane rows, then the four row results read as scalars
template <int CTRL> __device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const int lo = dpp_i<CTRL>((int)(uint32_t)v), hi = dpp_i<CTRL>((int)(uint32_t)(v >> 32));
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = umax64(v, dpp_u64<DPP_QUAD_1032>(v));
  v = umax64(v, dpp_u64<DPP_QUAD_2301>(v));
  v = umax64(v, dpp_u64<DPP_ROW_HALF_MIRROR>(v));
  v = umax64(v, dpp_u64<DPP_ROW_MIRROR>(v));
  return umax64(umax64(readlane_u64(v, 0), readlane_u64(v, 16)),
                umax64(readlane_u64(v, 32), readlane_u64(v, 48)));
}

// deterministic block sum for blockDim.x == 256 (4 waves); red: >= 4 floats of LDS
__device__ __forceinline__ float block_sum256(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// ---------------------------------------------------------------------------
// direct loads into LDS (gfx950 global_load_lds, 16 bytes per lane: lane i
// writes lds_wave_base + 16 i) and their waits
// ---------------------------------------------------------------------------
__device__ __forceinline__ void lds_dma16(const void* g, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}
// a pointer the whole wave holds, in scalar registers
__device__ __forceinline__ const char* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
// wait until at most n vector-memory loads of this wave are outstanding (gfx9
// s_waitcnt encoding: vmcnt low bits [3:0] and high bits [15:14]; expcnt and
// lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace dg
