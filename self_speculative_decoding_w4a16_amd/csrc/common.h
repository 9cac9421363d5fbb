// Shared device helpers for the gfx950 kernels of libsubspec.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define SS_WAVE 64

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

namespace ss {

// ---------------------------------------------------------------- bf16 / fp16
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bf16, round to nearest even; NaN stays a NaN (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf(uint16_t lo, uint16_t hi) {
  return (uint32_t)lo | ((uint32_t)hi << 16);
}

__device__ __forceinline__ float h2f(uint16_t h) {
  _Float16 v = __builtin_bit_cast(_Float16, h);
  return (float)v;
}
__device__ __forceinline__ uint16_t f2h_sat(float f) {
  f = fminf(fmaxf(f, -65504.0f), 65504.0f);
  _Float16 v = (_Float16)f;
  return __builtin_bit_cast(uint16_t, v);
}

// fp32 accumulate of two bf16 products: acc + a.x*b.x + a.y*b.y
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, SS_WAVE);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, SS_WAVE));
  return v;
}

// (value, index) max with the lowest index winning ties.  Non-finite logits
// (NaN, +-Inf) carry no probability and never win: cand() turns them into the
// empty candidate {-inf, kNoIndex}, which every finite value beats; a
// reduction that ends on kNoIndex had no finite value (token 0 by convention,
// see argmax_token).
constexpr int kNoIndex = 0x7fffffff;
struct ArgMax {
  float v;
  int i;
};
__device__ __forceinline__ bool finite(float v) { return fabsf(v) < INFINITY; }
__device__ __forceinline__ ArgMax cand(float v, int i) {
  return finite(v) ? ArgMax{v, i} : ArgMax{-INFINITY, kNoIndex};
}
__device__ __forceinline__ int argmax_token(const ArgMax& a) { return a.i == kNoIndex ? 0 : a.i; }
__device__ __forceinline__ ArgMax better(ArgMax a, ArgMax b) {
  if (b.v > a.v || (b.v == a.v && b.i < a.i)) return b;
  return a;
}
__device__ __forceinline__ ArgMax wave_argmax(ArgMax a) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    ArgMax b;
    b.v = __shfl_xor(a.v, o, SS_WAVE);
    b.i = __shfl_xor(a.i, o, SS_WAVE);
    a = better(a, b);
  }
  return a;
}

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, SS_WAVE);
  return v;
}

// ------------------------------------------------------- exact sampling weights
// w = exp(fl32(fl32(z - M) / T)) in float32, then W = floor(w * 2^40) as an
// integer, so that every later sum and comparison is exact and order-free.
// M is the largest finite logit of the row; a non-finite z has weight 0.
__device__ __forceinline__ unsigned long long fixed_weight(float z, float M, float T) {
  const bool f = finite(z);
  float t = __fdiv_rn(__fsub_rn(f ? z : M, M), T);
  float w = fminf(fmaxf(expf(t), 0.0f), 1.0f);  // z <= M: no change; a NaN (M = -inf) becomes 0
  const unsigned long long W = (unsigned long long)((double)w * 1099511627776.0);
  return f ? W : 0ull;
}

// 128-bit unsigned helpers for the exact accept test.
struct U128 {
  unsigned long long hi, lo;
};
__device__ __forceinline__ U128 mul64(unsigned long long a, unsigned long long b) {
  U128 r;
  r.lo = a * b;
  r.hi = __umul64hi(a, b);
  return r;
}
__device__ __forceinline__ U128 shl128(U128 a, int s) {  // 0 < s < 64
  U128 r;
  r.hi = (a.hi << s) | (a.lo >> (64 - s));
  r.lo = a.lo << s;
  return r;
}
__device__ __forceinline__ bool lt128(U128 a, U128 b) {
  return a.hi < b.hi || (a.hi == b.hi && a.lo < b.lo);
}
__device__ __forceinline__ U128 sub128(U128 a, U128 b) {
  U128 r;
  r.lo = a.lo - b.lo;
  r.hi = a.hi - b.hi - (a.lo < b.lo ? 1ull : 0ull);
  return r;
}
__device__ __forceinline__ unsigned long long shr128(U128 a, int s) {  // result must fit 64 bits
  if (s == 0) return a.lo;
  if (s >= 64) return a.hi >> (s - 64);
  return (a.lo >> s) | (a.hi << (64 - s));
}

// Residual weight max(0, Wt*Sd - Wd*St) >> shift (exact, 128-bit products).
__device__ __forceinline__ unsigned long long resid_w(unsigned long long Wt, unsigned long long Sd,
                                                      unsigned long long Wd, unsigned long long St,
                                                      int shift) {
  const U128 a = mul64(Wt, Sd), b = mul64(Wd, St);
  if (!lt128(b, a)) return 0ull;
  return shr128(sub128(a, b), shift);
}

// bit length of v minus one; 0 for v = 0 (a draft row without mass)
__device__ __forceinline__ int bitlen_minus1(unsigned long long v) { return v ? 63 - __clzll(v) : 0; }

}  // namespace ss
