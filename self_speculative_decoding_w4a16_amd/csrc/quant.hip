// Substitute construction: uniform asymmetric group-64 quantisation of a bf16
// weight matrix at 4, 3 or 2 bits (the target's own layer at low precision,
// built without calibration data - "SubSpec: Speculate Deep and Accurate"
// paper note, Method details, at 2/3 bits; 4 bits per the "SubSpec" report,
// section 2.2).
//
// One thread per (row, 64-group): it reads the 128 bytes of its group with
// 16-byte loads, finds lo/hi, stores the fp16 {scale, min} and the group's
// codes.  Every operation that decides a code is a single correctly rounded
// float32 operation (no contraction), so codes are reproducible bit for bit.
// The scale is rounded up where rounding to nearest would leave L s below
// the span (L = 2^bits - 1), so every weight is within s/2 of its level.
//
// Code layouts per row: 4 bits two codes a byte (low nibble first); 2 bits
// four codes a byte (lowest bits first); 3 bits the 2-bit plane of the low
// two bits (K/4 bytes), then the third bits (K/8 bytes) in 4-byte words of 32
// weights whose bytes hold weights 0-7, 16-23, 8-15, 24-31 of the word.
#include "common.h"
#include "internal.h"
#include "profile.h"

#pragma clang fp contract(off)

namespace {

template <int BITS>
__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* __restrict__ w, int64_t n, int64_t k,
                                                       uint8_t* __restrict__ codes, uint16_t* __restrict__ meta) {
  constexpr int L = (1 << BITS) - 1;
  const int64_t groups_per_row = k / 64;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n * groups_per_row) return;
  const int64_t row = gid / groups_per_row;
  const int64_t g = gid - row * groups_per_row;
  const uint4* src = reinterpret_cast<const uint4*>(w + row * k + g * 64);

  uint32_t v[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint4 q = src[i];
    v[4 * i + 0] = q.x;
    v[4 * i + 1] = q.y;
    v[4 * i + 2] = q.z;
    v[4 * i + 3] = q.w;
  }
  float lo = ss::lo_bf(v[0]), hi = lo;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float a = ss::lo_bf(v[i]), b = ss::hi_bf(v[i]);
    lo = fminf(lo, fminf(a, b));
    hi = fmaxf(hi, fmaxf(a, b));
  }
  const float span = __fsub_rn(hi, lo);
  uint16_t s16 = ss::f2h_sat(__fdiv_rn(span, (float)L));
  // the levels must reach hi: the smallest fp16 scale with L s >= span
  // (L s is exact in float32; s >= 0, so the next fp16 value up is s16 + 1)
  if (__fmul_rn(ss::h2f(s16), (float)L) < span && s16 < 0x7bffu) s16 = (uint16_t)(s16 + 1u);
  if ((s16 & 0x7fffu) == 0) s16 = 0x3c00u;  // scale 0 -> 1.0
  const uint16_t m16 = ss::f2h_sat(lo);
  const float s = ss::h2f(s16), m = ss::h2f(m16);

  uint32_t q[64];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float xs[2] = {ss::lo_bf(v[i]), ss::hi_bf(v[i])};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float t = __fdiv_rn(__fsub_rn(xs[h], m), s);
      q[2 * i + h] = (uint32_t)fminf(fmaxf(rintf(t), 0.0f), (float)L);
    }
  }
  reinterpret_cast<uint32_t*>(meta)[row * groups_per_row + g] = ss::pack_bf(s16, m16);
  if (BITS == 4) {
    uint32_t out[8] = {};
#pragma unroll
    for (int kk = 0; kk < 64; ++kk) out[kk >> 3] |= q[kk] << (4 * (kk & 7));
    uint4* dst = reinterpret_cast<uint4*>(codes + row * (k / 2) + g * 32);
    dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
    dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
    return;
  }
  // the 2-bit plane (the whole code at 2 bits, its low two bits at 3)
  uint32_t lo2[4] = {};
#pragma unroll
  for (int kk = 0; kk < 64; ++kk) lo2[kk >> 4] |= (q[kk] & 3u) << (2 * (kk & 15));
  const int64_t rb = BITS == 2 ? k / 4 : 3 * k / 8;
  *reinterpret_cast<uint4*>(codes + row * rb + g * 16) = make_uint4(lo2[0], lo2[1], lo2[2], lo2[3]);
  if (BITS == 3) {
    constexpr int kFirst[4] = {0, 16, 8, 24};  // first weight of each byte of a 32-weight word
    uint32_t hw[2] = {};
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int t = 0; t < 8; ++t) hw[h] |= ((q[32 * h + kFirst[b] + t] >> 2) & 1u) << (8 * b + t);
    *reinterpret_cast<uint2*>(codes + row * rb + k / 4 + g * 8) = make_uint2(hw[0], hw[1]);
  }
}

}  // namespace

hipError_t launch_quantize(const uint16_t* w, int64_t n, int64_t k, int bits, uint8_t* codes, uint16_t* meta,
                           hipStream_t s) {
  const int64_t total = n * (k / 64);
  const dim3 grid((unsigned)((total + 255) / 256)), block(256);
  switch (bits) {
    case 4: SS_LAUNCH(quantize_kernel<4>, grid, block, 0, s, w, n, k, codes, meta); break;
    case 3: SS_LAUNCH(quantize_kernel<3>, grid, block, 0, s, w, n, k, codes, meta); break;
    case 2: SS_LAUNCH(quantize_kernel<2>, grid, block, 0, s, w, n, k, codes, meta); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
