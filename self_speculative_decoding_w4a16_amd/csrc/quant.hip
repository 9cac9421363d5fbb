// 4-bit substitute construction: uniform asymmetric group-64 quantisation of a
// bf16 weight matrix (the target's own layer at low precision, built without
// calibration data - "SubSpec: Speculate Deep and Accurate" paper note,
// Method details; 4 bits per "SubSpec" report section 2.2).
//
// One thread per (row, 64-group): it reads the 128 bytes of its group with
// 16-byte loads, finds lo/hi, stores the fp16 {scale, min} and the 32 code
// bytes.  The scale is rounded up where rounding to nearest would leave
// 15 s below the span, so every weight is within s/2 of its level.  Every operation that decides a code is a single correctly rounded
// float32 operation (no contraction), so codes are reproducible bit for bit.
#include "common.h"
#include "internal.h"
#include "profile.h"

#pragma clang fp contract(off)

namespace {

__global__ __launch_bounds__(256) void w4_quantize_kernel(const uint16_t* __restrict__ w,
                                                          int64_t n, int64_t k,
                                                          uint8_t* __restrict__ codes,
                                                          uint16_t* __restrict__ meta) {
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
  uint16_t s16 = ss::f2h_sat(__fdiv_rn(span, 15.0f));
  // the 16 levels must reach hi: the smallest fp16 scale with 15 s >= span
  // (15 s is exact in float32; s >= 0, so the next fp16 value up is s16 + 1)
  if (__fmul_rn(ss::h2f(s16), 15.0f) < span && s16 < 0x7bffu) s16 = (uint16_t)(s16 + 1u);
  if ((s16 & 0x7fffu) == 0) s16 = 0x3c00u;  // scale 0 -> 1.0
  const uint16_t m16 = ss::f2h_sat(lo);
  const float s = ss::h2f(s16), m = ss::h2f(m16);

  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float xs[2] = {ss::lo_bf(v[i]), ss::hi_bf(v[i])};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float t = __fdiv_rn(__fsub_rn(xs[h], m), s);
      float r = rintf(t);
      r = fminf(fmaxf(r, 0.0f), 15.0f);
      const int kk = 2 * i + h;  // position inside the group
      out[kk >> 3] |= (uint32_t)r << (4 * (kk & 7));
    }
  }
  uint4* dst = reinterpret_cast<uint4*>(codes + row * (k / 2) + g * 32);
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
  reinterpret_cast<uint32_t*>(meta)[row * groups_per_row + g] = ss::pack_bf(s16, m16);
}

}  // namespace

hipError_t launch_w4_quantize(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes,
                              uint16_t* meta, hipStream_t s) {
  const int64_t total = n * (k / 64);
  const int64_t blocks = (total + 255) / 256;
  SS_LAUNCH(w4_quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, s, w, n, k, codes,
                     meta);
  return hipGetLastError();
}
