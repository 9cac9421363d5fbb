// Skinny GEMM on 4-bit substitute weights, on the matrix cores: Y[t][n] =
// sum_k X[t][k] (q[n][k] s + m) for t < m <= 16 positions - the draft of up to
// 16 sequences decoded together, which share the substitute weights ("SubSpec"
// report, section 10.3, item 11: cross-request sharing of the substitutes).
// The weights stream from HBM once for all positions, so the per-token weight
// traffic falls as 1/m.
//
//  * v_mfma_f32_16x16x32_bf16 with A = 16 weight rows x 32 k as (128 + q)
//    bf16 values (one and-or per pair of nibbles, exact) and B = 32 k x 16
//    positions of x.  Each MFMA's 32 k lie in one 64-group, so the group's
//    scale and min apply after its two MFMAs:
//        sum_k (q s + m) x = s * sum_k (128 + q) x + (m - 128 s) * sum_k x.
//  * Lane (r, g) of a wave (r = lane % 16: weight row, g = lane / 16) covers,
//    per 128-k chunk, k = kc + 64 h + 16 g + 8 w + j for MFMA step 2 h + w
//    (h, w in 0..1, j < 8): two 8-byte pieces of its row's codes.  Its eight
//    nibbles of a step come out as the pairs (q0, q4), (q1, q5), (q2, q6),
//    (q3, q7); the activations are staged in LDS in that same order, per
//    (step, lane group, position), so both operands agree on every k.
//  * A block of NW waves shares the staged activations; each wave owns 16
//    rows.  Narrow matrices split k over blocks (fp32 partials, summed in
//    split order by a second launch).
#include "common.h"
#include "internal.h"
#include "profile.h"

namespace {

constexpr int KC = 128;                    // k per chunk (two 64-groups)
constexpr int kBufferWord3 = 0x00020000;   // buffer resource word 3 (CDNA): raw 32-bit data
constexpr int kOutside = 0x40000000;       // offset past every resource: loads zeros
constexpr int kNonTemporal = 2;
constexpr int kTargetBlocks = 512;

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <int NW>
__global__ __launch_bounds__(NW * 64) void gemm_w4_kernel(const uint8_t* __restrict__ codes,
                                                          const uint16_t* __restrict__ meta, int64_t n, int K,
                                                          const uint16_t* __restrict__ x, int m, uint16_t* y,
                                                          float* part, int splits, int to_part) {
  // staged activations of one chunk: [step 4][lane group 4][position 16][8 bf16]
  __shared__ __align__(16) u32x4 xs[4 * 4 * 16];
  __shared__ float xsum[2][16];  // sum of x over each 64-group of the chunk, per position
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int chunks = K / KC;
  const int split = blockIdx.y;
  const int c0 = (int)((int64_t)chunks * split / splits), c1 = (int)((int64_t)chunks * (split + 1) / splits);
  const int64_t row0 = ((int64_t)blockIdx.x * NW + wave) * 16;
  const int rows = (int)std::max<int64_t>(0, std::min<int64_t>(16, n - row0));
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(codes + row0 * (K / 2)), 0, rows * (K / 2), kBufferWord3);
  const __amdgpu_buffer_rsrc_t mrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(meta + row0 * (K / 32)), 0, rows * (K / 16), kBufferWord3);
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), 0, m * K * 2, kBufferWord3);
  const uint32_t mask = __builtin_amdgcn_readfirstlane(0x000F000Fu);
  uint32_t magic = 0x43004300u;
  asm volatile("" : "+v"(magic));

  // D layout: lane holds rows 4 (lane / 16) + i of position lane % 16
  const int orow = 4 * g;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int c = c0; c < c1; ++c) {
    const int kc = c * KC;
    // this wave's codes and scale/min of the chunk (zeros past the rows)
    u32x2 piece[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      piece[h] = __builtin_amdgcn_raw_buffer_load_b64(crs, r * (K / 2) + kc / 2 + 32 * h + 8 * g, 0, kNonTemporal);
    uint32_t sm[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        sm[i][h] = __builtin_amdgcn_raw_buffer_load_b32(mrs, (orow + i) * (K / 16) + 4 * (kc / 64 + h), 0, 0);
    // stage x: thread -> (position, 8 consecutive k = one lane slot)
    __syncthreads();  // the previous chunk's reads are done
    for (int e = tid; e < 16 * 16; e += NW * 64) {
      const int pos = e >> 4, t = e & 15;  // t-th run of 8 k in the chunk
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(xrs, pos < m ? pos * K * 2 + (kc + 8 * t) * 2 : kOutside,
                                                            0, 0);
      // run t: half h = t / 8, lane group (t % 8) / 2, half-step w = t % 2
      const int h = t >> 3, gg = (t & 7) >> 1, w = t & 1, s = 2 * h + w;
      const uint32_t e0 = v.x, e1 = v.y, e2 = v.z, e3 = v.w;  // (x0,x1) (x2,x3) (x4,x5) (x6,x7)
      xs[(s * 4 + gg) * 16 + pos] = u32x4{(e0 & 0xffffu) | (e2 << 16), (e0 >> 16) | (e2 & 0xffff0000u),
                                          (e1 & 0xffffu) | (e3 << 16), (e1 >> 16) | (e3 & 0xffff0000u)};
    }
    __syncthreads();
    if (tid < 32) {  // group sums per position, from the staged values
      const int pos = tid & 15, h = tid >> 4;
      float sx = 0.0f;
#pragma unroll
      for (int w = 0; w < 2; ++w)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          const u32x4 v = xs[((2 * h + w) * 4 + gg) * 16 + pos];
          sx += ss::lo_bf(v.x) + ss::hi_bf(v.x) + ss::lo_bf(v.y) + ss::hi_bf(v.y) + ss::lo_bf(v.z) +
                ss::hi_bf(v.z) + ss::lo_bf(v.w) + ss::hi_bf(v.w);
        }
      xsum[h][pos] = sx;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const uint32_t cw = w ? piece[h].y : piece[h].x;
        const u32x4 av = u32x4{(cw & mask) | magic, ((cw >> 4) & mask) | magic, ((cw >> 8) & mask) | magic,
                               ((cw >> 12) & mask) | magic};
        const u32x4 b = xs[((2 * h + w) * 4 + g) * 16 + r];
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, b),
                                                    d, 0, 0, 0);
      }
      const float sxv = xsum[h][r];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sc = ss::h2f((uint16_t)(sm[i][h] & 0xffffu));
        const float mn = ss::h2f((uint16_t)(sm[i][h] >> 16));
        acc[i] += sc * d[i] + (mn - 128.0f * sc) * sxv;
      }
    }
  }
  // lane holds rows orow + i of position r
  if (r < m) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = row0 + orow + i;
      if (row < n) {
        if (splits > 1 || to_part)
          part[((int64_t)split * m + r) * n + row] = acc[i];
        else
          y[(int64_t)r * n + row] = ss::f2bf(acc[i]);
      }
    }
  }
}

}  // namespace

int gemm_w4_splits(int64_t n, int64_t k) {
  const int64_t groups = (n + 16 * 4 - 1) / (16 * 4);
  const int chunks = (int)(k / KC);
  if (groups >= kTargetBlocks) return 1;
  return (int)std::max<int64_t>(1, std::min<int64_t>(chunks, (kTargetBlocks + groups - 1) / groups));
}

hipError_t launch_gemm_w4(const uint8_t* codes, const uint16_t* meta, int64_t n, int64_t k, const uint16_t* x, int m,
                          uint16_t* y, float* part, hipStream_t s, int* splits_out) {
  constexpr int NW = 4;
  const int splits = gemm_w4_splits(n, k);
  const int to_part = splits_out != nullptr;
  if (to_part) *splits_out = splits;
  const dim3 grid((unsigned)((n + 16 * NW - 1) / (16 * NW)), (unsigned)splits), block(NW * 64);
  SS_LAUNCH(gemm_w4_kernel<NW>, grid, block, 0, s, codes, meta, n, (int)k, x, m, y, part, splits, to_part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1 || to_part) return e;
  return launch_gemm_reduce(part, splits, m, n, y, n, s);
}
