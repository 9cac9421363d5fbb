// Skinny GEMM on 4-bit substitute weights, on the matrix cores: Y[t][n] =
// sum_k X[t][k] (q[n][k] s + m) for t < m <= 16 positions - the draft of up to
// 16 sequences decoded together, which share the substitute weights ("SubSpec"
// report, section 10.3, item 11: cross-request sharing of the substitutes),
// and the k chains of a static tree's draft level.  The weights stream from
// HBM once for all positions, so the per-token weight traffic falls as 1/m.
//
//  * v_mfma_f32_16x16x32_bf16 with A = 16 positions x 32 k of x and B = 32 k
//    x 16 weight rows as (128 + q) bf16 values (one and-or per pair of
//    nibbles, exact).  Each MFMA's 32 k lie in one 64-group, so the group's
//    scale and min apply after its two MFMAs:
//        sum_k (q s + m) x = s * sum_k (128 + q) x + (m - 128 s) * sum_k x,
//    the group sums of x coming from two more MFMAs with B = ones.
//  * Lane (r, g) of a wave (r = lane % 16, g = lane / 16) covers, per
//    128-k chunk, k = kc + 64 h + 16 g + 8 w + j for MFMA step 2 h + w (h, w
//    in 0..1, j < 8): for each of the wave's RT tiles of 16 weight rows, two
//    8-byte pieces of the codes of tile row r, whose eight nibbles of a step
//    come out as the pairs (q0, q4), (q1, q5), (q2, q6), (q3, q7); the same
//    lane loads the activations of position r at those k straight from
//    memory (x is small and stays in the caches), pairs them the same way,
//    and uses them for all RT tiles - so no LDS and no barrier.
//  * A = activations, B = weights: lane (r, g) of tile t ends with
//    positions 4 g + i of the tile's row r, so it applies only its own row's
//    scale/min (one 8-byte load per tile and chunk).
//  * Pipeline: the codes, scale/min pairs and activations of WD chunks are
//    in flight per lane (register slots named statically, every load
//    unconditional: offsets outside a buffer resource read zeros).
//  * One wave per block, 16 RT rows; narrow matrices split k over blocks
//    (fp32 partials, summed in split order by a second launch or by the
//    caller's consumer).
#include "common.h"
#include "internal.h"
#include "profile.h"

namespace {

constexpr int KC = 128;                    // k per chunk (two 64-groups)
constexpr int RT = 4;                      // tiles of 16 weight rows per wave
constexpr int WD = 2;                      // chunks in flight per lane
constexpr int kBufferWord3 = 0x00020000;   // buffer resource word 3 (CDNA): raw 32-bit data
constexpr int kOutside = 0x40000000;       // offset past every resource: loads zeros
constexpr int kTargetBlocks = 512;

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

struct Slot {
  u32x2 pc[RT][2];  // codes of the chunk's two groups, row r of each tile
  u32x2 mt[RT];     // scale/min of the two groups, row r of each tile
  u32x4 xv[4];      // activations of position r for the four MFMA steps
};

__global__ __launch_bounds__(64) void gemm_w4_kernel(const uint8_t* __restrict__ codes,
                                                     const uint16_t* __restrict__ meta, int64_t n, int K,
                                                     const uint16_t* __restrict__ x, int m, uint16_t* y,
                                                     float* part, int splits, int to_part) {
  const int lane = threadIdx.x;
  const int r = lane & 15, g = lane >> 4;
  const int chunks = K / KC;
  const int split = blockIdx.y;
  const int c0 = (int)((int64_t)chunks * split / splits), c1 = (int)((int64_t)chunks * (split + 1) / splits);
  const int64_t row0 = (int64_t)blockIdx.x * 16 * RT;
  const int rows = (int)std::max<int64_t>(0, std::min<int64_t>(16 * RT, n - row0));
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(codes + row0 * (K / 2)), 0, rows * (K / 2), kBufferWord3);
  const __amdgpu_buffer_rsrc_t mrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(meta + row0 * (K / 32)), 0, rows * (K / 16), kBufferWord3);
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), 0, m * K * 2, kBufferWord3);
  const uint32_t mask = __builtin_amdgcn_readfirstlane(0x000F000Fu);
  uint32_t magic = 0x43004300u;
  asm volatile("" : "+v"(magic));
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0 pairs
  const int xbase = r < m ? r * K * 2 : kOutside;

  // the loads of chunk c (zeros past the block's range)
  auto load_chunk = [&](int c, Slot& sl) {
    const bool in = c < c1;
    const int kc = c * KC;
#pragma unroll
    for (int st = 0; st < 4; ++st)  // step 2 h + w: k = kc + 64 h + 16 g + 8 w .. + 7
      sl.xv[st] = __builtin_amdgcn_raw_buffer_load_b128(
          xrs, in ? xbase + (kc + 64 * (st >> 1) + 16 * g + 8 * (st & 1)) * 2 : kOutside, 0, 0);
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int rr = 16 * t + r;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        sl.pc[t][h] =
            __builtin_amdgcn_raw_buffer_load_b64(crs, in ? rr * (K / 2) + kc / 2 + 32 * h + 8 * g : kOutside, 0, 0);
      sl.mt[t] = __builtin_amdgcn_raw_buffer_load_b64(mrs, in ? rr * (K / 16) + 4 * (kc / 64) : kOutside, 0, 0);
    }
  };
  f32x4_t acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const Slot& sl) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 b[2];
      f32x4_t ds = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const u32x4 v = sl.xv[2 * h + w];  // (x0,x1) (x2,x3) (x4,x5) (x6,x7) -> (x0,x4) (x1,x5) (x2,x6) (x3,x7)
        b[w] = u32x4{(v.x & 0xffffu) | (v.z << 16), (v.x >> 16) | (v.z & 0xffff0000u),
                     (v.y & 0xffffu) | (v.w << 16), (v.y >> 16) | (v.w & 0xffff0000u)};
        ds = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, b[w]),
                                                     __builtin_bit_cast(bf16x8_t, ones), ds, 0, 0, 0);
      }
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const uint32_t cw = w ? sl.pc[t][h].y : sl.pc[t][h].x;
          const u32x4 av = u32x4{(cw & mask) | magic, ((cw >> 4) & mask) | magic, ((cw >> 8) & mask) | magic,
                                 ((cw >> 12) & mask) | magic};
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, b[w]),
                                                      __builtin_bit_cast(bf16x8_t, av), d, 0, 0, 0);
        }
        const uint32_t smw = h ? sl.mt[t].y : sl.mt[t].x;
        const float sc = ss::h2f((uint16_t)(smw & 0xffffu));
        const float mn = ss::h2f((uint16_t)(smw >> 16));
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][i] += sc * d[i] + (mn - 128.0f * sc) * ds[i];
      }
    }
  };

  Slot sl[WD];
#pragma unroll
  for (int j = 0; j < WD; ++j) load_chunk(c0 + j, sl[j]);
  // chunk c lives in slot (c - c0) % WD; scheduling barriers keep each
  // step's instructions in it, so its wait covers only that chunk's loads
  auto step = [&](int c, int j) {
    __builtin_amdgcn_sched_barrier(0);
    compute(sl[j]);
    load_chunk(c + WD, sl[j]);
    __builtin_amdgcn_sched_barrier(0);
  };
  int c = c0;
  for (; c + WD <= c1; c += WD) {
#pragma unroll
    for (int j = 0; j < WD; ++j) step(c + j, j);
  }
#pragma unroll
  for (int j = 0; j < WD - 1; ++j)
    if (c + j < c1) step(c + j, j);

  // lane holds positions 4 g + i of row r of each tile
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int64_t row = row0 + 16 * t + r;
    if (row >= n) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pos = 4 * g + i;
      if (pos < m) {
        if (splits > 1 || to_part)
          part[((int64_t)split * m + pos) * n + row] = acc[t][i];
        else
          y[(int64_t)pos * n + row] = ss::f2bf(acc[t][i]);
      }
    }
  }
}

}  // namespace

int gemm_w4_splits(int64_t n, int64_t k) {
  const int64_t groups = (n + 16 * RT - 1) / (16 * RT);
  const int chunks = (int)(k / KC);
  if (groups >= kTargetBlocks) return 1;
  return (int)std::max<int64_t>(1, std::min<int64_t>(chunks, (kTargetBlocks + groups - 1) / groups));
}

hipError_t launch_gemm_w4(const uint8_t* codes, const uint16_t* meta, int64_t n, int64_t k, const uint16_t* x, int m,
                          uint16_t* y, float* part, hipStream_t s, int* splits_out) {
  const int splits = gemm_w4_splits(n, k);
  const int to_part = splits_out != nullptr;
  if (to_part) *splits_out = splits;
  const dim3 grid((unsigned)((n + 16 * RT - 1) / (16 * RT)), (unsigned)splits), block(64);
  SS_LAUNCH(gemm_w4_kernel, grid, block, 0, s, codes, meta, n, (int)k, x, m, y, part, splits, to_part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1 || to_part) return e;
  return launch_gemm_reduce(part, splits, m, n, y, n, s);
}
