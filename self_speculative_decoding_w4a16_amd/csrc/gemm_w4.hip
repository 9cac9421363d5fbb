// Skinny GEMM on 4-bit substitute weights, on the matrix cores: Y[t][n] =
// sum_k X[t][k] (q[n][k] s + m) for t < m <= 16 positions - the draft of up to
// 16 sequences decoded together, which share the substitute weights ("SubSpec"
// report, section 10.3, item 11: cross-request sharing of the substitutes),
// and the k chains of a static tree's draft level.  The weights stream from
// HBM once for all positions, so the per-token weight traffic falls as 1/m.
//
//  * v_mfma_f32_16x16x32_bf16 with A = 16 positions x 32 k of x and B = 32 k
//    x 16 weight rows as (128 + q) bf16 values (one and-or per pair of
//    nibbles, exact), with the group's scale and min applied to the sums of
//    its k:
//        sum_k (q s + m) x = s * sum_k (128 + q) x + (m - 128 s) * sum_k x,
//    the group sums of x coming from MFMAs with B = ones.
//  * Lane (r, g) of a wave (r = lane % 16, g = lane / 16) loads, per 128-k
//    chunk (two 64-groups) and for each of the wave's RT tiles of 16 weight
//    rows, the 16 code bytes 16 g .. 16 g + 15 of the chunk in tile row r
//    (so one load instruction reads 16 rows x 64 contiguous bytes), i.e.
//    k = kc + 32 g + 8 st + j for MFMA step st < 4, j < 8; a code word's
//    eight nibbles come out as the pairs (q0, q4), (q1, q5), (q2, q6),
//    (q3, q7).  The same lane loads the activations of position r at those k
//    straight from memory (x is small and stays in the caches), pairs them
//    the same way, and uses them for all RT tiles - so no LDS and no barrier.
//  * Lanes g = 0, 1 hold the chunk's first group and g = 2, 3 its second.
//    Up to 8 positions, A row p holds position p on the first group's
//    lanes and row 8 + p on the second's (every other A value zero), so one
//    MFMA per tile and step yields both groups' sums in separate D rows and
//    a lane scales its four values with one group's scale/min; the two
//    halves of each sum meet by a lane swap at the end.  Past 8 positions
//    every step runs two MFMAs per tile, one with the activations of the
//    second group's lanes zeroed and one with the first group's zeroed.
//  * A = activations, B = weights: lane (r, g) of tile t ends with
//    positions 4 g + i of the tile's row r, so it applies only its own row's
//    scale/min (one 8-byte load per tile and chunk).
//  * The gate/up projection can end in SiLU(gate) * up: its blocks then take
//    RT/2 tiles of gate rows and the RT/2 tiles of the matching up rows, so a
//    lane holds both factors of its outputs.
//  * Pipeline: the codes, scale/min pairs and activations of WD chunks are
//    in flight per lane (register slots named statically, every load
//    unconditional: offsets outside a buffer resource read zeros).
//  * One wave per block, 16 RT rows; narrow matrices split k over blocks
//    (fp32 partials, summed in split order by a second launch or by the
//    caller's consumer).
//  * Codes and meta row-major (subspec_quantize) or in 16-row tiles
//    (subspec_tile_codes): the lane reads the same 16 bytes and scale/min pair
//    either way, from one contiguous KiB per tile and chunk in the tiled
//    layout.
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
  u32x4 pc[RT];  // 16 code bytes of the chunk, row r of each tile
  u32x2 mt[RT];  // scale/min of the chunk's two groups, row r of each tile
  u32x4 xv[4];   // activations of position r for the four MFMA steps
};

// SILU: the gate/up projection (n = 2 silu_f rows) ending in SiLU(gate) * up;
// TL: tiled codes and meta; HALF: m <= 8 (one MFMA per tile and step)
template <bool SILU, bool TL, bool HALF>
__global__ __launch_bounds__(64) void gemm_w4_kernel(const uint8_t* __restrict__ codes,
                                                     const uint16_t* __restrict__ meta, int64_t n, int K,
                                                     const uint16_t* __restrict__ x, int m, uint16_t* y,
                                                     float* part, int splits, int to_part, int64_t silu_f) {
  const int lane = threadIdx.x;
  const int r = lane & 15, g = lane >> 4;
  const int chunks = K / KC;
  const int split = blockIdx.y;
  const int c0 = (int)((int64_t)chunks * split / splits), c1 = (int)((int64_t)chunks * (split + 1) / splits);
  // rows row0 + 16 t + r of tile t; with SILU the first RT/2 tiles are gate
  // rows from row0 and the others the matching up rows, silu_f rows further
  // (one resource spans both)
  constexpr int HT = RT / 2;
  const int64_t row0 = (int64_t)blockIdx.x * 16 * (SILU ? HT : RT);
  const int rows = (int)std::max<int64_t>(0, std::min<int64_t>(SILU ? silu_f + 16 * HT : 16 * RT, n - row0));
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
  // HALF: A row r is position r & 7 of the first group (r < 8: lanes g < 2)
  // or of the second (r >= 8: lanes g >= 2); other lanes read zeros
  const int xpos = HALF ? (r & 7) : r;
  const bool xreal = HALF ? (xpos < m && (r < 8) == (g < 2)) : r < m;
  const int xbase = xreal ? xpos * K * 2 : kOutside;

  // the loads of chunk c (zeros past the block's range)
  auto load_chunk = [&](int c, Slot& sl) {
    const bool in = c < c1;
    const int kc = c * KC;
#pragma unroll
    for (int st = 0; st < 4; ++st)  // step st: k = kc + 32 g + 8 st .. + 7
      sl.xv[st] = __builtin_amdgcn_raw_buffer_load_b128(xrs, in ? xbase + (kc + 32 * g + 8 * st) * 2 : kOutside, 0, 0);
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int rr = (SILU && t >= HT) ? (int)silu_f + 16 * (t - HT) + r : 16 * t + r;
      if constexpr (TL) {  // rows rr - r .. rr - r + 15 form one tile (silu_f % 16 == 0)
        const int tb = (rr >> 4) * (K / KC) + kc / KC;
        sl.pc[t] = __builtin_amdgcn_raw_buffer_load_b128(crs, in ? tb * 1024 + 16 * lane : kOutside, 0, 0);
        sl.mt[t] = __builtin_amdgcn_raw_buffer_load_b64(mrs, in ? tb * 128 + 8 * r : kOutside, 0, 0);
      } else {
        sl.pc[t] = __builtin_amdgcn_raw_buffer_load_b128(crs, in ? rr * (K / 2) + kc / 2 + 16 * g : kOutside, 0, 0);
        sl.mt[t] = __builtin_amdgcn_raw_buffer_load_b64(mrs, in ? rr * (K / 16) + 4 * (kc / 64) : kOutside, 0, 0);
      }
    }
  };
  f32x4_t acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const bool first = g < 2;  // this lane's k lie in the chunk's first group
  auto compute_half = [&](const Slot& sl) {
    const f32x4_t zf = {0.f, 0.f, 0.f, 0.f};
    f32x4_t sx = zf, d[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) d[t] = zf;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const u32x4 v = sl.xv[st];  // (x0,x1) (x2,x3) (x4,x5) (x6,x7) -> (x0,x4) (x1,x5) (x2,x6) (x3,x7)
      const bf16x8_t a = __builtin_bit_cast(
          bf16x8_t, u32x4{(v.x & 0xffffu) | (v.z << 16), (v.x >> 16) | (v.z & 0xffff0000u),
                          (v.y & 0xffffu) | (v.w << 16), (v.y >> 16) | (v.w & 0xffff0000u)});
      sx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, ones), sx, 0, 0, 0);
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const uint32_t cw = sl.pc[t][st];
        const bf16x8_t av = __builtin_bit_cast(
            bf16x8_t, u32x4{(cw & mask) | magic, ((cw >> 4) & mask) | magic, ((cw >> 8) & mask) | magic,
                            ((cw >> 12) & mask) | magic});
        d[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, av, d[t], 0, 0, 0);
      }
    }
    // lane (r, g) holds D rows 4 g .. 4 g + 3: its own group's sums
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const uint32_t mw = first ? sl.mt[t].x : sl.mt[t].y;
      const float sc = ss::h2f((uint16_t)(mw & 0xffffu)), mn = ss::h2f((uint16_t)(mw >> 16));
      const float c0 = mn - 128.0f * sc;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[t][i] += sc * d[t][i] + c0 * sx[i];
    }
  };
  auto compute = [&](const Slot& sl) {
    if constexpr (HALF) {
      compute_half(sl);
      return;
    }
    const f32x4_t zf = {0.f, 0.f, 0.f, 0.f};
    f32x4_t s0 = zf, s1 = zf, d0[RT], d1[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) d0[t] = d1[t] = zf;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const u32x4 v = sl.xv[st];  // (x0,x1) (x2,x3) (x4,x5) (x6,x7) -> (x0,x4) (x1,x5) (x2,x6) (x3,x7)
      const u32x4 b = u32x4{(v.x & 0xffffu) | (v.z << 16), (v.x >> 16) | (v.z & 0xffff0000u),
                            (v.y & 0xffffu) | (v.w << 16), (v.y >> 16) | (v.w & 0xffff0000u)};
      const u32x4 zu = {0u, 0u, 0u, 0u};
      const bf16x8_t b0 = __builtin_bit_cast(bf16x8_t, first ? b : zu);
      const bf16x8_t b1 = __builtin_bit_cast(bf16x8_t, first ? zu : b);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b0, __builtin_bit_cast(bf16x8_t, ones), s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b1, __builtin_bit_cast(bf16x8_t, ones), s1, 0, 0, 0);
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const uint32_t cw = sl.pc[t][st];
        const bf16x8_t av = __builtin_bit_cast(
            bf16x8_t, u32x4{(cw & mask) | magic, ((cw >> 4) & mask) | magic, ((cw >> 8) & mask) | magic,
                            ((cw >> 12) & mask) | magic});
        d0[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b0, av, d0[t], 0, 0, 0);
        d1[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b1, av, d1[t], 0, 0, 0);
      }
    }
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const float sc0 = ss::h2f((uint16_t)(sl.mt[t].x & 0xffffu)), mn0 = ss::h2f((uint16_t)(sl.mt[t].x >> 16));
      const float sc1 = ss::h2f((uint16_t)(sl.mt[t].y & 0xffffu)), mn1 = ss::h2f((uint16_t)(sl.mt[t].y >> 16));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[t][i] += (sc0 * d0[t][i] + (mn0 - 128.0f * sc0) * s0[i]) + (sc1 * d1[t][i] + (mn1 - 128.0f * sc1) * s1[i]);
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

  if constexpr (HALF) {  // the second group's half of position 4 g + i sits 32 lanes away
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[t][i] += __shfl_xor(acc[t][i], 32, SS_WAVE);
  }
  // lane holds positions 4 g + i of row r of each tile (HALF: lanes g < 2)
  if constexpr (SILU) {
    // act[pos][j] = SiLU(gate) * up, both rounded to bf16 first (as the
    // unfused gate/up store and SiLU kernel do)
#pragma unroll
    for (int t = 0; t < HT; ++t) {
      const int64_t j = row0 + 16 * t + r;
      if (j >= silu_f) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pos = 4 * g + i;
        if (pos < m) {
          const float gt = ss::bf2f(ss::f2bf(acc[t][i])), up = ss::bf2f(ss::f2bf(acc[t + HT][i]));
          y[(int64_t)pos * silu_f + j] = ss::f2bf(gt / (1.0f + expf(-gt)) * up);
        }
      }
    }
    return;
  }
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

namespace {

template <bool SILU, bool TL, bool HALF>
hipError_t launch_k(dim3 grid, const uint8_t* codes, const uint16_t* meta, int64_t n, int64_t k, const uint16_t* x,
                    int m, uint16_t* y, float* part, int splits, int to_part, int64_t silu_f, hipStream_t s) {
  SS_LAUNCH((gemm_w4_kernel<SILU, TL, HALF>), grid, dim3(64), 0, s, codes, meta, n, (int)k, x, m, y, part, splits,
            to_part, silu_f);
  return hipGetLastError();
}

template <bool SILU>
hipError_t launch_sel(bool tiled, dim3 grid, const uint8_t* codes, const uint16_t* meta, int64_t n, int64_t k,
                      const uint16_t* x, int m, uint16_t* y, float* part, int splits, int to_part, int64_t silu_f,
                      hipStream_t s) {
  if (tiled) {
    if (m <= 8) return launch_k<SILU, true, true>(grid, codes, meta, n, k, x, m, y, part, splits, to_part, silu_f, s);
    return launch_k<SILU, true, false>(grid, codes, meta, n, k, x, m, y, part, splits, to_part, silu_f, s);
  }
  if (m <= 8) return launch_k<SILU, false, true>(grid, codes, meta, n, k, x, m, y, part, splits, to_part, silu_f, s);
  return launch_k<SILU, false, false>(grid, codes, meta, n, k, x, m, y, part, splits, to_part, silu_f, s);
}

}  // namespace

hipError_t launch_gemm_w4(const uint8_t* codes, const uint16_t* meta, int64_t n, int64_t k, const uint16_t* x, int m,
                          uint16_t* y, float* part, hipStream_t s, int* splits_out, bool tiled) {
  const int splits = gemm_w4_splits(n, k);
  const int to_part = splits_out != nullptr;
  if (to_part) *splits_out = splits;
  const dim3 grid((unsigned)((n + 16 * RT - 1) / (16 * RT)), (unsigned)splits);
  hipError_t e = launch_sel<false>(tiled, grid, codes, meta, n, k, x, m, y, part, splits, to_part, 0, s);
  if (e != hipSuccess || splits == 1 || to_part) return e;
  return launch_gemm_reduce(part, splits, m, n, y, n, s);
}

hipError_t launch_gemm_w4_silu(const uint8_t* codes, const uint16_t* meta, int64_t F, int64_t k, const uint16_t* x,
                               int m, uint16_t* act, hipStream_t s, bool tiled) {
  if (gemm_w4_splits(2 * F, k) != 1) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((F + 8 * RT - 1) / (8 * RT)));
  return launch_sel<true>(tiled, grid, codes, meta, 2 * F, k, x, m, act, (float*)nullptr, 1, 0, F, s);
}
