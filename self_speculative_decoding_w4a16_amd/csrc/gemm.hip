// Verify GEMM on the matrix cores: Y[t][n] = sum_k X[t][k] W[n][k] for the
// gamma+1 <= 64 positions of one verify pass.  The weights are loaded once for
// all positions ("How speculative decoding makes LLMs go brrr", Module 2), so
// the pass stays bound by streaming W from HBM; MFMA keeps the arithmetic off
// the critical path (arithmetic intensity <= 64 flop/byte, far below the
// matrix-core ridge).
//
//  * v_mfma_f32_16x16x32_bf16: A = 16 weight rows x 32 k, B = 32 k x 16
//    positions, D = 16 rows x 16 positions (lane l holds rows 4(l/16)..+3 of
//    column l%16).  A block owns RT 16-row tiles and ceil(m/16) position
//    tiles; its NW waves split k NW ways and add their partial sums through
//    LDS in a fixed tree (deterministic), then wave 0 runs the epilogue:
//    store, residual add, or SiLU(gate)*up with the gate tile and the up tile
//    in the same block.  NW (4, 8 or 16) grows when the matrix has few row
//    tiles, so that every launch keeps ~16 waves per compute unit streaming.
//  * Lane (r, g) of MFMA step s feeds k = kb + 32 s + 8 g .. +7 of row r, so
//    one load instruction reads 64 contiguous bytes of each of 16 rows; the
//    next step's loads are issued before the current step's MFMAs.
#include "common.h"
#include "internal.h"
#include "profile.h"

namespace {

constexpr int kTargetWaves = 4096;  // ~16 per compute unit

struct Plan {
  int64_t groups;  // blocks
  int rt;          // 16-row tiles per block
  int tt;          // position tiles
  int nw;          // waves per block (k split)
};

Plan make_plan(int64_t n, int64_t /*k*/, int m, int epi) {
  Plan p;
  p.tt = (m + 15) / 16;
  if (epi == GEPI_SILU) {
    p.rt = 2;  // tile 0: 16 gate rows, tile 1: the matching 16 up rows
    p.groups = (n + 15) / 16;
  } else {
    p.rt = (n >= 65536) ? 2 : 1;
    p.groups = (n + 16 * p.rt - 1) / (16 * p.rt);
  }
  p.nw = 4;
  if (p.groups * 4 < kTargetWaves) p.nw = 8;
  if (p.groups * 8 < kTargetWaves && p.rt == 1) p.nw = 16;  // LDS: 8 x TT x 1 KiB
  return p;
}

// k-substeps (MFMAs of k = 32) per pipeline step: fewer when many position
// tiles are in flight, to bound the registers of the double buffer.
template <int TT>
constexpr int ksub() { return TT >= 3 ? 2 : 4; }

template <int RT, int TT, int KS>
__device__ __forceinline__ void load_step(const u32x4* const (&wp)[RT], const bool (&wv)[RT],
                                          const u32x4* const (&xp)[TT], const bool (&xv)[TT],
                                          int o, u32x4 (&av)[RT][KS], u32x4 (&bv)[TT][KS]) {
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int s = 0; s < KS; ++s)
      av[t][s] = wv[t] ? __builtin_nontemporal_load(wp[t] + o + 4 * s) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < TT; ++u)
#pragma unroll
    for (int s = 0; s < KS; ++s) bv[u][s] = xv[u] ? xp[u][o + 4 * s] : u32x4{0u, 0u, 0u, 0u};
}

template <int RT, int TT, int KS>
__device__ __forceinline__ void mma_step(const u32x4 (&av)[RT][KS], const u32x4 (&bv)[TT][KS],
                                         f32x4_t (&acc)[RT][TT]) {
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int u = 0; u < TT; ++u)
        acc[t][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[t][s]),
                                                            __builtin_bit_cast(bf16x8_t, bv[u][s]),
                                                            acc[t][u], 0, 0, 0);
}

template <int RT, int TT, int EPI, int NW>
__global__ __launch_bounds__(NW * SS_WAVE) void gemm_kernel(GemmArgs a) {
  __shared__ f32x4_t red[NW / 2][RT][TT][SS_WAVE];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t grp = blockIdx.x;
  const int K = (int)a.k;
  const int r16 = lane & 15, g4 = lane >> 4;

  int64_t wrow[RT];
  bool wvalid[RT];
  int64_t obase;
  if (EPI == GEPI_SILU) {
    obase = grp * 16;
    wvalid[0] = wvalid[RT - 1] = (obase + r16) < a.n;
    wrow[0] = obase + r16;
    wrow[RT - 1] = a.n + obase + r16;
  } else {
    obase = grp * 16 * RT;
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      wrow[t] = obase + 16 * t + r16;
      wvalid[t] = wrow[t] < a.n;
    }
  }
  constexpr int KS = ksub<TT>();
  constexpr int KSTEP = 32 * KS;
  const int ksteps = K / KSTEP;
  const int s0 = (ksteps * wave) / NW, s1 = (ksteps * (wave + 1)) / NW;

  f32x4_t acc[RT][TT];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int u = 0; u < TT; ++u) acc[t][u] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const u32x4* wp[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t)
    wp[t] = reinterpret_cast<const u32x4*>(a.w + (wvalid[t] ? wrow[t] : 0) * (int64_t)K) + g4;
  const u32x4* xp[TT];
  bool xvalid[TT];
#pragma unroll
  for (int u = 0; u < TT; ++u) {
    const int tok = 16 * u + r16;
    xvalid[u] = tok < a.m;
    xp[u] = reinterpret_cast<const u32x4*>(a.x + (int64_t)(xvalid[u] ? tok : 0) * K) + g4;
  }

  if (s0 < s1) {
    u32x4 av[RT][KS], bv[TT][KS], an[RT][KS], bn[TT][KS];
    load_step<RT, TT, KS>(wp, wvalid, xp, xvalid, s0 * (KSTEP / 8), av, bv);
    for (int st = s0; st < s1; ++st) {
      const bool more = st + 1 < s1;
      if (more) load_step<RT, TT, KS>(wp, wvalid, xp, xvalid, (st + 1) * (KSTEP / 8), an, bn);
      mma_step<RT, TT, KS>(av, bv, acc);
      if (more) {
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
          for (int s = 0; s < KS; ++s) av[t][s] = an[t][s];
#pragma unroll
        for (int u = 0; u < TT; ++u)
#pragma unroll
          for (int s = 0; s < KS; ++s) bv[u][s] = bn[u][s];
      }
    }
  }

  // k-split reduction across the block's waves: a fixed tree (waves
  // [h, 2h) hand their sums to waves [0, h), h = NW/2, ..., 1)
#pragma unroll
  for (int h = NW / 2; h >= 1; h >>= 1) {
    if (wave >= h && wave < 2 * h) {
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int u = 0; u < TT; ++u) red[wave - h][t][u][lane] = acc[t][u];
    }
    __syncthreads();
    if (wave < h) {
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int u = 0; u < TT; ++u) acc[t][u] += red[wave][t][u][lane];
    }
    __syncthreads();
  }
  if (wave != 0) return;

  // epilogue: lane holds D[row 4*g4 + j][position r16]
#pragma unroll
  for (int u = 0; u < TT; ++u) {
    const int tok = 16 * u + r16;
    if (tok >= a.m) continue;
    uint16_t* yrow = a.y + (int64_t)tok * a.ldy;
    if (EPI == GEPI_SILU) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t col = obase + 4 * g4 + j;
        if (col < a.n) {
          const float g = ss::bf2f(ss::f2bf(acc[0][u][j]));
          const float up = ss::bf2f(ss::f2bf(acc[RT - 1][u][j]));
          yrow[col] = ss::f2bf(g / (1.0f + expf(-g)) * up);
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < RT; ++t) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t col = obase + 16 * t + 4 * g4 + j;
          if (col < a.n) {
            float v = acc[t][u][j];
            if (EPI == GEPI_RESID) v += ss::bf2f(a.resid[(int64_t)tok * a.ldy + col]);
            yrow[col] = ss::f2bf(v);
          }
        }
      }
    }
  }
}

template <int RT, int EPI, int NW>
hipError_t launch_nw(const GemmArgs& a, const Plan& p, hipStream_t s) {
  const dim3 grid((unsigned)p.groups), block(NW * SS_WAVE);
  switch (p.tt) {
    case 1: SS_LAUNCH((gemm_kernel<RT, 1, EPI, NW>), grid, block, 0, s, a); break;
    case 2: SS_LAUNCH((gemm_kernel<RT, 2, EPI, NW>), grid, block, 0, s, a); break;
    case 3: SS_LAUNCH((gemm_kernel<RT, 3, EPI, NW>), grid, block, 0, s, a); break;
    case 4: SS_LAUNCH((gemm_kernel<RT, 4, EPI, NW>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int RT, int EPI>
hipError_t launch_tt(const GemmArgs& a, const Plan& p, hipStream_t s) {
  if constexpr (RT == 1) {
    if (p.nw == 16) return launch_nw<RT, EPI, 16>(a, p, s);
  }
  if (p.nw == 8) return launch_nw<RT, EPI, 8>(a, p, s);
  return launch_nw<RT, EPI, 4>(a, p, s);
}

}  // namespace

size_t gemm_partials_bytes(int64_t, int64_t, int, int) { return 0; }
size_t gemm_counter_slots(int64_t, int64_t, int, int) { return 0; }

hipError_t launch_gemm(int epi, const GemmArgs& a, hipStream_t s) {
  Plan p = make_plan(a.n, a.k, a.m, epi);
  switch (epi) {
    case GEPI_STORE:
      return p.rt == 2 ? launch_tt<2, GEPI_STORE>(a, p, s) : launch_tt<1, GEPI_STORE>(a, p, s);
    case GEPI_RESID:
      return p.rt == 2 ? launch_tt<2, GEPI_RESID>(a, p, s) : launch_tt<1, GEPI_RESID>(a, p, s);
    case GEPI_SILU: return launch_tt<2, GEPI_SILU>(a, p, s);
  }
  return hipErrorInvalidValue;
}
