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
//    tiles; its 4 waves split k four ways and add their partial sums through
//    LDS in wave order (deterministic), then wave 0 runs the epilogue: store,
//    residual add, or SiLU(gate)*up with the gate tile and the up tile in the
//    same block.
//  * Lane (r, g) of MFMA step s feeds k = kb + 32 s + 8 g .. +7 of row r, so
//    one load instruction reads 64 contiguous bytes of each of 16 rows; the
//    next step's loads are issued before the current step's MFMAs.
#include "common.h"
#include "internal.h"
#include "profile.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int KSTEP = 128;  // k per step: 4 MFMAs of 32

struct Plan {
  int64_t groups;  // blocks
  int rt;          // 16-row tiles per block
  int tt;          // position tiles
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
  return p;
}

template <int RT, int TT>
__device__ __forceinline__ void load_step(const u32x4* const (&wp)[RT], const bool (&wv)[RT],
                                          const u32x4* const (&xp)[TT], const bool (&xv)[TT],
                                          int o, u32x4 (&av)[RT][4], u32x4 (&bv)[TT][4]) {
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      av[t][s] = wv[t] ? __builtin_nontemporal_load(wp[t] + o + 4 * s) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < TT; ++u)
#pragma unroll
    for (int s = 0; s < 4; ++s) bv[u][s] = xv[u] ? xp[u][o + 4 * s] : u32x4{0u, 0u, 0u, 0u};
}

template <int RT, int TT>
__device__ __forceinline__ void mma_step(const u32x4 (&av)[RT][4], const u32x4 (&bv)[TT][4],
                                         f32x4_t (&acc)[RT][TT]) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int u = 0; u < TT; ++u)
        acc[t][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[t][s]),
                                                            __builtin_bit_cast(bf16x8_t, bv[u][s]),
                                                            acc[t][u], 0, 0, 0);
}

template <int RT, int TT, int EPI>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs a) {
  __shared__ f32x4_t red[kWaves - 1][RT][TT][SS_WAVE];
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
  const int ksteps = K / KSTEP;
  const int s0 = (ksteps * wave) / kWaves, s1 = (ksteps * (wave + 1)) / kWaves;

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
    u32x4 av[RT][4], bv[TT][4], an[RT][4], bn[TT][4];
    load_step<RT, TT>(wp, wvalid, xp, xvalid, s0 * (KSTEP / 8), av, bv);
    for (int st = s0; st < s1; ++st) {
      const bool more = st + 1 < s1;
      if (more) load_step<RT, TT>(wp, wvalid, xp, xvalid, (st + 1) * (KSTEP / 8), an, bn);
      mma_step<RT, TT>(av, bv, acc);
      if (more) {
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
          for (int s = 0; s < 4; ++s) av[t][s] = an[t][s];
#pragma unroll
        for (int u = 0; u < TT; ++u)
#pragma unroll
          for (int s = 0; s < 4; ++s) bv[u][s] = bn[u][s];
      }
    }
  }

  // k-split reduction across the block's waves, in wave order
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int u = 0; u < TT; ++u) red[wave - 1][t][u][lane] = acc[t][u];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < kWaves - 1; ++w)
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int u = 0; u < TT; ++u) acc[t][u] += red[w][t][u][lane];

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

template <int RT, int EPI>
hipError_t launch_tt(const GemmArgs& a, const Plan& p, hipStream_t s) {
  const dim3 grid((unsigned)p.groups), block(kThreads);
  switch (p.tt) {
    case 1: SS_LAUNCH((gemm_kernel<RT, 1, EPI>), grid, block, 0, s, a); break;
    case 2: SS_LAUNCH((gemm_kernel<RT, 2, EPI>), grid, block, 0, s, a); break;
    case 3: SS_LAUNCH((gemm_kernel<RT, 3, EPI>), grid, block, 0, s, a); break;
    case 4: SS_LAUNCH((gemm_kernel<RT, 4, EPI>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
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
