// Verify GEMM on the matrix cores: Y[t][n] = sum_k X[t][k] W[n][k] for the
// gamma+1 <= 64 positions of one verify pass.  The weights are loaded once for
// all positions ("How speculative decoding makes LLMs go brrr", Module 2), so
// the pass stays bound by streaming W from HBM; MFMA keeps the arithmetic off
// the critical path (arithmetic intensity <= 64 flop/byte, far below the
// matrix-core ridge).
//
//  * v_mfma_f32_16x16x32_bf16: A = 16 weight rows x 32 k, B = 32 k x 16
//    positions, D = 16 rows x 16 positions.  A wave owns RT = 2 row tiles (32
//    rows) and ceil(m/16) position tiles.
//  * The reduction order inside the MFMA is free as long as A and B agree,
//    so each lane loads 64 contiguous bytes of one weight row per 128-k step
//    (lane group g takes k = kb + 32g .. kb + 32g + 31) and feeds them to 4
//    MFMAs; B is loaded with the same k mapping.  A wave load therefore reads
//    32 rows x 256 contiguous bytes.
//  * Short matrices are split along k so that the launch has thousands of
//    waves; partial sums go to scratch and the last wave to finish a row
//    group adds them in split order (deterministic) and runs the epilogue:
//    store, residual add or SiLU(gate)*up (gate tile and up tile in the same
//    wave).
#include "common.h"
#include "internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int RT = 2;        // 16-row tiles per wave
constexpr int KSTEP = 128;   // k per inner step

struct Plan {
  int64_t groups;  // row groups of 16*RT rows (out rows in SILU mode: 16 per group)
  int splits;
  int steps_per_split;
  int tt;          // position tiles
};

Plan make_plan(int64_t n, int64_t k, int m, int epi) {
  Plan p;
  const int64_t out_per_group = (epi == GEPI_SILU) ? 16 : 16 * RT;
  p.groups = (n + out_per_group - 1) / out_per_group;
  p.tt = (m + 15) / 16;
  const int ksteps = (int)(k / KSTEP);
  int splits = 1;
  const int64_t want_waves = 2048;
  if (p.groups < want_waves) {
    splits = (int)((want_waves + p.groups - 1) / p.groups);
    const int max_splits = ksteps / 2 > 0 ? ksteps / 2 : 1;  // >= 2 steps per split
    if (splits > max_splits) splits = max_splits;
  }
  p.steps_per_split = (ksteps + splits - 1) / splits;
  p.splits = (ksteps + p.steps_per_split - 1) / p.steps_per_split;
  return p;
}

template <int TT, int EPI>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs a, Plan p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t item = (int64_t)blockIdx.x * kWaves + wave;
  if (item >= p.groups * p.splits) return;
  const int64_t grp = item / p.splits;
  const int split = (int)(item - grp * p.splits);
  const int K = (int)a.k;
  const int r16 = lane & 15, g4 = lane >> 4;

  // physical weight rows of the two tiles for this lane
  int64_t wrow[RT];
  bool wvalid[RT];
  int64_t obase;  // first output column of the group
  if (EPI == GEPI_SILU) {
    obase = grp * 16;
    wvalid[0] = wvalid[1] = (obase + r16) < a.n;
    wrow[0] = obase + r16;
    wrow[1] = a.n + obase + r16;
  } else {
    obase = grp * 16 * RT;
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      wrow[t] = obase + 16 * t + r16;
      wvalid[t] = wrow[t] < a.n;
    }
  }
  const int kb0 = split * p.steps_per_split * KSTEP;
  int kb1 = kb0 + p.steps_per_split * KSTEP;
  if (kb1 > K) kb1 = K;

  f32x4_t acc[RT][TT];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int u = 0; u < TT; ++u) acc[t][u] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const u32x4* wp[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t)
    wp[t] = reinterpret_cast<const u32x4*>(a.w + (wvalid[t] ? wrow[t] : 0) * (int64_t)K + 32 * g4);
  const u32x4* xp[TT];
  bool xvalid[TT];
#pragma unroll
  for (int u = 0; u < TT; ++u) {
    const int tok = 16 * u + r16;
    xvalid[u] = tok < a.m;
    xp[u] = reinterpret_cast<const u32x4*>(a.x + (int64_t)(xvalid[u] ? tok : 0) * K + 32 * g4);
  }

  for (int kb = kb0; kb < kb1; kb += KSTEP) {
    const int o = kb / 8;  // offset in 16-byte units
    u32x4 av[RT][4], bv[TT][4];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        av[t][s] = wvalid[t] ? __builtin_nontemporal_load(wp[t] + o + s) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < TT; ++u)
#pragma unroll
      for (int s = 0; s < 4; ++s) bv[u][s] = xvalid[u] ? xp[u][o + s] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int u = 0; u < TT; ++u)
          acc[t][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, av[t][s]), __builtin_bit_cast(bf16x8_t, bv[u][s]),
              acc[t][u], 0, 0, 0);
  }

  // D layout: lane holds D[row 4*g4 + j][position r16], j = 0..3
  if (p.splits > 1) {
    // write partials [split][pos][row], then count arrivals of the group
    const int64_t nrows = (EPI == GEPI_SILU) ? 2 * a.n : a.n;
    float* part = a.partials + (int64_t)split * a.m * nrows;
#pragma unroll
    for (int t = 0; t < RT; ++t) {
#pragma unroll
      for (int u = 0; u < TT; ++u) {
        const int tok = 16 * u + r16;
        if (tok >= a.m) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          int64_t row = (EPI == GEPI_SILU) ? (t == 0 ? obase : a.n + obase) + 4 * g4 + j
                                           : obase + 16 * t + 4 * g4 + j;
          bool ok = (EPI == GEPI_SILU) ? (obase + 4 * g4 + j) < a.n : row < a.n;
          if (ok) part[(int64_t)tok * nrows + row] = acc[t][u][j];
        }
      }
    }
    __threadfence();
    uint32_t old = 0;
    if (lane == 0) old = atomicAdd(a.counters + grp, 1u);
    old = __shfl(old, 0, 64);
    if (old != (uint32_t)(p.splits - 1)) return;
    __threadfence();
    // last arrival: sum partials in split order
#pragma unroll
    for (int t = 0; t < RT; ++t) {
#pragma unroll
      for (int u = 0; u < TT; ++u) {
        const int tok = 16 * u + r16;
        if (tok >= a.m) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          int64_t row = (EPI == GEPI_SILU) ? (t == 0 ? obase : a.n + obase) + 4 * g4 + j
                                           : obase + 16 * t + 4 * g4 + j;
          bool ok = (EPI == GEPI_SILU) ? (obase + 4 * g4 + j) < a.n : row < a.n;
          float sum = 0.0f;
          if (ok) {
            for (int s = 0; s < p.splits; ++s)
              sum += __builtin_nontemporal_load(a.partials + ((int64_t)s * a.m + tok) * nrows + row);
          }
          acc[t][u][j] = sum;
        }
      }
    }
    if (lane == 0) a.counters[grp] = 0u;
  }

  // epilogue
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
          const float up = ss::bf2f(ss::f2bf(acc[1][u][j]));
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

template <int EPI>
hipError_t launch_tt(const GemmArgs& a, const Plan& p, hipStream_t s) {
  const int64_t waves = p.groups * p.splits;
  const unsigned blocks = (unsigned)((waves + kWaves - 1) / kWaves);
  switch (p.tt) {
    case 1: hipLaunchKernelGGL((gemm_kernel<1, EPI>), dim3(blocks), dim3(kThreads), 0, s, a, p); break;
    case 2: hipLaunchKernelGGL((gemm_kernel<2, EPI>), dim3(blocks), dim3(kThreads), 0, s, a, p); break;
    case 3: hipLaunchKernelGGL((gemm_kernel<3, EPI>), dim3(blocks), dim3(kThreads), 0, s, a, p); break;
    case 4: hipLaunchKernelGGL((gemm_kernel<4, EPI>), dim3(blocks), dim3(kThreads), 0, s, a, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

size_t gemm_partials_bytes(int64_t n, int64_t k, int m, int epi) {
  Plan p = make_plan(n, k, m, epi);
  if (p.splits <= 1) return 0;
  const int64_t nrows = (epi == GEPI_SILU) ? 2 * n : n;
  return (size_t)p.splits * (size_t)m * (size_t)nrows * sizeof(float);
}

size_t gemm_counter_slots(int64_t n, int64_t k, int m, int epi) {
  Plan p = make_plan(n, k, m, epi);
  return p.splits > 1 ? (size_t)p.groups : 0;
}

hipError_t launch_gemm(int epi, const GemmArgs& a, hipStream_t s) {
  Plan p = make_plan(a.n, a.k, a.m, epi);
  switch (epi) {
    case GEPI_STORE: return launch_tt<GEPI_STORE>(a, p, s);
    case GEPI_RESID: return launch_tt<GEPI_RESID>(a, p, s);
    case GEPI_SILU: return launch_tt<GEPI_SILU>(a, p, s);
  }
  return hipErrorInvalidValue;
}
