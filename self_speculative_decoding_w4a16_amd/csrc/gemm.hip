// Verify GEMM on the matrix cores: Y[t][n] = sum_k X[t][k] W[n][k] for the
// gamma+1 positions of one verify pass (and the rows of a tree's or a batch's
// pass).  The weights are loaded once for every slice of up to 64 positions
// (128 past 64) ("How speculative decoding makes LLMs go brrr", Module 2), so
// the pass stays bound by streaming W from HBM; MFMA keeps the arithmetic off
// the critical path (arithmetic intensity <= 128 flop/byte, below the
// matrix-core ridge).
//
//  * v_mfma_f32_16x16x32_bf16: A = 16 weight rows x 32 k, B = 32 k x 16
//    positions, D = 16 rows x 16 positions (lane l holds rows 4(l/16)..+3 of
//    position l%16).
//  * A block has NW waves (2, or 8 for the very wide lm_head and past 64
//    positions); each wave owns one 16-row tile and all position tiles of
//    its slice (up to 4, or 8 past 64 positions).  The block walks
//    its k range in chunks of 128: the activation chunk X[0..16 TT)[kc..+128)
//    is staged in LDS (double-buffered, one barrier a chunk) and read by all
//    NW waves.  Each wave loads its weight chunk row-contiguously (load s:
//    rows 4s .. 4s+3, 256 bytes of each, so every load instruction reads
//    whole 128-byte lines of 4 rows) and passes it through a 4 KiB LDS tile
//    of its own, XOR-swizzled by row so that both the row-wise writes and the
//    MFMA-layout reads are free of bank conflicts: lane (r, g) of MFMA step s
//    reads k = kc + 32 s + 8 g .. +7 of row r.  (Loading straight into the
//    MFMA layout reads 16 rows x 64 bytes per instruction, which streamed
//    ~10 % slower.)  The weight loads are non-temporal (streamed once), which
//    on this row-contiguous pattern measured 5-11 % faster than plain loads.
//  * Pipeline: the weights and activations of WD = 2 chunks are in flight per
//    wave.  Every load in the loop is unconditional (buffer loads: offsets
//    outside the resource return zeros), so the compiler's count of loads in
//    flight is exact and each wait covers only the chunk about to be used.
//  * Row tiles are few for the narrow matrices (QKV, O, down), so the k range
//    is also split over `splits` blocks; those write fp32 partial sums
//    [split][position][n] that the consumer adds in split order (the RoPE
//    kernel for QKV, the residual + RMSNorm kernel for O and down), so no
//    extra launch is spent on the reduction.  Otherwise the block runs the
//    epilogue itself: store, residual add, or SiLU(gate)*up (gate tiles in
//    the first NW/2 waves, the matching up tiles in the others).
#include "common.h"
#include "internal.h"
#include "profile.h"

namespace {

constexpr int KC = 128;             // k per chunk
constexpr int KS = KC / 32;         // MFMA steps (k = 32 each) per chunk
constexpr int WD = 2;               // weight chunks in flight per wave
constexpr int XROW = KC + 8;        // LDS row stride (bf16) of the staged activations
// split k until the grid has about 1.5 blocks per compute unit: the 7B verify
// pass (17 positions) measured 3.32 ms at 384 against 3.46 at 512, 3.50 at
// 320, 3.33 at 448 and 3.56 at 256 (graph-replayed passes)
constexpr int kTargetBlocks = 384;
constexpr int kBufferWord3 = 0x00020000;  // buffer resource word 3 (CDNA): raw 32-bit data
constexpr int kOutside = 0x40000000;      // byte offset past every resource: loads zeros
constexpr int kNonTemporal = 2;           // buffer load cache policy: nt (streamed weights)

struct Plan {
  int64_t groups;  // row groups (blocks along n)
  int tt;          // position tiles of one slice
  int splits;      // k splits (blocks along k)
  int nw;          // waves per block
  int slices;      // slices of slice_rows(m) positions (grid z)
};

// Waves per block.  Small blocks (2 waves) keep many independent blocks in
// flight, which streams best; the very wide matrices (lm_head) take 8 so that
// the activations are not staged again for every 32 rows.  Past 32 positions
// (three or four position tiles) the staged activations outweigh the 32
// weight rows of a 2-wave block, and the gate/up GEMM shares them over 8
// waves (32B shape, 49 positions: 150 -> 98 us; at 17 positions 8-wave
// blocks were slower, 57 against 47 us).  Its sums do not depend on the
// block shape (no k split); the split-k GEMMs keep 2-wave blocks, since
// fewer row groups would mean more splits and other partial sums (4 waves
// took the 32B down GEMM from 69 to 64 us, but changed every result that
// depends on those sums, e.g. the prefill's KV cache).
int block_waves(int64_t n, int epi, int m) {
  if (m > 64) return 8;  // slices of 128 positions (a tree's or a batch's verify pass)
  if (epi == GEPI_SILU) return m > 32 ? 8 : 2;
  return n >= 65536 ? 8 : 2;
}

int64_t rows_per_group(int64_t n, int epi, int m) {
  const int nw = block_waves(n, epi, m);
  return epi == GEPI_SILU ? 16 * nw / 2 : 16 * nw;
}

// Positions of one slice (grid z): up to 64, or 128 past 64 positions, so
// that a 289-node tree verify pass streams the weights 3 times, not 5.
int slice_rows(int m) { return m > 64 ? 128 : 64; }

Plan make_plan(int64_t n, int64_t k, int m, int epi) {
  Plan p;
  const int sl = slice_rows(m);
  const int ms = std::min(m, sl);  // positions of one slice
  p.slices = (m + sl - 1) / sl;
  p.tt = sl == 128 ? 8 : (ms + 15) / 16;
  p.nw = block_waves(n, epi, m);
  const int64_t rg = rows_per_group(n, epi, ms);
  p.groups = (n + rg - 1) / rg;
  const int chunks = (int)(k / KC);
  const int64_t blocks = p.groups * p.slices;
  p.splits = 1;
  if (epi != GEPI_SILU && blocks < kTargetBlocks)
    p.splits = (int)std::min<int64_t>(chunks, (kTargetBlocks + blocks - 1) / blocks);
  return p;
}

template <int NWR, int TT, int EPI>
__global__ __launch_bounds__(NWR * SS_WAVE) void gemm_kernel(GemmArgs a, int splits) {
  // staged activation rows: 16 TT positions, rounded up to what one pass of
  // the block's threads covers (the extra rows are loaded as zeros)
  constexpr int XPT = (16 * TT * KC / 8 + NWR * SS_WAVE - 1) / (NWR * SS_WAVE);  // 16-byte pieces per thread
  constexpr int XR = XPT * NWR * SS_WAVE * 8 / KC;
  __shared__ __align__(16) uint16_t xs[2][XR][XROW];
  __shared__ __align__(16) uint8_t wt[NWR][16 * KC * 2];  // per-wave weight tile [16 rows][KC], swizzled
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;
  const int K = (int)a.k;
  const int chunks = K / KC;
  const int split = blockIdx.y;
  const int c0 = (int)((int64_t)chunks * split / splits), c1 = (int)((int64_t)chunks * (split + 1) / splits);
  // this block's slice of at most 64 (or, with 8 position tiles, 128)
  // positions: rows of x and y
  constexpr int SL = TT > 4 ? 128 : 64;
  const int zrow = blockIdx.z * SL;
  const int mz = min(SL, a.m - zrow);

  // this wave's 16 weight rows
  int64_t row0;  // first physical row of the tile
  int64_t out0;  // first output column of the tile
  if (EPI == GEPI_SILU) {
    const int half = NWR / 2;
    out0 = (int64_t)blockIdx.x * 16 * half + 16 * (wave % half);
    row0 = (wave < half) ? out0 : a.n + out0;
  } else {
    out0 = (int64_t)blockIdx.x * 16 * NWR + 16 * wave;
    row0 = out0;
  }
  // Every load of the main loop is unconditional, so the compiler can count
  // the loads in flight exactly (a load skipped on one path makes it wait for
  // all of them).  Both operands are read through buffer resources: an
  // offset outside the resource loads zeros without touching memory, which
  // covers rows past n, positions past m and chunks past the block's range.
  const int rows = (int)std::max<int64_t>(0, std::min<int64_t>(16, a.n - out0));
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.w + row0 * (int64_t)K), 0, rows * K * 2, kBufferWord3);
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.x + (int64_t)zrow * K), 0, mz * K * 2, kBufferWord3);
  // lane l loads row 4 s + l / 16 (load s), bytes 16 (l % 16) .. +15 of the chunk
  const int wlane = ((lane >> 4) * K + 8 * (lane & 15)) * 2;
  auto chunk_off = [&](int c) { return c < c1 ? c * KC * 2 : kOutside; };

  // activation staging: thread -> (position, 16 bytes) of the chunk
  auto load_x = [&](int c, u32x4 (&xr)[XPT]) {
    const int co = chunk_off(c);
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int e = tid + i * NWR * SS_WAVE;
      const int pos = e / (KC / 8), q = e % (KC / 8);
      xr[i] = __builtin_amdgcn_raw_buffer_load_b128(xrs, pos * K * 2 + 16 * q + co, 0, 0);
    }
  };
  auto store_x = [&](const u32x4 (&xr)[XPT], int buf) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int e = tid + i * NWR * SS_WAVE;
      const int pos = e / (KC / 8), q = e % (KC / 8);
      *reinterpret_cast<u32x4*>(&xs[buf][pos][8 * q]) = xr[i];
    }
  };
  auto load_w = [&](int c, u32x4 (&av)[KS]) {
    const int off = wlane + chunk_off(c);
#pragma unroll
    for (int s = 0; s < KS; ++s) av[s] = __builtin_amdgcn_raw_buffer_load_b128(wrs, off + 4 * K * 2 * s, 0, kNonTemporal);
  };

  f32x4_t acc[TT];
#pragma unroll
  for (int u = 0; u < TT; ++u) acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Chunks c .. c + WD - 1 are in flight, each as its activations followed by
  // its weights, in rings of WD register buffers: chunk c lives in slot
  // (c - c0) % WD by name (the loop is unrolled by WD; a rotation by register
  // copies would wait for the loads still in flight).  Loads complete in
  // issue order, so waiting for the activations of chunk c + 1 (to stage
  // them in LDS while chunk c is multiplied) also waits for the weights of
  // chunk c, and for nothing later.
  u32x4 wb[WD][KS], xb[WD][XPT];
#pragma unroll
  for (int j = 0; j < WD; ++j) {
    load_x(c0 + j, xb[j]);
    load_w(c0 + j, wb[j]);
  }
  store_x(xb[0], 0);
  __syncthreads();
  auto step = [&](int c, u32x4 (&w)[KS], u32x4 (&xc)[XPT], const u32x4 (&xn)[XPT]) {
    const int buf = (c - c0) & 1;
    store_x(xn, buf ^ 1);  // chunk c + 1 (zeros past the range)
    load_x(c + WD, xc);    // chunk c is already in LDS
    // weights of chunk c through this wave's tile: 16-byte piece k of row r
    // sits at slot k ^ r of the row (the wave's own LDS ops run in order, so
    // the previous chunk's reads are done before these writes land)
    uint8_t* wtw = &wt[wave][0];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int row = 4 * s + (lane >> 4);
      *reinterpret_cast<u32x4*>(wtw + KC * 2 * row + 16 * ((lane & 15) ^ row)) = w[s];
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const u32x4 av = *reinterpret_cast<const u32x4*>(wtw + KC * 2 * r16 + 16 * ((4 * s + g4) ^ r16));
#pragma unroll
      for (int u = 0; u < TT; ++u) {
        const u32x4 b = *reinterpret_cast<const u32x4*>(&xs[buf][16 * u + r16][32 * s + 8 * g4]);
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                         __builtin_bit_cast(bf16x8_t, b), acc[u], 0, 0, 0);
      }
    }
    load_w(c + WD, w);
    __syncthreads();
  };
  int c = c0;
  for (; c + WD <= c1; c += WD) {
#pragma unroll
    for (int j = 0; j < WD; ++j) step(c + j, wb[j], xb[j], xb[(j + 1) % WD]);
  }
#pragma unroll
  for (int j = 0; j < WD - 1; ++j)
    if (c + j < c1) step(c + j, wb[j], xb[j], xb[(j + 1) % WD]);

  // epilogue: lane holds D[row 4 g4 + j][position 16 u + r16]
  if (EPI == GEPI_SILU) {
    // up tiles (waves NWR/2..) hand their sums to the gate tiles through LDS
    float* up = reinterpret_cast<float*>(&xs[0][0][0]);  // [NWR/2][TT][64][4] floats
    const int half = NWR / 2;
    if (wave >= half) {
#pragma unroll
      for (int u = 0; u < TT; ++u)
        *reinterpret_cast<f32x4_t*>(&up[(((wave - half) * TT + u) * SS_WAVE + lane) * 4]) = acc[u];
    }
    __syncthreads();
    if (wave >= half) return;
#pragma unroll
    for (int u = 0; u < TT; ++u) {
      const int tok = 16 * u + r16;
      if (tok >= mz) continue;
      const int64_t gt = zrow + tok;
      const f32x4_t uv = *reinterpret_cast<const f32x4_t*>(&up[((wave * TT + u) * SS_WAVE + lane) * 4]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t col = out0 + 4 * g4 + j;
        if (col < a.n) {
          const float gv = ss::bf2f(ss::f2bf(acc[u][j]));
          const float upv = ss::bf2f(ss::f2bf(uv[j]));
          a.y[gt * a.ldy + col] = ss::f2bf(gv / (1.0f + expf(-gv)) * upv);
        }
      }
    }
    return;
  }
#pragma unroll
  for (int u = 0; u < TT; ++u) {
    const int tok = 16 * u + r16;
    if (tok >= mz) continue;
    const int64_t gt = zrow + tok;  // position in the whole launch
    const int64_t col = out0 + 4 * g4;
    if (EPI == GEPI_PARTIAL) {
      float* dst = a.partials + ((int64_t)split * a.m + gt) * a.n + col;
      if (col + 3 < a.n && (a.n & 3) == 0) {
        *reinterpret_cast<f32x4_t*>(dst) = acc[u];  // 16-byte aligned: n % 4 == 0, col % 4 == 0
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (col + j < a.n) dst[j] = acc[u][j];
      }
      continue;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (col + j < a.n) {
        float v = acc[u][j];
        if (EPI == GEPI_RESID) v += ss::bf2f(a.resid[gt * a.ldy + col + j]);
        a.y[gt * a.ldy + col + j] = ss::f2bf(v);
      }
    }
  }
}

// Y[t][n] = bf16(sum over splits of the partials), in split order (the
// kernel-level GEMM entry point; the verify pass reduces in its consumers).
__global__ __launch_bounds__(256) void gemm_reduce_kernel(const float* part, int splits, int m, int64_t n,
                                                          uint16_t* y, int64_t ldy) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)m * n) return;
  const int64_t t = e / n, c = e % n;
  float v = 0.0f;
  for (int s = 0; s < splits; ++s) v += part[((int64_t)s * m + t) * n + c];
  y[t * ldy + c] = ss::f2bf(v);
}

template <int NW, int EPI>
hipError_t launch_nw(const GemmArgs& a, const Plan& p, hipStream_t s) {
  const dim3 grid((unsigned)p.groups, (unsigned)p.splits, (unsigned)p.slices), block(NW * SS_WAVE);
  switch (p.tt) {
    case 1: SS_LAUNCH((gemm_kernel<NW, 1, EPI>), grid, block, 0, s, a, p.splits); break;
    case 2: SS_LAUNCH((gemm_kernel<NW, 2, EPI>), grid, block, 0, s, a, p.splits); break;
    case 3: SS_LAUNCH((gemm_kernel<NW, 3, EPI>), grid, block, 0, s, a, p.splits); break;
    case 4: SS_LAUNCH((gemm_kernel<NW, 4, EPI>), grid, block, 0, s, a, p.splits); break;
    case 8:
      if constexpr (NW == 8) {
        SS_LAUNCH((gemm_kernel<NW, 8, EPI>), grid, block, 0, s, a, p.splits);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_tt(const GemmArgs& a, const Plan& p, hipStream_t s) {
  if (p.nw == 2) return launch_nw<2, EPI>(a, p, s);
  if (p.nw == 4) return launch_nw<4, EPI>(a, p, s);
  if (p.nw == 8) return launch_nw<8, EPI>(a, p, s);
  return hipErrorInvalidValue;
}

}  // namespace

int gemm_splits(int64_t n, int64_t k, int m, int epi) { return make_plan(n, k, m, epi).splits; }

size_t gemm_partials_bytes(int64_t n, int64_t k, int m, int epi) {
  const Plan p = make_plan(n, k, m, epi);
  return p.splits > 1 ? (size_t)p.splits * m * n * 4 : 0;
}

hipError_t launch_gemm(int epi, const GemmArgs& a, hipStream_t s, int* splits_out) {
  const Plan p = make_plan(a.n, a.k, a.m, epi);
  if (splits_out) *splits_out = p.splits;
  if (p.splits > 1) {
    // the caller reduces a.partials [splits][m][n]
    if (epi == GEPI_SILU || !a.partials) return hipErrorInvalidValue;
    return launch_tt<GEPI_PARTIAL>(a, p, s);
  }
  switch (epi) {
    case GEPI_STORE: return launch_tt<GEPI_STORE>(a, p, s);
    case GEPI_RESID: return launch_tt<GEPI_RESID>(a, p, s);
    case GEPI_SILU: return launch_tt<GEPI_SILU>(a, p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_reduce(const float* part, int splits, int m, int64_t n, uint16_t* y, int64_t ldy,
                              hipStream_t s) {
  const int64_t total = (int64_t)m * n;
  SS_LAUNCH(gemm_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, part, splits, m, n, y,
            ldy);
  return hipGetLastError();
}
