// Batch-1 GEMV for the draft step: y = W x with W either bf16 or the 4-bit
// substitute (codes + fp16 {scale, min} per 64-group).  Low-batch decode is
// bound by streaming the weights from memory ("How speculative decoding makes
// LLMs go brrr", Module 2), so the kernel is built around HBM bandwidth:
//
//  * x lives in LDS for the whole block.  For W4 it is stored as bf16 pairs
//    (x[k], x[k+4]) in the order the nibble extraction produces, and laid out
//    so that the 64 lanes of a wave read consecutive 16-byte slots (no bank
//    conflicts).  An RMSNorm (and, for layer 0, the embedding gather) is
//    computed in the prologue of every block, so it costs no extra launch.
//  * Every lane streams 16-byte chunks of R rows (R = 1, 2, 4) with several
//    chunks in flight; a wave covers whole rows, lane c takes chunks
//    c, c+64, ...  Rows are contiguous, so each wave load touches R fully
//    used 1 KiB segments.
//  * W4 dequantisation happens in registers: a nibble pair becomes the bf16
//    pair (128+q_a, 128+q_b) with one and-or, and v_dot2_f32_bf16 multiplies
//    it by the x pair.  Per half-group (32 weights)
//        sum_k (q_k s + m) x_k = s * sum_k (128+q_k) x_k + (m - 128 s) * sum_k x_k
//    so the scale and min are applied once per 32 weights; sum_k x_k comes
//    from LDS.
//  * Epilogues: store, residual add (bf16(resid + acc)), SiLU(gate)*up with
//    gate row n and up row F+n in the same wave, and logits with a per-block
//    (max, argmax) partial for the sampler.
#include "common.h"
#include "internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / SS_WAVE;

__device__ __forceinline__ float w4_word_dot(uint32_t cw, u32x4 xq, float d) {
  d = ss::dot2((cw & 0x000F000Fu) | 0x43004300u, xq.x, d);
  d = ss::dot2(((cw >> 4) & 0x000F000Fu) | 0x43004300u, xq.y, d);
  d = ss::dot2(((cw >> 8) & 0x000F000Fu) | 0x43004300u, xq.z, d);
  d = ss::dot2(((cw >> 12) & 0x000F000Fu) | 0x43004300u, xq.w, d);
  return d;
}

__device__ __forceinline__ float bf16_chunk_dot(u32x4 w, u32x4 xq, float d) {
  d = ss::dot2(w.x, xq.x, d);
  d = ss::dot2(w.y, xq.y, d);
  d = ss::dot2(w.z, xq.z, d);
  d = ss::dot2(w.w, xq.w, d);
  return d;
}

// LDS slot (in 16-byte units) of quad w (0..3) of W4 chunk c: lanes of a wave
// reading the same quad of consecutive chunks hit consecutive slots.
__device__ __forceinline__ int w4_slot(int c, int w) { return ((c >> 6) << 8) + (w << 6) + (c & 63); }
// LDS slots of x for W4: whole groups of 64 chunks (256 slots each).
__host__ __device__ __forceinline__ int w4_slots(int K) { return ((K / 32 + 63) / 64) * 256; }

template <int R, bool W4, int PRO, int EPI>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvArgs a) {
  extern __shared__ u32x4 smem4[];
  __shared__ float red[kWaves];
  __shared__ float red_v[kWaves];
  __shared__ int red_i[kWaves];
  __shared__ float s_inv;

  if (a.valid && *a.valid == 0) return;
  const int tid = threadIdx.x, lane = tid & (SS_WAVE - 1), wave = tid / SS_WAVE;
  const int K = (int)a.k;
  const int nq = K / 8;  // 8-element quads of x

  // ---------------------------------------------------------------- prologue
  const uint16_t* src = a.x;
  if (PRO == PRO_NORM) src = a.h;
  if (PRO == PRO_EMBED_NORM) src = a.embed + (int64_t)(*a.token) * K;
  float inv = 1.0f;
  if (PRO != PRO_X) {
    float ss = 0.0f;
    for (int q = tid; q < nq; q += kThreads) {
      u32x4 v = reinterpret_cast<const u32x4*>(src)[q];
      uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float lo = ss::lo_bf(wv[i]), hi = ss::hi_bf(wv[i]);
        ss += lo * lo;
        ss += hi * hi;
      }
    }
    ss = ss::wave_sum(ss);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    if (tid == 0) {
      float t = 0.0f;
      for (int i = 0; i < kWaves; ++i) t += red[i];
      s_inv = 1.0f / sqrtf(t / (float)K + a.eps);
    }
    __syncthreads();
    inv = s_inv;
    if (PRO == PRO_EMBED_NORM && blockIdx.x == 0) {
      for (int q = tid; q < nq; q += kThreads)
        reinterpret_cast<u32x4*>(a.h_out)[q] = reinterpret_cast<const u32x4*>(src)[q];
    }
  }
  for (int q = tid; q < nq; q += kThreads) {
    u32x4 v = reinterpret_cast<const u32x4*>(src)[q];
    uint32_t wv[4] = {v.x, v.y, v.z, v.w};
    uint16_t xb[8];
    if (PRO != PRO_X) {
      u32x4 g = reinterpret_cast<const u32x4*>(a.norm_w)[q];
      uint32_t gv[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xb[2 * i] = ss::f2bf(ss::lo_bf(wv[i]) * inv * ss::lo_bf(gv[i]));
        xb[2 * i + 1] = ss::f2bf(ss::hi_bf(wv[i]) * inv * ss::hi_bf(gv[i]));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xb[2 * i] = (uint16_t)(wv[i] & 0xffffu);
        xb[2 * i + 1] = (uint16_t)(wv[i] >> 16);
      }
    }
    if (W4) {
      u32x4 o = u32x4{ss::pack_bf(xb[0], xb[4]), ss::pack_bf(xb[1], xb[5]),
                           ss::pack_bf(xb[2], xb[6]), ss::pack_bf(xb[3], xb[7])};
      smem4[w4_slot(q >> 2, q & 3)] = o;
    } else {
      smem4[q] = u32x4{ss::pack_bf(xb[0], xb[1]), ss::pack_bf(xb[2], xb[3]),
                            ss::pack_bf(xb[4], xb[5]), ss::pack_bf(xb[6], xb[7])};
    }
  }
  float* xsum = reinterpret_cast<float*>(smem4 + (W4 ? w4_slots(K) : nq));
  if (W4) {
    __syncthreads();
    for (int c = tid; c < K / 32; c += kThreads) {
      float t = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        u32x4 v = smem4[w4_slot(c, w)];
        t += ss::lo_bf(v.x) + ss::hi_bf(v.x) + ss::lo_bf(v.y) + ss::hi_bf(v.y) +
             ss::lo_bf(v.z) + ss::hi_bf(v.z) + ss::lo_bf(v.w) + ss::hi_bf(v.w);
      }
      xsum[c] = t;
    }
  }
  __syncthreads();

  // ---------------------------------------------------------------- rows
  constexpr int RO = (EPI == EPI_SILU) ? R / 2 : R;  // output rows per wave
  const int64_t out0 = ((int64_t)blockIdx.x * kWaves + wave) * RO;
  int64_t prow[R];
  bool rv[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (EPI == EPI_SILU) {
      const int64_t o = out0 + (r % RO);
      rv[r] = o < a.n;
      prow[r] = (r < RO) ? o : a.n + o;
    } else {
      prow[r] = out0 + r;
      rv[r] = prow[r] < a.n;
    }
  }

  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;

  constexpr int U = (8 / R) > 1 ? (8 / R) : 1;  // chunks per row in flight
  if (W4) {
    const int C = K / 32;  // 16-byte code chunks per row
    const u32x4* crow[R];
    const uint32_t* mrow[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t pr = rv[r] ? prow[r] : 0;
      crow[r] = reinterpret_cast<const u32x4*>(a.codes + pr * (K / 2));
      mrow[r] = reinterpret_cast<const uint32_t*>(a.meta) + pr * (K / 64);
    }
    for (int c0 = lane; c0 < C; c0 += U * SS_WAVE) {
      u32x4 cw[U][R];
      uint32_t mt[U][R];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * SS_WAVE;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (c < C && rv[r]) {
            cw[u][r] = __builtin_nontemporal_load(crow[r] + c);
            mt[u][r] = mrow[r][c >> 1];
          } else {
            cw[u][r] = u32x4{0u, 0u, 0u, 0u};
            mt[u][r] = 0;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * SS_WAVE;
        if (c < C) {
          const u32x4 x0 = smem4[w4_slot(c, 0)], x1 = smem4[w4_slot(c, 1)];
          const u32x4 x2 = smem4[w4_slot(c, 2)], x3 = smem4[w4_slot(c, 3)];
          const float xs = xsum[c];
#pragma unroll
          for (int r = 0; r < R; ++r) {
            float d = 0.0f;
            d = w4_word_dot(cw[u][r].x, x0, d);
            d = w4_word_dot(cw[u][r].y, x1, d);
            d = w4_word_dot(cw[u][r].z, x2, d);
            d = w4_word_dot(cw[u][r].w, x3, d);
            const float s = ss::h2f((uint16_t)(mt[u][r] & 0xffffu));
            const float m = ss::h2f((uint16_t)(mt[u][r] >> 16));
            acc[r] += s * d + (m - 128.0f * s) * xs;
          }
        }
      }
    }
  } else {
    const int C = K / 8;  // 16-byte chunks of 8 bf16 weights
    const u32x4* wrow[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t pr = rv[r] ? prow[r] : 0;
      wrow[r] = reinterpret_cast<const u32x4*>(a.w + pr * K);
    }
    for (int c0 = lane; c0 < C; c0 += U * SS_WAVE) {
      u32x4 wv[U][R];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * SS_WAVE;
#pragma unroll
        for (int r = 0; r < R; ++r)
          wv[u][r] = (c < C && rv[r]) ? __builtin_nontemporal_load(wrow[r] + c) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * SS_WAVE;
        if (c < C) {
          const u32x4 xq = smem4[c];
#pragma unroll
          for (int r = 0; r < R; ++r) acc[r] = bf16_chunk_dot(wv[u][r], xq, acc[r]);
        }
      }
    }
  }

  // ---------------------------------------------------------------- epilogue
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = ss::wave_sum(acc[r]);

  if (EPI == EPI_SILU) {
#pragma unroll
    for (int r = 0; r < RO; ++r) {
      if (lane == r && rv[r]) {
        const float g = ss::bf2f(ss::f2bf(acc[r]));
        const float u = ss::bf2f(ss::f2bf(acc[r + RO]));
        const float sg = g / (1.0f + expf(-g));
        a.y[out0 + r] = ss::f2bf(sg * u);
      }
    }
  } else {
    ss::ArgMax best = {-INFINITY, 0x7fffffff};
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (lane == r && rv[r]) {
        float v = acc[r];
        if (EPI == EPI_RESID) v = ss::bf2f(a.resid[prow[r]]) + v;
        const uint16_t b = ss::f2bf(v);
        a.y[prow[r]] = b;
        if (EPI == EPI_LOGITS) {
          ss::ArgMax c = {ss::bf2f(b), (int)prow[r]};
          best = ss::better(best, c);
        }
      }
    }
    if (EPI == EPI_LOGITS) {
      best = ss::wave_argmax(best);
      if (lane == 0) {
        red_v[wave] = best.v;
        red_i[wave] = best.i;
      }
      __syncthreads();
      if (tid == 0) {
        ss::ArgMax b = {red_v[0], red_i[0]};
        for (int i = 1; i < kWaves; ++i) b = ss::better(b, ss::ArgMax{red_v[i], red_i[i]});
        a.part_max[blockIdx.x] = b.v;
        a.part_arg[blockIdx.x] = b.i;
      }
    }
  }
}

template <int R, bool W4, int PRO, int EPI>
hipError_t launch_one(const GemvArgs& a, hipStream_t s, int* blocks_out) {
  constexpr int RO = (EPI == EPI_SILU) ? R / 2 : R;
  const int64_t rows_per_block = (int64_t)kWaves * RO;
  const int64_t blocks = (a.n + rows_per_block - 1) / rows_per_block;
  const size_t lds = W4 ? (size_t)w4_slots((int)a.k) * 16 + (size_t)(a.k / 32) * 4 : (size_t)a.k * 2;
  if (blocks_out) *blocks_out = (int)blocks;
  hipLaunchKernelGGL((gemv_kernel<R, W4, PRO, EPI>), dim3((unsigned)blocks), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <bool W4, int PRO, int EPI>
hipError_t launch_r(int R, const GemvArgs& a, hipStream_t s, int* b) {
  if constexpr (EPI == EPI_SILU) {
    if (R >= 4) return launch_one<4, W4, PRO, EPI>(a, s, b);
    return launch_one<2, W4, PRO, EPI>(a, s, b);
  } else {
    if (R >= 4) return launch_one<4, W4, PRO, EPI>(a, s, b);
    if (R == 2) return launch_one<2, W4, PRO, EPI>(a, s, b);
    return launch_one<1, W4, PRO, EPI>(a, s, b);
  }
}

template <bool W4>
hipError_t launch_w(int R, int pro, int epi, const GemvArgs& a, hipStream_t s, int* b) {
  if (pro == PRO_X && epi == EPI_STORE) return launch_r<W4, PRO_X, EPI_STORE>(R, a, s, b);
  if (pro == PRO_X && epi == EPI_RESID) return launch_r<W4, PRO_X, EPI_RESID>(R, a, s, b);
  if (pro == PRO_NORM && epi == EPI_STORE) return launch_r<W4, PRO_NORM, EPI_STORE>(R, a, s, b);
  if (pro == PRO_EMBED_NORM && epi == EPI_STORE) return launch_r<W4, PRO_EMBED_NORM, EPI_STORE>(R, a, s, b);
  if (pro == PRO_NORM && epi == EPI_SILU) return launch_r<W4, PRO_NORM, EPI_SILU>(R, a, s, b);
  if (pro == PRO_NORM && epi == EPI_LOGITS) return launch_r<W4, PRO_NORM, EPI_LOGITS>(R, a, s, b);
  return hipErrorInvalidValue;
}

}  // namespace

// Rows per wave: enough blocks to fill 256 CUs several times over, and as
// many rows per lane as that allows (more bytes in flight per lane).
static int pick_r(int64_t n, int epi) {
  const int64_t rows = (epi == EPI_SILU) ? 2 * n : n;
  if (rows >= 16384) return 4;
  if (rows >= 4096 || epi == EPI_SILU) return 2;
  return 1;
}

int gemv_rows_per_block(bool /*w4*/, int64_t n, int epi) {
  const int r = pick_r(n, epi);
  return kWaves * ((epi == EPI_SILU) ? r / 2 : r);
}

hipError_t launch_gemv(bool w4, int pro, int epi, const GemvArgs& a, hipStream_t s, int* blocks_out) {
  const int R = pick_r(a.n, epi);
  return w4 ? launch_w<true>(R, pro, epi, a, s, blocks_out) : launch_w<false>(R, pro, epi, a, s, blocks_out);
}
