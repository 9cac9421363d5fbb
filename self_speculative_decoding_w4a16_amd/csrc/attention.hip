// Attention over the shared KV cache for the draft step (one query position)
// and the verify pass (gamma+1 query positions, causal: row j sees positions
// [0, kv_len + j]) - "How speculative decoding makes LLMs go brrr", Module 2;
// draft and target read and write one cache ("SubSpec: Speculate Deep and
// Accurate" paper note, Method details, KV-cache sharing).
//
// Three kernels:
//  rope_append  rotate-half RoPE of q and k (angles in float64, applied in
//               float32), q -> q_rot, k/v -> cache at their positions.
//  attn_part    grid (kv head, key split): the GQA group's query rows against
//               up to 64 keys staged in LDS; per row a partial (max, sum, o[d]).
//  attn_combine grid (q head, row): merges the splits in split order.
#include "common.h"
#include "internal.h"

namespace {

constexpr int KPS = 64;    // keys per split
constexpr int D = 128;     // head dim handled by these kernels
constexpr int QB = 32;     // query rows per pass inside a block

__global__ __launch_bounds__(64) void rope_append_kernel(AttnArgs a) {
  const int j = blockIdx.x;          // query row
  const int head = blockIdx.y;       // 0..Hq-1: q heads, Hq..Hq+Hkv-1: kv heads
  const int i = threadIdx.x;         // pair index 0..d/2-1
  const int half = a.d / 2;
  if (i >= half) return;
  const int pos = *a.kv_len + a.pos_offset + j;
  const int rows = a.n_q + 2 * a.n_kv;
  const uint16_t* src = a.qkv + (int64_t)j * rows * a.d;
  const double inv_freq = exp(-(2.0 * i / a.d) * log((double)a.theta));
  double sd, cd;
  sincos((double)pos * inv_freq, &sd, &cd);
  const float c = (float)cd, s = (float)sd;
  if (head < a.n_q) {
    const uint16_t* x = src + head * a.d;
    const float x1 = ss::bf2f(x[i]), x2 = ss::bf2f(x[i + half]);
    uint16_t* o = a.q_rot + (int64_t)j * a.n_q * a.d + head * a.d;
    o[i] = ss::f2bf(x1 * c - x2 * s);
    o[i + half] = ss::f2bf(x2 * c + x1 * s);
  } else {
    const int hk = head - a.n_q;
    if (pos < 0 || pos >= a.cap) return;
    const uint16_t* k = src + (a.n_q + hk) * a.d;
    const uint16_t* v = src + (a.n_q + a.n_kv + hk) * a.d;
    const float x1 = ss::bf2f(k[i]), x2 = ss::bf2f(k[i + half]);
    uint16_t* kc = a.k_cache + ((int64_t)hk * a.cap + pos) * a.d;
    uint16_t* vc = a.v_cache + ((int64_t)hk * a.cap + pos) * a.d;
    kc[i] = ss::f2bf(x1 * c - x2 * s);
    kc[i + half] = ss::f2bf(x2 * c + x1 * s);
    vc[i] = v[i];
    vc[i + half] = v[i + half];
  }
}

// rows of the GQA group: r = g * m + j  (g: q head within the group, j: position row)
__global__ __launch_bounds__(256) void attn_part_kernel(AttnArgs a) {
  __shared__ u32x4 ks[KPS][D / 8 + 1];  // padded: conflict-free 16-byte reads
  __shared__ u32x4 vs[KPS][D / 8 + 1];
  __shared__ float qs[QB][D];          // 16 KB
  __shared__ float sc[QB][KPS + 1];    // 8.3 KB
  __shared__ float rmax[QB], rsum[QB];

  const int hk = blockIdx.x, split = blockIdx.y;
  const int tid = threadIdx.x;
  const int G = a.n_q / a.n_kv;
  const int base = *a.kv_len + a.pos_offset;      // position of row 0
  int n_keys = base + a.m;                         // keys visible to the last row
  if (n_keys > a.cap) n_keys = a.cap;
  const int k0 = split * KPS;
  if (k0 >= n_keys) return;
  const int nk = min(KPS, n_keys - k0);
  const float scale = 0.088388347648318440f;  // 1/sqrt(128)

  const u32x4* kg = reinterpret_cast<const u32x4*>(a.k_cache + ((int64_t)hk * a.cap + k0) * D);
  const u32x4* vg = reinterpret_cast<const u32x4*>(a.v_cache + ((int64_t)hk * a.cap + k0) * D);
  for (int e = tid; e < nk * (D / 8); e += 256) {
    ks[e / (D / 8)][e % (D / 8)] = kg[e];
    vs[e / (D / 8)][e % (D / 8)] = vg[e];
  }

  const int total_rows = G * a.m;
  for (int r0 = 0; r0 < total_rows; r0 += QB) {
    const int nr = min(QB, total_rows - r0);
    __syncthreads();
    for (int e = tid; e < nr * D; e += 256) {
      const int rr = e / D, dd = e % D;
      const int r = r0 + rr, g = r / a.m, j = r % a.m;
      qs[rr][dd] = ss::bf2f(a.q_rot[((int64_t)j * a.n_q + hk * G + g) * D + dd]);
    }
    __syncthreads();
    // scores: thread -> (key, row group of 8)
    {
      const int key = tid & 63, rg = tid >> 6;
      float acc[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] = 0.0f;
      if (key < nk) {
        for (int dc = 0; dc < D / 8; ++dc) {
          const u32x4 kv = ks[key][dc];
          const float kf[8] = {ss::lo_bf(kv.x), ss::hi_bf(kv.x), ss::lo_bf(kv.y), ss::hi_bf(kv.y),
                               ss::lo_bf(kv.z), ss::hi_bf(kv.z), ss::lo_bf(kv.w), ss::hi_bf(kv.w)};
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const int rr = rg + 4 * t;
            if (rr < nr) {
#pragma unroll
              for (int e = 0; e < 8; ++e) acc[t] += qs[rr][dc * 8 + e] * kf[e];
            }
          }
        }
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int rr = rg + 4 * t;
        if (rr < nr) {
          const int j = (r0 + rr) % a.m;
          const bool ok = key < nk && (k0 + key) <= base + j;
          sc[rr][key] = ok ? acc[t] * scale : -INFINITY;
        }
      }
    }
    __syncthreads();
    // row max / exp / sum: one wave per row, lanes over keys
    {
      const int lane = tid & 63, w = tid >> 6;
      for (int rr = w; rr < nr; rr += 4) {
        const float v = sc[rr][lane];
        const float mx = ss::wave_max(v);
        const float e = (mx == -INFINITY) ? 0.0f : expf(v - mx);
        sc[rr][lane] = e;
        const float sm = ss::wave_sum(e);
        if (lane == 0) {
          rmax[rr] = mx;
          rsum[rr] = sm;
        }
      }
    }
    __syncthreads();
    // o[row][d] = sum_key p * v: thread -> (row, 16 dims)
    for (int e = tid; e < nr * (D / 16); e += 256) {
      const int rr = e / (D / 16), dq = e % (D / 16);
      float o[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) o[t] = 0.0f;
      for (int key = 0; key < nk; ++key) {
        const float p = sc[rr][key];
        const u32x4 v0 = vs[key][2 * dq], v1 = vs[key][2 * dq + 1];
        const uint32_t vw[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          o[2 * t] += p * ss::lo_bf(vw[t]);
          o[2 * t + 1] += p * ss::hi_bf(vw[t]);
        }
      }
      const int r = r0 + rr, g = r / a.m, j = r % a.m;
      float* dst = a.part + ((((int64_t)(hk * G + g) * a.splits + split) * a.m + j) * (D + 2));
#pragma unroll
      for (int t = 0; t < 16; ++t) dst[2 + dq * 16 + t] = o[t];
      if (dq == 0) {
        dst[0] = rmax[rr];
        dst[1] = rsum[rr];
      }
    }
  }
}

__global__ __launch_bounds__(128) void attn_combine_kernel(AttnArgs a) {
  const int hq = blockIdx.x, j = blockIdx.y, dd = threadIdx.x;
  const int base = *a.kv_len + a.pos_offset;
  int n_keys = base + a.m;
  if (n_keys > a.cap) n_keys = a.cap;
  const int active = (n_keys + KPS - 1) / KPS;
  const float* p = a.part + (((int64_t)hq * a.splits) * a.m + j) * (D + 2);
  const int64_t stride = (int64_t)a.m * (D + 2);
  float M = -INFINITY;
  for (int s = 0; s < active; ++s) M = fmaxf(M, p[s * stride]);
  float l = 0.0f, o = 0.0f;
  for (int s = 0; s < active; ++s) {
    const float ms = p[s * stride];
    if (ms == -INFINITY) continue;
    const float f = expf(ms - M);
    l += f * p[s * stride + 1];
    o += f * p[s * stride + 2 + dd];
  }
  a.out[((int64_t)j * a.n_q + hq) * D + dd] = ss::f2bf(o / l);
}

}  // namespace

int attn_keys_per_split() { return KPS; }

hipError_t launch_rope_append(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(rope_append_kernel, dim3(a.m, a.n_q + a.n_kv), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(attn_part_kernel, dim3(a.n_kv, a.splits), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(a.n_q, a.m), dim3(D), 0, s, a);
  return hipGetLastError();
}
