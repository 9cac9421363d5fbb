// Attention over the shared KV cache for the draft step (one query position)
// and the verify pass (gamma+1 query positions, causal: row j sees positions
// [0, kv_len + j]) - "How speculative decoding makes LLMs go brrr", Module 2;
// draft and target read and write one cache ("SubSpec: Speculate Deep and
// Accurate" paper note, Method details, KV-cache sharing).
//
// Kernels:
//  rope_append        rotate-half RoPE of q and k for the verify rows (angles
//                     in float64, applied in float32); q -> q_rot, k/v -> cache.
//  decode_attn        grid (kv head, 128-key split[, row]): per split partial
//                     (max, sum, o[d]) for every query head of the GQA group.
//  rows_merge         merges the verify partials in split order.
// The draft step's partials are merged by the output projection's prologue.
#include "common.h"
#include "internal.h"
#include "profile.h"

namespace {

constexpr int D = 128;     // head dim handled by these kernels

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

// ----------------------------------------------------------------------------
// Decode attention for one query position (the draft step): grid (kv head,
// key split of DKPB keys), 512 threads.  Every block rotates the GQA group's
// queries itself; the block whose split holds the new position rotates the
// new key, appends K/V to the cache and uses them directly (no other block
// reads that position in this launch).  Thread (key j, quarter c) holds 32
// dims of K[j] and V[j]; scores are reduced over the 4 quarters with lane
// shuffles.  Each block writes, per query head of its group, the partial
// (max m, sum l, o[d] = sum_j exp(s_j - m) V[j][d]) of its split; the
// consumer (the output projection's prologue) merges the splits, so no
// block waits on another.
constexpr int DKPB = 128;
constexpr int DREC = 4 + D;  // partial record: m, l, 2 pad, o[D] (16-byte aligned o)

// CACHED = false: the draft step (one row, q and the new k/v rotated and
// appended here).  CACHED = true: verify rows (blockIdx.z = row j at position
// kv_len + j; rope_append already wrote q_rot and the cache), causal limit
// kv_len + j, partials at [kv head][split][row][group head].
template <bool CACHED>
__global__ __launch_bounds__(512) void decode_attn_kernel(AttnArgs a, const int32_t* valid) {
  constexpr int GMAX = 16;
  constexpr int NW = 8;                    // waves per block
  __shared__ float qs[GMAX][D];            // rotated queries (float)
  __shared__ float kn[D];                  // rotated new key
  __shared__ u32x4 vs[DKPB][D / 8 + 1];    // V tile (padded rows)
  __shared__ float ps[GMAX][DKPB];         // probabilities p[h][key]
  __shared__ float wmax[NW][GMAX], wsum[NW][GMAX];
  __shared__ float hmax[GMAX];
  __shared__ float rc[D / 2], rs[D / 2];

  if (valid && *valid == 0) return;
  const int hk = blockIdx.x, split = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int G = a.n_q / a.n_kv;
  const int row = CACHED ? (int)blockIdx.z : 0;
  const int kv0 = *a.kv_len;
  const int pos = kv0 + a.pos_offset + row;  // position of this query (its last key)
  if (pos < 0 || pos >= a.cap) return;
  // key slot t -> cache position: dense t; sparse draft index[t] for t < n_idx,
  // then the speculative positions kv_len + (t - n_idx)
  const bool sparse = !CACHED && a.index != nullptr;
  const int n_idx = sparse ? min(max(*a.n_index, 0), a.index_cap) : 0;
  const int32_t* ilist = sparse ? a.index + (int64_t)hk * a.index_cap : nullptr;
  const int n_keys = sparse ? n_idx + a.pos_offset + 1 : pos + 1;
  const int active = (n_keys + DKPB - 1) / DKPB;
  if (split >= active) return;
  const int k0 = split * DKPB;
  const int nk = min(DKPB, n_keys - k0);
  const bool has_new = !CACHED && (k0 + nk - 1) == n_keys - 1;

  // ---- loads: thread (key j, quarter c) takes 32 dims of K[j] and V[j]
  const int j = tid >> 2, c = tid & 3;
  const bool kvalid = j < nk && (CACHED || (k0 + j) != n_keys - 1);
  u32x4 kr[4], vr[4];
  {
    int t = k0 + (kvalid ? j : 0);
    if (sparse) t = t < n_idx ? min(max(ilist[t], 0), a.cap - 1) : kv0 + (t - n_idx);
    const int64_t row = (int64_t)hk * a.cap + t;
    const u32x4* kp = reinterpret_cast<const u32x4*>(a.k_cache + row * D) + 4 * c;
    const u32x4* vp = reinterpret_cast<const u32x4*>(a.v_cache + row * D) + 4 * c;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kr[i] = kvalid ? kp[i] : u32x4{0u, 0u, 0u, 0u};
      vr[i] = kvalid ? vp[i] : u32x4{0u, 0u, 0u, 0u};
    }
  }
  // ---- RoPE: the 64 angles once per block in float64, applied in float32
  const int half = D / 2;
  if (CACHED) {
    for (int e = tid; e < G * D; e += 512) {
      const int h = e / D, i = e % D;
      qs[h][i] = ss::bf2f(a.q_rot[((int64_t)row * a.n_q + hk * G + h) * D + i]);
    }
  } else if (tid < half) {
    const double inv_freq = exp(-(2.0 * tid / D) * log((double)a.theta));
    double sd, cd;
    sincos((double)pos * inv_freq, &sd, &cd);
    rc[tid] = (float)cd;
    rs[tid] = (float)sd;
  }
  __syncthreads();
  for (int e = tid; !CACHED && e < (G + (has_new ? 1 : 0)) * half; e += 512) {
    const int h = e / half, i = e % half;
    const float cs = rc[i], sn = rs[i];
    const uint16_t* x = (h < G) ? a.qkv + (hk * G + h) * D : a.qkv + (a.n_q + hk) * D;
    const float x1 = ss::bf2f(x[i]), x2 = ss::bf2f(x[i + half]);
    const uint16_t r1 = ss::f2bf(x1 * cs - x2 * sn), r2 = ss::f2bf(x2 * cs + x1 * sn);
    if (h < G) {
      qs[h][i] = ss::bf2f(r1);
      qs[h][i + half] = ss::bf2f(r2);
    } else {
      kn[i] = ss::bf2f(r1);
      kn[i + half] = ss::bf2f(r2);
      uint16_t* kc = a.k_cache + ((int64_t)hk * a.cap + pos) * D;
      kc[i] = r1;
      kc[i + half] = r2;
    }
  }
  if (has_new && tid < D / 8) {
    const u32x4* vsrc = reinterpret_cast<const u32x4*>(a.qkv + (a.n_q + a.n_kv + hk) * D);
    u32x4* vdst = reinterpret_cast<u32x4*>(a.v_cache + ((int64_t)hk * a.cap + pos) * D);
    const u32x4 v = vsrc[tid];
    vdst[tid] = v;
    vs[nk - 1][tid] = v;
  }
  if (kvalid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) vs[j][4 * c + i] = vr[i];
  }
  __syncthreads();
  // ---- scores: 32-dim partial dots, reduced over the 4 quarters of a key
  float kf[32];
  if (!CACHED && j < nk && (k0 + j) == n_keys - 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) kf[i] = kn[32 * c + i];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        kf[8 * i + 2 * t] = ss::lo_bf(w[t]);
        kf[8 * i + 2 * t + 1] = ss::hi_bf(w[t]);
      }
    }
  }
  const float scale = 0.088388347648318440f;  // 1/sqrt(128)
  float sc[GMAX];
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    float d = 0.0f;
    if (h < G) {
#pragma unroll
      for (int i = 0; i < 32; ++i) d += qs[h][32 * c + i] * kf[i];
    }
    d += __shfl_xor(d, 1, 64);
    d += __shfl_xor(d, 2, 64);
    sc[h] = (j < nk) ? d * scale : -INFINITY;
  }
  // ---- softmax statistics per head over the block's keys
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    if (h < G) {
      float m = sc[h];
#pragma unroll
      for (int o = 4; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      if (lane == 0) wmax[wave][h] = m;
    }
  }
  __syncthreads();
  if (tid < G) {
    float m = wmax[0][tid];
    for (int w = 1; w < NW; ++w) m = fmaxf(m, wmax[w][tid]);
    hmax[tid] = m;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    if (h < G) {
      const float p = (j < nk) ? expf(sc[h] - hmax[h]) : 0.0f;
      if (c == 0) ps[h][j] = p;
      float sm = (c == 0) ? p : 0.0f;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) sm += __shfl_xor(sm, o, 64);
      if (lane == 0) wsum[wave][h] = sm;
    }
  }
  __syncthreads();
  // ---- o[h][d] = sum_j p[h][j] V[j][d]: thread -> (head, 2 dims)
  const uint32_t* vw = reinterpret_cast<const uint32_t*>(&vs[0][0]);
  constexpr int VROW = (D / 8 + 1) * 4;  // words per padded V row
  for (int e = tid; e < G * (D / 2); e += 512) {
    const int h = e / (D / 2), dp = e % (D / 2);
    float o0 = 0.f, o1 = 0.f;
#pragma unroll 8
    for (int jj = 0; jj < nk; ++jj) {
      const float p = ps[h][jj];
      const uint32_t v = vw[jj * VROW + dp];
      o0 += p * ss::lo_bf(v);
      o1 += p * ss::hi_bf(v);
    }
    float* dst = a.part + (((int64_t)(hk * a.splits + split) * (CACHED ? a.m : 1) + row) * G + h) * DREC;
    dst[4 + 2 * dp] = o0;
    dst[4 + 2 * dp + 1] = o1;
    if (dp == 0) {
      float l = 0.0f;
      for (int w = 0; w < NW; ++w) l += wsum[w][h];
      dst[0] = hmax[h];
      dst[1] = l;
    }
  }
}

// Merge of the verify partials: grid (q head, row), 128 threads (one per dim);
// splits in order, batches of 4 independent loads.
__global__ __launch_bounds__(128) void rows_merge_kernel(AttnArgs a) {
  const int hq = blockIdx.x, row = blockIdx.y, dd = threadIdx.x;
  const int G = a.n_q / a.n_kv, hk = hq / G, g = hq % G;
  const int pos = *a.kv_len + a.pos_offset + row;
  if (pos < 0 || pos >= a.cap) return;
  const int active = (pos + DKPB) / DKPB;
  const int64_t sstride = (int64_t)a.m * G * DREC;
  const float* base = a.part + (((int64_t)hk * a.splits * a.m + row) * G + g) * DREC;
  float M = -INFINITY, L = 0.0f, o = 0.0f;
  for (int s0 = 0; s0 < active; s0 += 4) {
    float mv[4], lv[4], ov[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bool ok = s0 + t < active;
      const float* q = base + (ok ? s0 + t : 0) * sstride;
      mv[t] = ok ? q[0] : -INFINITY;
      lv[t] = ok ? q[1] : 0.0f;
      ov[t] = ok ? q[4 + dd] : 0.0f;
    }
    float Mb = M;
#pragma unroll
    for (int t = 0; t < 4; ++t) Mb = fmaxf(Mb, mv[t]);
    const float r = (M == -INFINITY) ? 0.0f : expf(M - Mb);
    L *= r;
    o *= r;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float f = (mv[t] == -INFINITY) ? 0.0f : expf(mv[t] - Mb);
      L += f * lv[t];
      o += f * ov[t];
    }
    M = Mb;
  }
  a.out[((int64_t)row * a.n_q + hq) * D + dd] = ss::f2bf(o / L);
  if (a.ml && dd == 0) {
    a.ml[((int64_t)row * a.n_q + hq) * 2] = M;
    a.ml[((int64_t)row * a.n_q + hq) * 2 + 1] = L;
  }
}

// ----------------------------------------------------------------------------
// Importance scores of one layer ("The second ledger of speculative decoding",
// section 3.2): score[hk][j] = sum over the last W verify rows r and the
// query heads h of KV head hk of the attention probability
// exp(q_{r,h} . k_j / sqrt(d) - M_{r,h}) / L_{r,h} (0 past row r's causal
// limit), with (M, L) the softmax statistics the merge wrote.  Grid (KV head,
// block of SKB keys), one thread per key: the thread holds k_j (64 bf16
// pairs) and dots it with the W x G queries staged in LDS as bf16 pairs.
constexpr int SKB = 256;
constexpr int SMAXP = 240;  // W x G pairs that fit the 64 KiB of LDS

__global__ __launch_bounds__(SKB) void attn_scores_kernel(AttnArgs a, float* score, int window) {
  extern __shared__ uint32_t qsm[];  // [P][D/2] query pairs, then [P][2] (M, L)
  const int hk = blockIdx.x, tid = threadIdx.x;
  const int kv0 = *a.kv_len;
  const int n_keys = min(kv0 + a.m, a.cap);
  const int j0 = blockIdx.y * SKB;
  if (kv0 < 0 || j0 >= n_keys) return;  // block-uniform
  const int G = a.n_q / a.n_kv;
  const int W = min(window, a.m), r0 = a.m - W;
  const int P = W * G;
  float* mls = reinterpret_cast<float*>(qsm + P * (D / 2));
  for (int e = tid; e < P * (D / 2); e += SKB) {
    const int p = e / (D / 2), w = e % (D / 2);
    const int r = r0 + p / G, h = p % G;
    qsm[e] = reinterpret_cast<const uint32_t*>(a.q_rot + ((int64_t)r * a.n_q + hk * G + h) * D)[w];
  }
  for (int p = tid; p < P; p += SKB) {
    const int r = r0 + p / G, h = p % G;
    mls[2 * p] = a.ml[((int64_t)r * a.n_q + hk * G + h) * 2];
    mls[2 * p + 1] = a.ml[((int64_t)r * a.n_q + hk * G + h) * 2 + 1];
  }
  __syncthreads();
  const int j = j0 + tid;
  if (j >= n_keys) return;
  uint32_t kw[D / 2];
  const u32x4* kp = reinterpret_cast<const u32x4*>(a.k_cache + ((int64_t)hk * a.cap + j) * D);
#pragma unroll
  for (int i = 0; i < D / 8; ++i) {
    const u32x4 v = kp[i];
    kw[4 * i] = v.x;
    kw[4 * i + 1] = v.y;
    kw[4 * i + 2] = v.z;
    kw[4 * i + 3] = v.w;
  }
  const float scale = 0.088388347648318440f;  // 1/sqrt(128)
  float acc = 0.0f;
  for (int p = 0; p < P; ++p) {
    const int r = r0 + p / G;
    if (j > kv0 + r) continue;  // past row r's causal limit
    const uint32_t* q = qsm + p * (D / 2);
    float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
    for (int w = 0; w < D / 2; w += 2) {
      d0 = ss::dot2(kw[w], q[w], d0);
      d1 = ss::dot2(kw[w + 1], q[w + 1], d1);
    }
    acc += expf((d0 + d1) * scale - mls[2 * p]) / mls[2 * p + 1];
  }
  score[(int64_t)hk * a.cap + j] = acc;
}

}  // namespace

hipError_t launch_rope_append(const AttnArgs& a, hipStream_t s) {
  SS_LAUNCH(rope_append_kernel, dim3(a.m, a.n_q + a.n_kv), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_attention(const AttnArgs& a, const int32_t* valid, hipStream_t s) {
  if (a.n_q / a.n_kv > 16) return hipErrorInvalidValue;
  SS_LAUNCH(decode_attn_kernel<false>, dim3(a.n_kv, a.splits), dim3(512), 0, s, a, valid);
  return hipGetLastError();
}

hipError_t launch_rows_attention(const AttnArgs& a, hipStream_t s) {
  if (a.n_q / a.n_kv > 16) return hipErrorInvalidValue;
  SS_LAUNCH(decode_attn_kernel<true>, dim3(a.n_kv, a.splits, a.m), dim3(512), 0, s, a,
                     (const int32_t*)nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SS_LAUNCH(rows_merge_kernel, dim3(a.n_q, a.m), dim3(D), 0, s, a);
  return hipGetLastError();
}

int decode_attn_keys_per_split() { return DKPB; }

int attn_scores_max_pairs() { return SMAXP; }

hipError_t launch_attn_scores(const AttnArgs& a, float* score, int window, hipStream_t s) {
  const int G = a.n_q / a.n_kv;
  const int P = (window < a.m ? window : a.m) * G;
  if (P > SMAXP || P < 1 || !a.ml) return hipErrorInvalidValue;
  const size_t lds = (size_t)P * (D / 2) * 4 + (size_t)P * 8;
  SS_LAUNCH(attn_scores_kernel, dim3(a.n_kv, (a.cap + SKB - 1) / SKB), dim3(SKB), lds, s, a, score, window);
  return hipGetLastError();
}
