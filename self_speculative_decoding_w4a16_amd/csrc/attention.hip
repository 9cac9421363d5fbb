// Attention over the shared KV cache for the draft step (one query position)
// and the verify pass (gamma+1 query positions, causal: row j sees positions
// [0, kv_len + j]) - "How speculative decoding makes LLMs go brrr", Module 2;
// draft and target read and write one cache ("SubSpec: Speculate Deep and
// Accurate" paper note, Method details, KV-cache sharing).
//
// Kernels (RoPE angles come from a per-step / per-pass table computed in
// float64 and applied in float32):
//  rope_append        rotate-half RoPE of q and k for the verify rows;
//                     q -> q_rot, k/v -> cache.
//  rows_attn          verify: grid (kv head, 128-key split, row): per split
//                     partial (max, sum, o[d]) for every query head of the
//                     GQA group.
//  rows_merge         merges the verify partials in split order.
//  draft_attn         draft step: RoPE + KV append + grid (kv head, 256-key
//                     split) partials, merged by the output projection's
//                     prologue; dense or over the sparse index.
//  attn_scores        verify: importance scores for the sparse draft index.
#include "common.h"
#include "draft_attn.h"
#include "internal.h"
#include "profile.h"

#include <stdlib.h>

namespace {

// Row j of a rows launch (verify pass, tree levels) is node
// t = pos_offset + j * row_stride at slot kv_len + t (AttnArgs).
__device__ __forceinline__ int row_node(const AttnArgs& a, int j) {
  return a.pos_offset + j * (a.row_stride > 1 ? a.row_stride : 1);
}
// Sequence z of a batched launch (AttnArgs.seqs > 1): its kv_len, cache
// heads and rows of every per-row buffer.  The QKV split-k partials keep
// their layout [split][seqs m][columns]: their split stride is seqs m rows.
__device__ __forceinline__ void seq_rebase(AttnArgs& a, int z) {
  if (a.seqs <= 1) return;
  const int G = a.n_q / a.n_kv;
  const int64_t rows = (int64_t)z * a.m;
  a.kv_len += z;
  a.k_cache += (int64_t)z * a.n_kv * a.cap * a.d;
  a.v_cache += (int64_t)z * a.n_kv * a.cap * a.d;
  a.qkv += rows * (a.n_q + 2 * a.n_kv) * a.d;
  if (a.qkv_part) a.qkv_part += rows * (a.n_q + 2 * a.n_kv) * a.d;
  a.q_rot += rows * a.n_q * a.d;
  a.out += rows * a.n_q * a.d;
  a.rope_cs += rows * a.d;
  a.part += (int64_t)z * a.n_kv * a.splits * a.m * G * (a.d + 4);
}
__device__ __forceinline__ int seq_count(const AttnArgs& a) { return a.seqs > 1 ? a.seqs : 1; }

// Lowest slot of node t's own chain in the static tree (tree_d > 0); node t
// sees slots <= kv_len and those from this one up to its own.  0 in a chain.
__device__ __forceinline__ int chain_lo(const AttnArgs& a, int kvl, int t) {
  return (a.tree_d > 0 && t > 0) ? kvl + 1 + ((t - 1) / a.tree_d) * a.tree_d : 0;
}

// RoPE + KV append of the verify rows: grid (row, head), 64 threads (pair
// index i: values i and i + d/2).  With split-k partials of the QKV GEMM
// (S of them; S < 0: a loop) the values are their sums in split order; every
// load (kv_len, the RoPE table, the values) is issued before the first use.
template <int S>
__global__ __launch_bounds__(64) void rope_append_kernel(AttnArgs a) {
  const int z = blockIdx.x / a.m;    // sequence (batched launches)
  const int j = blockIdx.x - z * a.m;  // query row of that sequence
  const int head = blockIdx.y;       // 0..Hq-1: q heads, Hq..Hq+Hkv-1: kv heads
  const int64_t part_rows = (int64_t)a.m * seq_count(a);  // rows of one split of the QKV partials
  seq_rebase(a, z);
  const int i = threadIdx.x;         // pair index 0..d/2-1
  const int half = a.d / 2;
  if (i >= half) return;
  const int kvl = *a.kv_len;
  const int rows = a.n_q + 2 * a.n_kv;
  const float c = a.rope_cs[((int64_t)j * half + i) * 2], s = a.rope_cs[((int64_t)j * half + i) * 2 + 1];
  const bool is_q = head < a.n_q;
  const int hk = head - a.n_q;
  // columns: x = (c0, c1) rotated; for a kv head also v = (c2, c3)
  const int c0 = is_q ? head * a.d + i : (a.n_q + hk) * a.d + i, c1 = c0 + half;
  const int c2 = is_q ? c0 : (a.n_q + a.n_kv + hk) * a.d + i, c3 = c2 + half;
  float x[4];
  if (S == 0) {
    const uint16_t* src = a.qkv + (int64_t)j * rows * a.d;
    x[0] = ss::bf2f(src[c0]);
    x[1] = ss::bf2f(src[c1]);
    x[2] = ss::bf2f(src[c2]);
    x[3] = ss::bf2f(src[c3]);
  } else {
    const int64_t rs = (int64_t)rows * a.d;  // one row of one split
    const float* p = a.qkv_part + (int64_t)j * rs;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    if (S > 0) {
      float pv[S > 0 ? S : 1][4];
#pragma unroll
      for (int sp = 0; sp < S; ++sp) {
        const float* ps = p + (int64_t)sp * part_rows * rs;
        pv[sp][0] = ps[c0];
        pv[sp][1] = ps[c1];
        pv[sp][2] = ps[c2];
        pv[sp][3] = ps[c3];
      }
#pragma unroll
      for (int sp = 0; sp < S; ++sp)  // split order
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += pv[sp][e];
    } else {
      for (int sp = 0; sp < a.qkv_splits; ++sp) {
        const float* ps = p + (int64_t)sp * part_rows * rs;
        acc[0] += ps[c0];
        acc[1] += ps[c1];
        acc[2] += ps[c2];
        acc[3] += ps[c3];
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = ss::bf2f(ss::f2bf(acc[e]));  // the projection output is bf16
  }
  const uint16_t r0 = ss::f2bf(x[0] * c - x[1] * s), r1 = ss::f2bf(x[1] * c + x[0] * s);
  if (is_q) {
    uint16_t* o = a.q_rot + (int64_t)j * a.n_q * a.d + head * a.d;
    o[i] = r0;
    o[i + half] = r1;
  } else {
    const int pos = kvl + row_node(a, j);  // the row's slot
    if (pos < 0 || pos >= a.cap) return;
    uint16_t* kc = a.k_cache + ((int64_t)hk * a.cap + pos) * a.d;
    uint16_t* vc = a.v_cache + ((int64_t)hk * a.cap + pos) * a.d;
    kc[i] = r0;
    kc[i + half] = r1;
    vc[i] = ss::f2bf(x[2]);
    vc[i + half] = ss::f2bf(x[3]);
  }
}

// ----------------------------------------------------------------------------
// Verify attention on the matrix cores: grid (kv head, key split of DKPB =
// 128 keys), 512 threads = 8 waves.  The block takes all m x G queries of
// its kv head (query qi = row j * G + group head h), so the split's K and V
// are read once per layer.  Row j's query sits at position kv_len + j and
// sees keys [0, kv_len + j]; rope_append already wrote q_rot and the rows'
// K/V.
//  * LDS: the K tile [128 keys][d] (B operand of S = Q K^T), the V tile
//    transposed [d][128 keys] (B operand of O = P V), and per wave a P tile
//    [16 queries][128 keys] (A operand of PV, written from the S layout).
//  * Tiles of 16 queries are spread over the waves.  Per tile: S in 8 key
//    tiles x 4 k-steps of v_mfma_f32_16x16x32_bf16 (lane l of the result
//    holds queries 4(l/16)..+3 of key l%16), causal mask, row max and sum over
//    the 128 keys (the 16 lanes of a DPP row), P = exp(S - m) split into bf16
//    hi and lo parts (two MFMAs each: products at fp32 level), O in 8 dim
//    tiles x 4 key steps.
//  * Partials (m, l, o[d]) per (split, row, group head) -- the layout
//    rows_merge reads; rows with no key in the split write none.
constexpr int DKPB = 128;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// max / sum over the 16 lanes of a DPP row (every lane gets the result)
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x141>(v));  // row_half_mirror: the other quad of the half-row
  return fmaxf(v, dpp_f<0x140>(v));  // row_mirror: the other half-row
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  return v + dpp_f<0x140>(v);
}

constexpr int RW = 8;  // waves per block of the verify attention

__global__ __launch_bounds__(RW * 64) void rows_attn_kernel(AttnArgs a) {
  constexpr int NT = 8;            // key tiles of 16 (= DKPB / 16) and dim tiles of 16 (= D / 16)
  constexpr int KROW = D + 8;      // LDS row strides (bf16), padded
  constexpr int VROW = DKPB + 8;
  constexpr int NTH = RW * 64;
  __shared__ __align__(16) uint16_t ks[DKPB][KROW];
  __shared__ __align__(16) uint32_t vt[D][VROW / 2];   // V^T: bf16 pairs of consecutive keys
  __shared__ __align__(16) uint16_t pt[RW][2][16][VROW];  // per wave: P hi, P lo

  const int hk = blockIdx.x, split = blockIdx.y, tid = threadIdx.x;
  seq_rebase(a, blockIdx.z);
  const int lane = tid & 63, wave = tid >> 6, r16 = lane & 15, g4 = lane >> 4;
  const int G = a.n_q / a.n_kv, Qn = a.m * G;
  const int k0 = split * DKPB;
  const int n_tiles = (Qn + 15) / 16;
  // kv_len is read first and used after the tile loads are issued: the K/V
  // rows are clamped to the cache (not to kv_len) and masked when staged
  const int kvl = *a.kv_len;
  const int kv0 = kvl + a.pos_offset;  // slot of row 0

  // A operand of a query tile: lane -> query 16 t + r16, dims 32 s + 8 g4 .. +7
  auto load_q = [&](int t, u32x4 (&qa)[4]) {
    const int qi = 16 * t + r16;
    const bool qok = qi < Qn;
    const int j = qok ? qi / G : 0, h = qok ? qi % G : 0;
    const u32x4* qp = reinterpret_cast<const u32x4*>(a.q_rot + ((int64_t)j * a.n_q + hk * G + h) * D);
#pragma unroll
    for (int st = 0; st < 4; ++st) qa[st] = qok ? qp[4 * st + g4] : u32x4{0u, 0u, 0u, 0u};
  };
  u32x4 qa[4];
  load_q(wave < n_tiles ? wave : 0, qa);

  // ---- K tile, and V^T as pairs of consecutive keys (keys past n_keys are
  // zeros).  V: thread -> (key pair kp, 16-byte piece q) with the 64 lanes of
  // a wave on 64 consecutive pairs, so the transposed stores hit distinct
  // banks.  K (stored row-major): thread -> (piece e % 16, key pair e / 16),
  // so a wave load reads 4 whole 256-byte rows instead of 64 pieces.
  {
    constexpr int PER = (DKPB / 2) * (D / 8) / NTH;  // (pair, piece) items per thread
    u32x4 k2[PER][2], v2[PER][2];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid + NTH * i, kp = e & (DKPB / 2 - 1), q = e / (DKPB / 2);
      const int kpk = e / (D / 8), qk = e & (D / 8 - 1);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int64_t row = (int64_t)hk * a.cap + min(k0 + 2 * kp + u, a.cap - 1);
        const int64_t rowk = (int64_t)hk * a.cap + min(k0 + 2 * kpk + u, a.cap - 1);
        k2[i][u] = reinterpret_cast<const u32x4*>(a.k_cache + rowk * D)[qk];
        v2[i][u] = reinterpret_cast<const u32x4*>(a.v_cache + row * D)[q];
      }
    }
    const int n_keys = min(kvl + row_node(a, a.m - 1) + 1, a.cap);  // keys of the last row in range
    if (kv0 < 0 || n_keys <= 0 || split >= (n_keys + DKPB - 1) / DKPB) return;  // block-uniform
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid + NTH * i, kp = e & (DKPB / 2 - 1), q = e / (DKPB / 2);
      const int kpk = e / (D / 8), qk = e & (D / 8 - 1);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (k0 + 2 * kpk + u >= n_keys) k2[i][u] = u32x4{0u, 0u, 0u, 0u};
        if (k0 + 2 * kp + u >= n_keys) v2[i][u] = u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) *reinterpret_cast<u32x4*>(&ks[2 * kpk + u][8 * qk]) = k2[i][u];
      const uint32_t w0[4] = {v2[i][0].x, v2[i][0].y, v2[i][0].z, v2[i][0].w};
      const uint32_t w1[4] = {v2[i][1].x, v2[i][1].y, v2[i][1].z, v2[i][1].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        vt[8 * q + 2 * t][kp] = (w0[t] & 0xffffu) | (w1[t] << 16);
        vt[8 * q + 2 * t + 1][kp] = (w0[t] >> 16) | (w1[t] & 0xffff0000u);
      }
    }
  }
  __syncthreads();

  const float scale = 0.088388347648318440f;  // 1/sqrt(128)
  const uint16_t* vt16 = reinterpret_cast<const uint16_t*>(&vt[0][0]);
  for (int t = wave; t < n_tiles; t += RW) {
    if (t != wave) load_q(t, qa);
    // S = Q K^T
    f32x4_t sa[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      sa[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const u32x4 b = *reinterpret_cast<const u32x4*>(&ks[16 * n + r16][32 * st + 8 * g4]);
        sa[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qa[st]),
                                                        __builtin_bit_cast(bf16x8_t, b), sa[n], 0, 0, 0);
      }
    }
    // causal (or tree) mask, row max / sum; this lane's queries are 16 t + 4 g4 + i
    float mx[4], sm[4];
    int qrow[4];
    bool qv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int qi = 16 * t + 4 * g4 + i;
      qv[i] = qi < Qn;
      qrow[i] = qv[i] ? qi / G : 0;
      const int tn = row_node(a, qrow[i]);
      const int last_key = kvl + tn;  // this row's own slot
      const int lo = chain_lo(a, kvl, tn);
      qv[i] = qv[i] && last_key < a.cap && k0 <= last_key;
      float m = -INFINITY;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const int key = k0 + 16 * n + r16;
        const bool ok = qv[i] && key <= last_key && (key <= kvl || key >= lo);
        sa[n][i] = ok ? sa[n][i] * scale : -INFINITY;
        m = fmaxf(m, sa[n][i]);
      }
      mx[i] = row16_max(m);
      float l = 0.0f;
#pragma unroll
      for (int n = 0; n < NT; ++n) {  // exp(x) as 2^(x log2 e)
        const float p = (mx[i] == -INFINITY) ? 0.0f
                                             : __builtin_amdgcn_exp2f((sa[n][i] - mx[i]) * 1.4426950408889634f);
        sa[n][i] = p;
        l += p;
      }
      sm[i] = row16_sum(l);
    }
    // P (hi, lo bf16) into this wave's tile: [query 4 g4 + i][key 16 n + r16]
#pragma unroll
    for (int n = 0; n < NT; ++n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = sa[n][i];
        const uint16_t hi = ss::f2bf(p);
        pt[wave][0][4 * g4 + i][16 * n + r16] = hi;
        pt[wave][1][4 * g4 + i][16 * n + r16] = ss::f2bf(p - ss::bf2f(hi));
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    // O = P V: A = P [query r16][keys 32 st + 8 g4 ..], B = V^T [dim 16 n + r16][keys ..]
    f32x4_t oa[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) oa[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const u32x4 ph = *reinterpret_cast<const u32x4*>(&pt[wave][0][r16][32 * st + 8 * g4]);
      const u32x4 pl = *reinterpret_cast<const u32x4*>(&pt[wave][1][r16][32 * st + 8 * g4]);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const u32x4 b = *reinterpret_cast<const u32x4*>(vt16 + (16 * n + r16) * VROW + 32 * st + 8 * g4);
        oa[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ph),
                                                        __builtin_bit_cast(bf16x8_t, b), oa[n], 0, 0, 0);
        oa[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, pl),
                                                        __builtin_bit_cast(bf16x8_t, b), oa[n], 0, 0, 0);
      }
    }
    __builtin_amdgcn_wave_barrier();  // the P tile is rewritten by the next query tile
    // partials of this lane's queries: o[dim 16 n + r16]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!qv[i]) continue;
      const int qi = 16 * t + 4 * g4 + i, h = qi % G;
      float* dst = a.part + (((int64_t)(hk * a.splits + split) * a.m + qrow[i]) * G + h) * DREC;
#pragma unroll
      for (int n = 0; n < NT; ++n) dst[4 + 16 * n + r16] = oa[n][i];
      if (r16 == 0) {
        dst[0] = mx[i];
        dst[1] = sm[i];
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Draft-step attention (one query position; the split-key decode of "How
// speculative decoding makes LLMs go brrr", Module 2, memory-bound): grid
// (kv head, split of DSK = 64 keys), 256 threads = 4 waves of 16 keys, G (the
// GQA group size) a template constant.  Small splits keep many compute units
// busy; draft_merge combines the splits afterwards.
//  * Every load is issued first: lane (key l%16, quarter l/16) takes a
//    quarter of its key's K row (64 B); lane l takes the 4-byte V slice
//    (dims 2l, 2l+1) of each of its wave's 16 keys; thread e takes the q (or
//    new k) pairs it rotates and their RoPE table entries.  Positions are
//    clamped and masked, not branched.
//  * Rotation of the group's queries and, in the block that holds it, the
//    new key; the new K/V is appended to the cache.
//  * Scores: each quarter dots its 32 dims with the G queries (v_dot2 on
//    bf16 pairs in LDS), quarters added by two lane swaps; softmax
//    statistics per wave over its 16 keys.
//  * PV: lane = dimension pair over the wave's keys; the 4 waves combine in
//    LDS into the block's partial (m, l, o[d]) per query head.
//  * Sparse draft: key slots map to the index list, then to the speculative
//    positions kv_len .. kv_len + step.
constexpr int DSK = 64;

template <int G>
__global__ __launch_bounds__(256) void draft_attn_kernel(AttnArgs a, const int32_t* valid) {
  constexpr int NWV = 4, KW = 16;
  constexpr int NROT = (G + 1) * (D / 4);  // rotation items: pairs (2i, 2i+1) of q heads and new k
  __shared__ __align__(16) uint32_t qp[G][D / 2];  // rotated queries, bf16 pairs
  __shared__ __align__(16) uint32_t knew[D / 2];   // rotated new key, bf16 pairs
  __shared__ uint32_t vnew[D / 2];                 // new value, bf16 pairs
  __shared__ __align__(16) float ps[NWV][G][KW];   // probabilities per wave, head, key
  __shared__ float wm[NWV][G], wl[NWV][G];
  __shared__ float wo[NWV][G][D];

  const int vflag = valid ? *valid : 1;
  const int hk = blockIdx.x, split = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const DraftKeys ks = draft_keys(a, hk);
  if (vflag == 0 || ks.pos < 0 || ks.pos >= a.cap) return;
  const int active = (ks.n_keys + DSK - 1) / DSK;
  if (split >= active) return;
  const int k0 = split * DSK;
  const int kend = min(k0 + DSK, ks.n_keys);  // slots [k0, kend) of this block
  const bool has_new = kend == ks.n_keys;     // the new key is slot n_keys - 1
  const int wk0 = k0 + KW * wave;             // first slot of this wave
  auto slot_pos = [&](int t) {
    if (!ks.ilist) return t;
    const int ti = min(t, max(ks.n_idx - 1, 0));
    const int ip = min(max(ks.ilist[ti], 0), a.cap - 1);
    return t < ks.n_idx ? ip : ks.kv0 + (t - ks.n_idx);
  };
  const uint16_t* kc = a.k_cache + (int64_t)hk * a.cap * D;
  const uint16_t* vc = a.v_cache + (int64_t)hk * a.cap * D;

  // ---- loads
  const int kl = lane & (KW - 1), kq = lane >> 4;
  const int my_slot = wk0 + kl;
  const bool kin = my_slot < kend;
  const bool k_is_new = kin && my_slot == ks.n_keys - 1;
  const bool kload = kin && !k_is_new;
  u32x4 kr[D / 32];
  {
    const u32x4* kp =
        reinterpret_cast<const u32x4*>(kc + (int64_t)slot_pos(kload ? my_slot : k0) * D) + kq * (D / 32);
#pragma unroll
    for (int i = 0; i < D / 32; ++i) kr[i] = kp[i];
  }
  uint32_t vv[KW];
  const int last_old = min(kend, ks.n_keys - 1);  // V of slots [.., last_old) comes from the cache
#pragma unroll
  for (int kk = 0; kk < KW; ++kk) {
    const int t = wk0 + kk;  // wave-uniform
    vv[kk] = reinterpret_cast<const uint32_t*>(vc + (int64_t)slot_pos(t < last_old ? t : k0) * D)[lane];
  }
  // rotation inputs: item e = (head h, pair index i2): x[2 i2], x[2 i2 + 1] and
  // x[64 + 2 i2], x[64 + 2 i2 + 1], with their (cos, sin)
  const int half = D / 2;
  uint32_t xlo[(NROT + 255) / 256], xhi[(NROT + 255) / 256];
  f32x4_t cs[(NROT + 255) / 256];
#pragma unroll
  for (int r = 0; r < (NROT + 255) / 256; ++r) {
    const int e = tid + 256 * r;
    const int h = e / (half / 2), i2 = e % (half / 2);
    const bool ok = e < NROT && (h < G || has_new);
    const uint16_t* x = (h < G) ? a.qkv + (hk * G + h) * D : a.qkv + (a.n_q + hk) * D;
    xlo[r] = ok ? reinterpret_cast<const uint32_t*>(x)[i2] : 0u;
    xhi[r] = ok ? reinterpret_cast<const uint32_t*>(x + half)[i2] : 0u;
    cs[r] = ok ? reinterpret_cast<const f32x4_t*>(a.rope_cs)[i2] : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const uint32_t vn_src = (has_new && tid < D / 2)
                              ? reinterpret_cast<const uint32_t*>(a.qkv + (a.n_q + a.n_kv + hk) * D)[tid]
                              : 0u;

  // ---- RoPE rotation of the group's queries (and the new key)
#pragma unroll
  for (int r = 0; r < (NROT + 255) / 256; ++r) {
    const int e = tid + 256 * r;
    const int h = e / (half / 2), i2 = e % (half / 2);
    if (e < NROT && (h < G || has_new)) {
      // cs = (cos_i, sin_i, cos_{i+1}, sin_{i+1}) for i = 2 i2
      const float a1 = ss::lo_bf(xlo[r]), b1 = ss::hi_bf(xlo[r]);  // x[i], x[i+1]
      const float a2 = ss::lo_bf(xhi[r]), b2 = ss::hi_bf(xhi[r]);  // x[i+64], x[i+65]
      const uint32_t lo = ss::pack_bf(ss::f2bf(a1 * cs[r][0] - a2 * cs[r][1]),
                                      ss::f2bf(b1 * cs[r][2] - b2 * cs[r][3]));
      const uint32_t hi = ss::pack_bf(ss::f2bf(a2 * cs[r][0] + a1 * cs[r][1]),
                                      ss::f2bf(b2 * cs[r][2] + b1 * cs[r][3]));
      if (h < G) {
        qp[h][i2] = lo;
        qp[h][half / 2 + i2] = hi;
      } else {
        knew[i2] = lo;
        knew[half / 2 + i2] = hi;
        uint32_t* kdst = reinterpret_cast<uint32_t*>(a.k_cache + ((int64_t)hk * a.cap + ks.pos) * D);
        kdst[i2] = lo;
        kdst[half / 2 + i2] = hi;
      }
    }
  }
  if (has_new && tid < D / 2) {
    vnew[tid] = vn_src;
    reinterpret_cast<uint32_t*>(a.v_cache + ((int64_t)hk * a.cap + ks.pos) * D)[tid] = vn_src;
  }
  __syncthreads();

  // ---- scores: lane (key, quarter) dots its 32 dims; quarters added by lane swaps
  if (k_is_new) {
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      const int w = kq * (D / 8) + 4 * i;
      kr[i] = u32x4{knew[w], knew[w + 1], knew[w + 2], knew[w + 3]};
    }
  }
  const float scale = 0.088388347648318440f;  // 1/sqrt(128)
  float sc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      const u32x4 q = *reinterpret_cast<const u32x4*>(&qp[h][kq * (D / 8) + 4 * i]);
      d0 = ss::dot2(kr[i].x, q.x, d0);
      d1 = ss::dot2(kr[i].y, q.y, d1);
      d0 = ss::dot2(kr[i].z, q.z, d0);
      d1 = ss::dot2(kr[i].w, q.w, d1);
    }
    float d = d0 + d1;
    d += __shfl_xor(d, 16, 64);
    d += __shfl_xor(d, 32, 64);
    sc[h] = kin ? d * scale : -INFINITY;
  }
  // ---- per-wave softmax statistics over the wave's 16 keys
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float m = sc[h];
#pragma unroll
    for (int o = 1; o < KW; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    const float p = kin ? expf(sc[h] - m) : 0.0f;
    float l = p;
#pragma unroll
    for (int o = 1; o < KW; o <<= 1) l += __shfl_xor(l, o, 64);
    if (kq == 0) ps[wave][h][kl] = p;
    if (lane == 0) {
      wm[wave][h] = m;
      wl[wave][h] = l;
    }
  }
  __syncthreads();
  // ---- PV: lane = dimension pair over the wave's keys
  const int new_kk = (has_new && ks.n_keys - 1 >= wk0 && ks.n_keys - 1 < wk0 + KW) ? ks.n_keys - 1 - wk0 : -1;
  const uint32_t vn = vnew[lane];
  float vlo[KW], vhi[KW];
#pragma unroll
  for (int kk = 0; kk < KW; ++kk) {
    const uint32_t v = (kk == new_kk) ? vn : vv[kk];
    vlo[kk] = ss::lo_bf(v);
    vhi[kk] = ss::hi_bf(v);
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float o0 = 0.0f, o1 = 0.0f;
#pragma unroll
    for (int kk = 0; kk < KW; kk += 4) {
      const f32x4_t p4 = *reinterpret_cast<const f32x4_t*>(&ps[wave][h][kk]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        o0 += p4[u] * vlo[kk + u];
        o1 += p4[u] * vhi[kk + u];
      }
    }
    wo[wave][h][2 * lane] = o0;
    wo[wave][h][2 * lane + 1] = o1;
  }
  __syncthreads();
  // ---- combine the 4 waves into the block's partial per query head
  for (int e = tid; e < G * D; e += 256) {
    const int h = e / D, dd = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWV; ++w) M = fmaxf(M, wm[w][h]);
    float L = 0.0f, o = 0.0f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      const float f = (wm[w][h] == -INFINITY) ? 0.0f : expf(wm[w][h] - M);
      L += f * wl[w][h];
      o += f * wo[w][h][dd];
    }
    float* dst = a.part + ((int64_t)(hk * a.splits + split) * G + h) * DREC;
    dst[4 + dd] = o;
    if (dd == 0) {
      dst[0] = M;
      dst[1] = L;
    }
  }
}

// The per-head draft attention (short contexts): grid (query head, split),
// the body in draft_attn.h.
template <bool SPARSE, int DQR, bool REFILL>
__global__ __launch_bounds__(DQW * 64) void draft_attn_head_kernel(AttnArgs a, const int32_t* valid) {
  draft_attn_head<SPARSE, DQR, REFILL, false>(a, valid, blockIdx.x, blockIdx.y, gridDim.y, nullptr);
}


// Merge of one row's split partials (m, l, o[D]) by a block of MP x D
// threads: thread (dim dd, group p) merges splits p, p + MP, ... in order,
// 8 independent loads at a time (so a long context costs active / (8 MP)
// memory round trips, not active / 8), then the MP group results are
// combined in group order through LDS.  Returns (M, L, o) in the threads of
// group 0; natural-log units.
constexpr int MP = 8;  // split groups per merge block
constexpr int kSeqMergeSplits = 32;  // verify merges with at most this many splits walk them in one thread
__device__ __forceinline__ void merge_rows(const float* base, int64_t sstride, int active, int dd, int p,
                                           float& M, float& L, float& o) {
  __shared__ float gm[MP], gl[MP], go[MP][D];
  M = -INFINITY;
  L = 0.0f;
  o = 0.0f;
  for (int s0 = p; s0 < active; s0 += 8 * MP) {
    float mv[8], lv[8], ov[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int sp = s0 + t * MP;
      const bool ok = sp < active;
      const float* q = base + (ok ? sp : 0) * sstride;
      mv[t] = ok ? q[0] : -INFINITY;
      lv[t] = ok ? q[1] : 0.0f;
      ov[t] = ok ? q[4 + dd] : 0.0f;
    }
    float Mb = M;
#pragma unroll
    for (int t = 0; t < 8; ++t) Mb = fmaxf(Mb, mv[t]);
    const float r = (M == -INFINITY) ? 0.0f : expf(M - Mb);
    L *= r;
    o *= r;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float f = (mv[t] == -INFINITY) ? 0.0f : expf(mv[t] - Mb);
      L += f * lv[t];
      o += f * ov[t];
    }
    M = Mb;
  }
  go[p][dd] = o;
  if (dd == 0) {
    gm[p] = M;
    gl[p] = L;
  }
  __syncthreads();
  if (p == 0) {
    float Mt = -INFINITY;
#pragma unroll
    for (int q = 0; q < MP; ++q) Mt = fmaxf(Mt, gm[q]);
    float Lt = 0.0f, ot = 0.0f;
#pragma unroll
    for (int q = 0; q < MP; ++q) {
      const float f = (gm[q] == -INFINITY) ? 0.0f : expf(gm[q] - Mt);
      Lt += f * gl[q];
      ot += f * go[q][dd];
    }
    M = Mt;
    L = Lt;
    o = ot;
  }
}

// Merge of the draft step's split partials: grid (q head), MP x 128 threads.
// Writes the attention output (bf16) that the output projection reads.
__global__ __launch_bounds__(MP * D) void draft_merge_kernel(AttnArgs a, const int32_t* valid) {
  const int vflag = valid ? *valid : 1;
  const int hq = blockIdx.x, dd = threadIdx.x % D, p = threadIdx.x / D;
  const int G = a.n_q / a.n_kv, hk = hq / G, g = hq % G;
  const DraftKeys ks = draft_keys(a, hk);
  if (vflag == 0 || ks.pos < 0 || ks.pos >= a.cap) return;
  const int active = min((ks.n_keys + DSK - 1) / DSK, a.splits);
  float M, L, o;
  merge_rows(a.part + ((int64_t)hk * a.splits * G + g) * DREC, (int64_t)G * DREC, active, dd, p, M, L, o);
  if (p == 0) a.out[(int64_t)hq * D + dd] = ss::f2bf(o / L);
}

// Verify attention for long contexts: as rows_attn_kernel, but one block
// walks a.split_keys / 128 consecutive 128-key tiles of its kv head, keeping
// per query row a running (max, sum, o) across them, and the next tile's K/V
// are loaded into registers while the current one is used from LDS, so the
// loads overlap the arithmetic and the partials (and the merge) shrink by the
// tile count.  Needs at most one query tile per wave (m x G <= 16 RW rows).
__global__ __launch_bounds__(RW * 64) void rows_attn_long_kernel(AttnArgs a) {
  constexpr int NT = 8;
  constexpr int KROW = D + 8;
  constexpr int VROW = DKPB + 8;
  constexpr int NTH = RW * 64;
  constexpr int PER = (DKPB / 2) * (D / 8) / NTH;
  __shared__ __align__(16) uint16_t ks[DKPB][KROW];
  __shared__ __align__(16) uint32_t vt[D][VROW / 2];
  __shared__ __align__(16) uint16_t pt[RW][2][16][VROW];

  const int hk = blockIdx.x, split = blockIdx.y, tid = threadIdx.x;
  seq_rebase(a, blockIdx.z);
  const int lane = tid & 63, wave = tid >> 6, r16 = lane & 15, g4 = lane >> 4;
  const int G = a.n_q / a.n_kv, Qn = a.m * G;
  const int n_tiles = (Qn + 15) / 16;
  const int kbase = split * a.split_keys;
  const bool has_q = wave < n_tiles;  // this wave's query tile: wave
  const int t = has_q ? wave : 0;

  u32x4 qa[4];
  {
    const int qi = 16 * t + r16;
    const bool qok = has_q && qi < Qn;
    const int j = qok ? qi / G : 0, h = qok ? qi % G : 0;
    const u32x4* qp = reinterpret_cast<const u32x4*>(a.q_rot + ((int64_t)j * a.n_q + hk * G + h) * D);
#pragma unroll
    for (int st = 0; st < 4; ++st) qa[st] = qok ? qp[4 * st + g4] : u32x4{0u, 0u, 0u, 0u};
  }
  // K/V of tile tau into registers.  V: thread -> (key pair kp, 16-byte
  // piece q), the layout its transpose into LDS needs (a wave load touches 64
  // rows).  K, stored row-major: thread -> (piece e % 16, key pair e / 16),
  // so a wave load reads 4 whole 256-byte rows.
  u32x4 k2[PER][2], v2[PER][2];
  auto load_tile = [&](int tau) {
    const int k0 = kbase + tau * DKPB;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid + NTH * i, kp = e & (DKPB / 2 - 1), q = e / (DKPB / 2);
      const int kpk = e / (D / 8), qk = e & (D / 8 - 1);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int64_t row = (int64_t)hk * a.cap + min(k0 + 2 * kp + u, a.cap - 1);
        const int64_t rowk = (int64_t)hk * a.cap + min(k0 + 2 * kpk + u, a.cap - 1);
        k2[i][u] = reinterpret_cast<const u32x4*>(a.k_cache + rowk * D)[qk];
        v2[i][u] = reinterpret_cast<const u32x4*>(a.v_cache + row * D)[q];
      }
    }
  };
  load_tile(0);
  const int kvl = *a.kv_len;
  const int kv0 = kvl + a.pos_offset;  // slot of row 0
  const int n_keys = min(kvl + row_node(a, a.m - 1) + 1, a.cap);
  if (kv0 < 0 || n_keys <= kbase) return;  // block-uniform
  const int n_tau = min(a.split_keys / DKPB, (n_keys - kbase + DKPB - 1) / DKPB);

  float Mr[4], Lr[4];
  f32x4_t O[NT];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    Mr[i] = -INFINITY;
    Lr[i] = 0.0f;
  }
#pragma unroll
  for (int n = 0; n < NT; ++n) O[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const float scale = 0.088388347648318440f;  // 1/sqrt(128)
  const uint16_t* vt16 = reinterpret_cast<const uint16_t*>(&vt[0][0]);

  for (int tau = 0; tau < n_tau; ++tau) {
    const int k0 = kbase + tau * DKPB;
    if (tau > 0) __syncthreads();  // every wave is done with the previous tile
    // stage tile tau (keys past n_keys as zeros)
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid + NTH * i, kp = e & (DKPB / 2 - 1), q = e / (DKPB / 2);
      const int kpk = e / (D / 8), qk = e & (D / 8 - 1);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (k0 + 2 * kpk + u >= n_keys) k2[i][u] = u32x4{0u, 0u, 0u, 0u};
        if (k0 + 2 * kp + u >= n_keys) v2[i][u] = u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) *reinterpret_cast<u32x4*>(&ks[2 * kpk + u][8 * qk]) = k2[i][u];
      const uint32_t w0[4] = {v2[i][0].x, v2[i][0].y, v2[i][0].z, v2[i][0].w};
      const uint32_t w1[4] = {v2[i][1].x, v2[i][1].y, v2[i][1].z, v2[i][1].w};
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        vt[8 * q + 2 * tt][kp] = (w0[tt] & 0xffffu) | (w1[tt] << 16);
        vt[8 * q + 2 * tt + 1][kp] = (w0[tt] >> 16) | (w1[tt] & 0xffff0000u);
      }
    }
    __syncthreads();
    // the next tile's loads overlap this tile's arithmetic (past the block's
    // tiles they read clamped rows that are never staged)
    load_tile(tau + 1 < n_tau ? tau + 1 : tau);
    if (!has_q) continue;
    // S = Q K^T
    f32x4_t sa[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      sa[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const u32x4 b = *reinterpret_cast<const u32x4*>(&ks[16 * n + r16][32 * st + 8 * g4]);
        sa[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qa[st]),
                                                        __builtin_bit_cast(bf16x8_t, b), sa[n], 0, 0, 0);
      }
    }
    float mx[4], sm[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int qi = 16 * t + 4 * g4 + i;
      const bool qv = qi < Qn;
      const int tn = row_node(a, qv ? qi / G : 0);
      const int last_key = kvl + tn;
      const int lo = chain_lo(a, kvl, tn);
      const bool any = qv && last_key < a.cap && k0 <= last_key;
      float m = -INFINITY;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const int key = k0 + 16 * n + r16;
        const bool ok = any && key <= last_key && (key <= kvl || key >= lo);
        sa[n][i] = ok ? sa[n][i] * scale : -INFINITY;
        m = fmaxf(m, sa[n][i]);
      }
      mx[i] = row16_max(m);
      float l = 0.0f;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const float pv = (mx[i] == -INFINITY) ? 0.0f
                                              : __builtin_amdgcn_exp2f((sa[n][i] - mx[i]) * 1.4426950408889634f);
        sa[n][i] = pv;
        l += pv;
      }
      sm[i] = row16_sum(l);
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = sa[n][i];
        const uint16_t hi = ss::f2bf(pv);
        pt[wave][0][4 * g4 + i][16 * n + r16] = hi;
        pt[wave][1][4 * g4 + i][16 * n + r16] = ss::f2bf(pv - ss::bf2f(hi));
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    f32x4_t oa[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) oa[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const u32x4 ph = *reinterpret_cast<const u32x4*>(&pt[wave][0][r16][32 * st + 8 * g4]);
      const u32x4 pl = *reinterpret_cast<const u32x4*>(&pt[wave][1][r16][32 * st + 8 * g4]);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const u32x4 b = *reinterpret_cast<const u32x4*>(vt16 + (16 * n + r16) * VROW + 32 * st + 8 * g4);
        oa[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ph),
                                                        __builtin_bit_cast(bf16x8_t, b), oa[n], 0, 0, 0);
        oa[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, pl),
                                                        __builtin_bit_cast(bf16x8_t, b), oa[n], 0, 0, 0);
      }
    }
    __builtin_amdgcn_wave_barrier();  // the P tile is rewritten by the next key tile
    // fold the tile into the running (max, sum, o) of this lane's rows
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (mx[i] == -INFINITY) continue;
      const float Mn = fmaxf(Mr[i], mx[i]);
      const float fo = (Mr[i] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((Mr[i] - Mn) * 1.4426950408889634f);
      const float fn = __builtin_amdgcn_exp2f((mx[i] - Mn) * 1.4426950408889634f);
      Lr[i] = Lr[i] * fo + sm[i] * fn;
#pragma unroll
      for (int n = 0; n < NT; ++n) O[n][i] = O[n][i] * fo + oa[n][i] * fn;
      Mr[i] = Mn;
    }
  }
  if (!has_q) return;
  // partials of this lane's rows whose own slot is at or past this split (the
  // merge reads every split up to the row's slot; in a tree a split can hold
  // only other chains' keys: then the partial is (-inf, 0, 0))
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int qi = 16 * t + 4 * g4 + i;
    if (qi >= Qn) continue;
    const int row = qi / G, h = qi % G;
    if (kvl + row_node(a, row) < kbase) continue;
    float* dst = a.part + (((int64_t)(hk * a.splits + split) * a.m + row) * G + h) * DREC;
#pragma unroll
    for (int n = 0; n < NT; ++n) dst[4 + 16 * n + r16] = O[n][i];
    if (r16 == 0) {
      dst[0] = Mr[i];
      dst[1] = Lr[i];
    }
  }
}

// Merge of the verify partials, few splits (short contexts): grid (q head,
// row), 128 threads (one per dim); splits in order, batches of 4 independent
// loads, the first batch loaded before kv_len is known.
__global__ __launch_bounds__(128) void rows_merge_seq_kernel(AttnArgs a) {
  constexpr int B = 4;  // splits per batch of independent loads
  const int hq = blockIdx.x, dd = threadIdx.x;
  const int z = blockIdx.y / a.m, row = blockIdx.y - z * a.m;  // sequence, its row
  seq_rebase(a, z);
  const int G = a.n_q / a.n_kv, hk = hq / G, g = hq % G;
  const int64_t sstride = (int64_t)a.m * G * DREC;
  const float* base = a.part + (((int64_t)hk * a.splits * a.m + row) * G + g) * DREC;
  float mv[B], lv[B], ov[B];
  auto load = [&](int s0) {
#pragma unroll
    for (int t = 0; t < B; ++t) {
      const float* q = base + min(s0 + t, a.splits - 1) * sstride;
      mv[t] = q[0];
      lv[t] = q[1];
      ov[t] = q[4 + dd];
    }
  };
  load(0);
  const int pos = *a.kv_len + row_node(a, row);  // the row's slot: its last key
  if (pos < 0 || pos >= a.cap) return;
  const int kps = a.split_keys > 0 ? a.split_keys : DKPB;
  const int active = (pos + kps) / kps;
  float M = -INFINITY, L = 0.0f, o = 0.0f;
  for (int s0 = 0; s0 < active; s0 += B) {
    if (s0 > 0) load(s0);
#pragma unroll
    for (int t = 0; t < B; ++t) {
      const bool ok = s0 + t < active;
      mv[t] = ok ? mv[t] : -INFINITY;
      lv[t] = ok ? lv[t] : 0.0f;
      ov[t] = ok ? ov[t] : 0.0f;
    }
    float Mb = M;
#pragma unroll
    for (int t = 0; t < B; ++t) Mb = fmaxf(Mb, mv[t]);
    const float r = (M == -INFINITY) ? 0.0f : expf(M - Mb);
    L *= r;
    o *= r;
#pragma unroll
    for (int t = 0; t < B; ++t) {
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

// Merge of the verify partials, many splits (long contexts): grid (q head,
// row), MP x 128 threads.
__global__ __launch_bounds__(MP * D) void rows_merge_kernel(AttnArgs a) {
  const int hq = blockIdx.x, dd = threadIdx.x % D, p = threadIdx.x / D;
  const int z = blockIdx.y / a.m, row = blockIdx.y - z * a.m;  // sequence, its row
  seq_rebase(a, z);
  const int G = a.n_q / a.n_kv, hk = hq / G, g = hq % G;
  const int pos = *a.kv_len + row_node(a, row);  // the row's slot: its last key
  if (pos < 0 || pos >= a.cap) return;
  const int kps = a.split_keys > 0 ? a.split_keys : DKPB;
  const int active = (pos + kps) / kps;
  float M, L, o;
  merge_rows(a.part + (((int64_t)hk * a.splits * a.m + row) * G + g) * DREC, (int64_t)a.m * G * DREC, active,
             dd, p, M, L, o);
  if (p != 0) return;
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
// block of SKB = 128 keys), 4 waves: the key tile is staged in LDS and the
// scores of the P = W x G queries against it come from the matrix cores
// (v_mfma_f32_16x16x32_bf16, query tiles of 16 spread over the waves); each
// probability tile is summed over its 16 queries, then the waves' sums are
// added in wave order.
constexpr int SKB = 128;
constexpr int SMAXP = 240;  // W x G queries (15 tiles of 16)
constexpr int SW = 4;       // waves of the score kernel

__global__ __launch_bounds__(SW * 64) void attn_scores_kernel(AttnArgs a, float* score, int window) {
  constexpr int KROW = D + 8;  // padded LDS row (bf16)
  __shared__ __align__(16) uint16_t ks[SKB][KROW];
  __shared__ float mls[SMAXP][2];
  __shared__ float red[SW][SKB];
  const int hk = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, r16 = lane & 15, g4 = lane >> 4;
  const int G = a.n_q / a.n_kv;
  const int W = min(window, a.m), r0 = a.m - W;
  const int P = W * G, n_qt = (P + 15) / 16;
  const int j0 = blockIdx.y * SKB;
  // the key tile (rows clamped to the cache; keys past n_keys are never
  // written out) is loaded before kv_len is read
  constexpr int PER = SKB * (D / 8) / (SW * 64);  // 16-byte pieces per thread
  u32x4 kv[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = tid + SW * 64 * i, key = e / (D / 8), q = e % (D / 8);
    const int64_t row = (int64_t)hk * a.cap + min(j0 + key, a.cap - 1);
    kv[i] = reinterpret_cast<const u32x4*>(a.k_cache + row * D)[q];
  }
  const int kv0 = *a.kv_len;
  const int n_keys = min(kv0 + a.m, a.cap);
  if (kv0 < 0 || j0 >= n_keys) return;  // block-uniform
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = tid + SW * 64 * i, key = e / (D / 8), q = e % (D / 8);
    *reinterpret_cast<u32x4*>(&ks[key][8 * q]) = kv[i];
  }
  for (int p = tid; p < P; p += SW * 64) {
    const int r = r0 + p / G, h = p % G;
    mls[p][0] = a.ml[((int64_t)r * a.n_q + hk * G + h) * 2];
    mls[p][1] = a.ml[((int64_t)r * a.n_q + hk * G + h) * 2 + 1];
  }
  __syncthreads();

  const float scale = 0.088388347648318440f;  // 1/sqrt(128)
  float acc[SKB / 16];  // this wave's sum for key 16 n + r16 (lanes g4 == 0)
#pragma unroll
  for (int n = 0; n < SKB / 16; ++n) acc[n] = 0.0f;
  for (int t = wave; t < n_qt; t += SW) {
    // A operand: lane -> query 16 t + r16, dims 32 st + 8 g4 .. +7
    const int pa = 16 * t + r16;
    const bool aok = pa < P;
    const u32x4* qp = reinterpret_cast<const u32x4*>(
        a.q_rot + ((int64_t)(r0 + (aok ? pa : 0) / G) * a.n_q + hk * G + (aok ? pa : 0) % G) * D);
    u32x4 qa[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) qa[st] = aok ? qp[4 * st + g4] : u32x4{0u, 0u, 0u, 0u};
    // this lane's queries 16 t + 4 g4 + i: (M, L) and causal limit
    float mq[4], lq[4];
    int lim[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = 16 * t + 4 * g4 + i;
      const bool ok = p < P;
      mq[i] = ok ? mls[p][0] : 0.0f;
      lq[i] = ok ? mls[p][1] : 1.0f;
      lim[i] = ok ? kv0 + r0 + p / G : -1;  // keys <= this row's position
    }
#pragma unroll
    for (int n = 0; n < SKB / 16; ++n) {
      f32x4_t sa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const u32x4 b = *reinterpret_cast<const u32x4*>(&ks[16 * n + r16][32 * st + 8 * g4]);
        sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qa[st]),
                                                     __builtin_bit_cast(bf16x8_t, b), sa, 0, 0, 0);
      }
      const int j = j0 + 16 * n + r16;
      float c = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (j <= lim[i]) c += expf(sa[i] * scale - mq[i]) / lq[i];
      c += __shfl_xor(c, 16, 64);
      c += __shfl_xor(c, 32, 64);
      acc[n] += c;
    }
  }
  if (g4 == 0) {
#pragma unroll
    for (int n = 0; n < SKB / 16; ++n) red[wave][16 * n + r16] = acc[n];
  }
  __syncthreads();
  if (tid < SKB) {
    const int j = j0 + tid;
    if (j < n_keys) {
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < SW; ++w) v += red[w][tid];
      score[(int64_t)hk * a.cap + j] = v;
    }
  }
}

}  // namespace

static int seq_count_host(const AttnArgs& a) { return a.seqs > 1 ? a.seqs : 1; }

hipError_t launch_rope_append(const AttnArgs& a, hipStream_t s) {
  const dim3 grid(a.m * seq_count_host(a), a.n_q + a.n_kv), block(64);
  switch (a.qkv_part ? a.qkv_splits : 0) {
#define SS_S(n) \
  case n: SS_LAUNCH(rope_append_kernel<n>, grid, block, 0, s, a); break;
    SS_S(0) SS_S(1) SS_S(2) SS_S(3) SS_S(4) SS_S(5) SS_S(6) SS_S(7) SS_S(8)
#undef SS_S
    default: SS_LAUNCH(rope_append_kernel<-1>, grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_decode_attention(const AttnArgs& a, const int32_t* valid, hipStream_t s) {
  if (a.max_keys <= DQ_MAXKEYS) {
    const int S = a.head_splits;
    if (S < 1 || S > DQ_MAXSPLITS || (S > 1 && (!a.counters || !a.part))) return hipErrorInvalidValue;
    // chunks of 16 keys per wave: what the bound on keys fills; up to 3 all
    // loaded up front, beyond that a ring of 3 refilled after use
    const int per_wave = (a.max_keys + 16 * DQW * S - 1) / (16 * DQW * S);
    const dim3 grid(a.n_q, S), block(DQW * 64);
    const bool sp = a.index != nullptr;
    if (per_wave <= 1) {
      if (sp) SS_LAUNCH((draft_attn_head_kernel<true, 1, false>), grid, block, 0, s, a, valid);
      else SS_LAUNCH((draft_attn_head_kernel<false, 1, false>), grid, block, 0, s, a, valid);
    } else if (per_wave == 2) {
      if (sp) SS_LAUNCH((draft_attn_head_kernel<true, 2, false>), grid, block, 0, s, a, valid);
      else SS_LAUNCH((draft_attn_head_kernel<false, 2, false>), grid, block, 0, s, a, valid);
    } else if (per_wave == 3) {
      if (sp) SS_LAUNCH((draft_attn_head_kernel<true, 3, false>), grid, block, 0, s, a, valid);
      else SS_LAUNCH((draft_attn_head_kernel<false, 3, false>), grid, block, 0, s, a, valid);
    } else {
      if (sp) SS_LAUNCH((draft_attn_head_kernel<true, 3, true>), grid, block, 0, s, a, valid);
      else SS_LAUNCH((draft_attn_head_kernel<false, 3, true>), grid, block, 0, s, a, valid);
    }
    return hipGetLastError();
  }
  const dim3 grid(a.n_kv, a.splits), block(256);
  switch (a.n_q / a.n_kv) {
#define SS_G(g) \
  case g: SS_LAUNCH(draft_attn_kernel<g>, grid, block, 0, s, a, valid); break;
    SS_G(1) SS_G(2) SS_G(3) SS_G(4) SS_G(5) SS_G(6) SS_G(7) SS_G(8)
#undef SS_G
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SS_LAUNCH(draft_merge_kernel, dim3(a.n_q), dim3(MP * D), 0, s, a, valid);
  return hipGetLastError();
}

hipError_t launch_rows_attention(const AttnArgs& a, hipStream_t s) {
  if (a.split_keys > DKPB) {
    if (a.split_keys % DKPB != 0 || a.m * (a.n_q / a.n_kv) > 16 * RW) return hipErrorInvalidValue;
    SS_LAUNCH(rows_attn_long_kernel, dim3(a.n_kv, a.splits, seq_count_host(a)), dim3(RW * 64), 0, s, a);
  } else {
    SS_LAUNCH(rows_attn_kernel, dim3(a.n_kv, a.splits, seq_count_host(a)), dim3(RW * 64), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // few splits: one thread per dim walks them in order; many (long
  // contexts): MP split groups per block cut the serial memory round trips
  if (a.splits <= kSeqMergeSplits)
    SS_LAUNCH(rows_merge_seq_kernel, dim3(a.n_q, a.m * seq_count_host(a)), dim3(D), 0, s, a);
  else
    SS_LAUNCH(rows_merge_kernel, dim3(a.n_q, a.m * seq_count_host(a)), dim3(MP * D), 0, s, a);
  return hipGetLastError();
}

int decode_attn_keys_per_split() { return DKPB; }

// One 128-key tile per block while the grid has under ~256 blocks; past that
// (long contexts) a block walks enough tiles, up to 16, to bring the grid to
// about one block per compute unit (the kernel's LDS allows one), if its
// query tiles fit one per wave.  At 60K keys and 8 KV heads: 15 tiles, 99 us
// a layer against 107 for 8 and 118 for 4.
int verify_attn_split_keys(int cap, int n_kv, int rows_x_group) {
  const int tiles = (cap + DKPB - 1) / DKPB;
  int t = (tiles * n_kv + 255) / 256;
  if (t > 16) t = 16;
  if (t < 2 || rows_x_group > 16 * RW) return DKPB;
  return DKPB * t;
}
int draft_attn_keys_per_split() { return DSK; }

// Key splits per query head: one per 96 keys of the launch's bound, at most 8
// (at the 7B shape with ~900 keys, 8 splits measured 6.8 us a layer against
// 7.5 for 4 and 8.6 for 1; over a ~6000-key sparse index, 8 splits 21.4 us
// against 26.9 for 16).  The caller also keeps the grid (query heads x
// splits) within one block per compute unit.
int draft_head_ring(const AttnArgs& a) {
  const int S = a.head_splits;
  if (a.max_keys > DQ_MAXKEYS || S < 1 || S > DQ_MAXSPLITS || (S > 1 && (!a.counters || !a.part))) return 0;
  const int per_wave = (a.max_keys + 16 * DQW * S - 1) / (16 * DQW * S);
  return per_wave <= 1 ? 1 : (per_wave == 2 ? 2 : 3);
}

int draft_head_splits(int max_keys) {
  const int s = (max_keys + 95) / 96;
  return s < 1 ? 1 : (s > 8 ? 8 : s);
}

int attn_scores_max_pairs() { return SMAXP; }

hipError_t launch_attn_scores(const AttnArgs& a, float* score, int window, hipStream_t s) {
  const int G = a.n_q / a.n_kv;
  const int P = (window < a.m ? window : a.m) * G;
  if (P > SMAXP || P < 1 || !a.ml) return hipErrorInvalidValue;
  SS_LAUNCH(attn_scores_kernel, dim3(a.n_kv, (a.cap + SKB - 1) / SKB), dim3(SW * 64), 0, s, a, score, window);
  return hipGetLastError();
}
