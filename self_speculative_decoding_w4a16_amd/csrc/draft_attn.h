// Draft-step attention over one query position: the per-query-head block
// body, run by its own launch (attention.hip) or by extra blocks of the QKV
// projection's launch (gemv_w4t.hip) - "How speculative decoding makes LLMs
// go brrr", Module 2; draft and target share one KV cache ("SubSpec:
// Speculate Deep and Accurate" paper note, Method details, KV-cache sharing).
#ifndef SUBSPEC_DRAFT_ATTN_H
#define SUBSPEC_DRAFT_ATTN_H

#include "common.h"
#include "internal.h"

namespace {

constexpr int D = 128;       // head dim handled by the attention kernels
constexpr int DREC = 4 + D;  // partial record: m, l, 2 pad, o[D] (16-byte aligned o)

struct DraftKeys {
  int kv0, pos, n_idx, n_keys;
  const int32_t* ilist;
};

// Key slots of the draft query of kv head hk (dense: slot t = position t).
// Both scalars are read unconditionally (kv_len stands in for the absent
// index length), so the loads need no branch and their latency overlaps
// whatever follows until the first use.
__device__ __forceinline__ DraftKeys draft_keys(const AttnArgs& a, int hk) {
  DraftKeys k;
  const bool sparse = a.index != nullptr;
  k.kv0 = *a.kv_len;
  const int n_raw = *(sparse ? a.n_index : a.kv_len);
  k.pos = k.kv0 + a.pos_offset;
  k.n_idx = sparse ? min(max(n_raw, 0), a.index_cap) : 0;
  k.ilist = sparse ? a.index + (int64_t)hk * a.index_cap : nullptr;
  k.n_keys = sparse ? k.n_idx + a.pos_offset + 1 : k.pos + 1;
  return k;
}

// Draft-step attention with S = a.head_splits blocks per query head (short
// contexts; no merge launch): grid (query head, split), 512 threads = 8
// waves; wave w of split s takes the 16-key chunks 8 s + w + 8 S i, so the
// head's K/V reads are spread over S compute units (one unit alone cannot
// pull them at HBM rate).  Lane (part kp = lane % 8, key kg = lane / 8)
// holds 16 bytes of each half of the K and V rows of keys kg and 8 + kg of
// the chunk, dims 8 kp .. +7 and 64 + 8 kp .. +7, so every load instruction
// reads whole 128-byte rows of 8 keys; a score is the lane's partial dot
// summed over its 8 lanes (three in-register DPP steps).  Every lane keeps a
// running softmax (reference max m, sum l) and an output partial o[16] over
// the keys it sees, rescaled only when a score exceeds m by more than 8 (in
// log2 units; the weights stay below 2^8); lanes and waves are combined once
// at the end.  Loads run DQR (1-3) chunks ahead in a ring named statically,
// the first ones issued before kv_len is known (dense keys); a buffer is
// refilled after use only where a wave has more chunks than the ring holds
// (REFILL: more than 3 a wave), else every chunk is loaded up front and no
// load is issued past the wave's last chunk.  Every
// block of a kv head rotates the new key itself (its score needs it); split 0
// scores it, and split 0 of the group's first head appends the new K/V to the
// cache (no block reads that slot from memory).  With S > 1 each block writes
// its partial (m, l, o[d]) with agent-coherent stores, waits for them to
// complete and counts itself in counters[hq]; the block that sees the count
// reach S reads the S partials with agent-coherent loads, writes the merged
// row and resets the counter, so no cache flush is needed.
//
// In the QKV launch (FUSED): the same blocks run after the QKV GEMV's blocks
// in one grid.  They issue their K/V loads first (they do not depend on the
// projection), then wait for the query head's rows (and, in split 0, the kv
// head's new key and value rows) to be counted complete in ready[] by the
// GEMV blocks, which store those rows with agent-coherent stores and count
// each 16-row tile in once the stores are done; the rows are then read with
// agent-coherent loads.  The GEMV blocks wait for nothing and come first in
// the grid (workgroups start in order), so every wait ends.  A wait is also
// bounded in time: past kReadyWaitTicks it gives up, sets bit 0 of the last
// line of ready[] and goes on (the results are then not defined).  Each count
// has a 128-byte line of its own (ready[kReadyStride g]).
constexpr int DQW = 8;            // waves
constexpr int DQ_MAXKEYS = 8192;  // keys up to which the per-head kernel is used
constexpr int DQ_MAXSPLITS = 16;  // blocks per query head, at most
constexpr uint64_t kReadyWaitTicks = 20000000;  // 0.2 s of the 100 MHz wall clock

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// v summed over the 8 lanes of a half-row (every lane gets the sum)
__device__ __forceinline__ float oct_sum(float v) {
  v += dpp<0xB1>(v);         // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);         // quad_perm [2,3,0,1]
  return v + dpp<0x141>(v);  // row_half_mirror: lane i <-> 7 - i, the other quad
}

// SPARSE: keys from the index (else slot t = cache row t); DQR: chunks in
// flight per wave (1-3, no more than the launch's bound on keys fills).
// Both are compile-time so that every load is issued on every path and each
// wait covers exactly what it needs.
template <bool SPARSE, int DQR, bool REFILL, bool FUSED>
__device__ __forceinline__ void draft_attn_head(const AttnArgs& a, const int32_t* valid, int hq, int split, int S,
                                                uint32_t* ready) {
  static_assert(!(SPARSE && FUSED), "the in-launch form attends over the dense cache only");
  constexpr int KW = 16;
  constexpr int NP = DQW * 4;  // partials: 4 rows of 16 lanes per wave
  __shared__ __align__(16) uint32_t qp[D / 2];    // rotated query, bf16 pairs
  __shared__ __align__(16) uint32_t knew[D / 2];  // rotated new key
  __shared__ __align__(16) uint32_t vnew[D / 2];
  __shared__ float pm[NP], pl[NP], pf[NP];
  __shared__ float po[NP][D];

  const int tid = threadIdx.x;
  const int G = a.n_q / a.n_kv, hk = hq / G;
  const int lane = tid & 63, wave = tid >> 6;
  const int c_first = split * DQW + wave, c_step = DQW * S;  // this wave's chunks
  const uint16_t* kc = a.k_cache + (int64_t)hk * a.cap * D;
  const uint16_t* vc = a.v_cache + (int64_t)hk * a.cap * D;
  const int kp = lane & 7, kg = lane >> 3;
  constexpr bool sparse = SPARSE;
  // position flag and kv_len: read first (scalar loads; kv_len stands in for
  // an absent flag, so no branch), tested after the loads that do not depend
  // on them are issued and the rotation is done
  const int v_raw = *(valid ? valid : a.kv_len);
  const int vflag = valid ? v_raw : 1;
  const DraftKeys ks = draft_keys(a, hk);

  // The new token's q, k and v rows and its RoPE factors are loaded first,
  // by every thread (indices wrapped; used by threads 0-63: query pairs,
  // 64-127: new-key pairs, 32 active lanes each, 128-191: the new value):
  // they do not depend on kv_len, and the rotation then overlaps the K/V
  // loads instead of waiting for them.
  const int half = D / 2, i2 = tid & 63;
  const bool rot = tid < 128 && i2 < half / 2;
  const uint16_t* xrow = (tid < 64) ? a.qkv + (int64_t)hq * D : a.qkv + (int64_t)(a.n_q + hk) * D;
  const uint16_t* vrow = a.qkv + (int64_t)(a.n_q + a.n_kv + hk) * D;
  uint32_t xlo = 0, xhi = 0, vin = 0;  // (in the QKV launch: read after the wait)
  if constexpr (!FUSED) {
    xlo = reinterpret_cast<const uint32_t*>(xrow)[i2 & 31];
    xhi = reinterpret_cast<const uint32_t*>(xrow + half)[i2 & 31];
  }
  const f32x4_t cs = reinterpret_cast<const f32x4_t*>(a.rope_cs)[i2 & 31];
  if constexpr (!FUSED) vin = reinterpret_cast<const uint32_t*>(vrow)[i2];
  // keep these loads ahead of the K/V loads (loads complete in issue order)
  __builtin_amdgcn_sched_barrier(0);

  // chunk loads: [key kg, key 8 + kg] x [half 0, half 1] of the K/V rows at
  // row(t) for slot t
  struct Chunk {
    u32x4 k[4], v[4];
  };
  auto load_rows = [&](int c, Chunk& b, auto row_of) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int64_t row = (int64_t)row_of(c * KW + 8 * e + kg) * D;
      const u32x4* kr = reinterpret_cast<const u32x4*>(kc + row) + kp;
      const u32x4* vr = reinterpret_cast<const u32x4*>(vc + row) + kp;
      b.k[2 * e] = kr[0];
      b.k[2 * e + 1] = kr[8];
      b.v[2 * e] = vr[0];
      b.v[2 * e + 1] = vr[8];
    }
  };
  // Dense: slot t is cache row t, so the first chunks are loaded before
  // kv_len is known (rows clamped to the cache; slots from the new key on
  // are masked, and their V zeroed, when consumed).
  Chunk ring[DQR];
  auto dense_row = [&](int t) { return min(t, a.cap - 1); };
  if (!sparse) {
#pragma unroll
    for (int j = 0; j < DQR; ++j) load_rows(c_first + j * c_step, ring[j], dense_row);
  }

  // ---- in the QKV launch: wait for this head's rows, then read them
  // Lane 0 of wave 0 waits for the query head's 128 rows, lanes 1 and 2 of
  // split 0 for the kv head's new key and value rows (only split 0 uses
  // them).  Each reader counts itself in once past the wait; the last of a
  // group's readers (S for a query head, G split-0 blocks for a kv head)
  // resets the count at its end.
  bool rneed = false;
  int rgrp = 0, rreaders = 1;
  uint32_t rold = 0;
  if constexpr (FUSED) {
    if (vflag == 0) return;  // block-uniform: the QKV blocks skipped the launch too
    rneed = wave == 0 && (lane == 0 || (split == 0 && (lane == 1 || lane == 2)));
    rgrp = lane == 0 ? hq : (lane == 1 ? a.n_q + hk : a.n_q + a.n_kv + hk);
    rreaders = lane == 0 ? S : G;
    if (wave == 0) {
      const uint64_t t0 = wall_clock64();
      bool gave_up = false;
      for (;;) {
        const uint32_t c = rneed ? __hip_atomic_load(ready + kReadyStride * rgrp, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT)
                                 : (uint32_t)D;
        if (__all(c >= (uint32_t)D)) break;
        if (wall_clock64() - t0 > kReadyWaitTicks) {
          gave_up = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (gave_up && lane == 0)
        __hip_atomic_fetch_or(ready + kReadyStride * (kReadyLines - 1), 1u, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
      if (rneed)
        rold = __hip_atomic_fetch_add(ready + kReadyStride * rgrp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    const uint32_t* xw = reinterpret_cast<const uint32_t*>(xrow);
    xlo = __hip_atomic_load(xw + (i2 & 31), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    xhi = __hip_atomic_load(xw + half / 2 + (i2 & 31), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    vin = __hip_atomic_load(reinterpret_cast<const uint32_t*>(vrow) + i2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  auto release = [&]() {
    if (FUSED && rneed && rold == (uint32_t)(D + rreaders - 1))
      __hip_atomic_store(ready + kReadyStride * rgrp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };

  // ---- RoPE of the query (threads 0-63) and the new key (64-127) into LDS;
  // new V (128-191)
  uint32_t klo = 0, khi = 0;
  if (rot) {
    const float a1 = ss::lo_bf(xlo), b1 = ss::hi_bf(xlo);
    const float a2 = ss::lo_bf(xhi), b2 = ss::hi_bf(xhi);
    klo = ss::pack_bf(ss::f2bf(a1 * cs[0] - a2 * cs[1]), ss::f2bf(b1 * cs[2] - b2 * cs[3]));
    khi = ss::pack_bf(ss::f2bf(a2 * cs[0] + a1 * cs[1]), ss::f2bf(b2 * cs[2] + b1 * cs[3]));
    uint32_t* dst = (tid < 64) ? qp : knew;
    dst[i2] = klo;
    dst[half / 2 + i2] = khi;
  } else if (tid >= 128 && tid < 192) {
    vnew[tid - 128] = vin;
  }
  if (vflag == 0 || ks.pos < 0 || ks.pos >= a.cap) {  // block-uniform
    release();
    return;
  }
  // the group's first block appends the new K/V to the cache
  if (hq % G == 0 && split == 0) {
    if (rot && tid >= 64) {
      uint32_t* kdst = reinterpret_cast<uint32_t*>(a.k_cache + ((int64_t)hk * a.cap + ks.pos) * D);
      kdst[i2] = klo;
      kdst[half / 2 + i2] = khi;
    } else if (tid >= 128 && tid < 192) {
      reinterpret_cast<uint32_t*>(a.v_cache + ((int64_t)hk * a.cap + ks.pos) * D)[tid - 128] = vin;
    }
  }
  const int last = ks.n_keys - 1;  // slot of the new key
  const int n_chunks = (ks.n_keys + KW - 1) / KW;
  // sparse slot t -> cache row, split in two so that the index entry can be
  // loaded a round before the K/V row it addresses (slots past the index are
  // the speculative positions)
  auto index_entry = [&](int t) {
    t = t < last ? t : 0;
    return ks.ilist[min(t, max(ks.n_idx - 1, 0))];
  };
  auto sparse_row_of = [&](int t, int entry) {
    t = t < last ? t : 0;
    const int ip = min(max(entry, 0), a.cap - 1);
    return t < ks.n_idx ? ip : ks.kv0 + (t - ks.n_idx);
  };
  auto sparse_row = [&](int t) { return sparse_row_of(t, index_entry(t)); };
  auto load_chunk = [&](int c, Chunk& b) {
    if (sparse)
      load_rows(c, b, sparse_row);
    else
      load_rows(c, b, dense_row);
  };
  // sparse: the index entries of each slot's next chunk, loaded a round
  // ahead (a refill then issues its K/V loads without waiting for them)
  int nidx[DQR][2];
  auto clamp_chunk = [&](int c) { return c < n_chunks ? c : 0; };
  auto load_entries = [&](int c, int (&e2)[2]) {
#pragma unroll
    for (int e = 0; e < 2; ++e) e2[e] = index_entry(c * KW + 8 * e + kg);
  };
  if (sparse) {
#pragma unroll
    for (int j = 0; j < DQR; ++j) {
      const int c = c_first + j * c_step;
      load_chunk(clamp_chunk(c), ring[j]);
    }
    if (REFILL) {
#pragma unroll
      for (int j = 0; j < DQR; ++j) load_entries(clamp_chunk(c_first + (j + DQR) * c_step), nidx[j]);
    }
  }

  __syncthreads();

  // scores in log2 units: exp(s / sqrt(128)) = 2^(s * log2(e) / sqrt(128))
  const float scale = 0.088388347648318440f * 1.4426950408889634f;
  const u32x4 q0 = reinterpret_cast<const u32x4*>(qp)[kp], q1 = reinterpret_cast<const u32x4*>(qp)[8 + kp];
  float m = -INFINITY, l = 0.0f, o[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) o[j] = 0.0f;

  auto score = [&](const u32x4& k0, const u32x4& k1) {
    float d0 = ss::dot2(k0.x, q0.x, 0.0f), d1 = ss::dot2(k0.y, q0.y, 0.0f);
    d0 = ss::dot2(k0.z, q0.z, d0);
    d1 = ss::dot2(k0.w, q0.w, d1);
    d0 = ss::dot2(k1.x, q1.x, d0);
    d1 = ss::dot2(k1.y, q1.y, d1);
    d0 = ss::dot2(k1.z, q1.z, d0);
    d1 = ss::dot2(k1.w, q1.w, d1);
    return oct_sum(d0 + d1) * scale;
  };
  // keys with scores sa, sb (inactive: -inf) and V halves (va0, va1), (vb0, vb1)
  auto update = [&](float sa, float sb, const u32x4& va0, const u32x4& va1, const u32x4& vb0,
                    const u32x4& vb1) {
    const float mx = fmaxf(sa, sb);
    if (mx > m + 8.0f) {  // raise the reference (first key: m = -inf)
      const float r = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - mx);
      l *= r;
#pragma unroll
      for (int j = 0; j < 16; ++j) o[j] *= r;
      m = mx;
    }
    const float pa = (sa == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(sa - m);
    const float pb = (sb == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(sb - m);
    l += pa + pb;
    const uint32_t wa[8] = {va0.x, va0.y, va0.z, va0.w, va1.x, va1.y, va1.z, va1.w};
    const uint32_t wb[8] = {vb0.x, vb0.y, vb0.z, vb0.w, vb1.x, vb1.y, vb1.z, vb1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      o[2 * e] += pa * ss::lo_bf(wa[e]) + pb * ss::lo_bf(wb[e]);
      o[2 * e + 1] += pa * ss::hi_bf(wa[e]) + pb * ss::hi_bf(wb[e]);
    }
  };
  // consume chunk c from its buffer (the new key is taken after the loop); in
  // the chunk holding the new key, the V rows of its slots and beyond may be
  // stale (zero weight, but not necessarily finite): they are zeroed
  auto step = [&](int c, const Chunk& b) {
    const int t = c * KW + kg;
    const float sa = score(b.k[0], b.k[1]), sb = score(b.k[2], b.k[3]);
    if (c == last / KW) {  // wave-uniform
      const u32x4 z = {0u, 0u, 0u, 0u};
      update(t < last ? sa : -INFINITY, t + 8 < last ? sb : -INFINITY, t < last ? b.v[0] : z,
             t < last ? b.v[1] : z, t + 8 < last ? b.v[2] : z, t + 8 < last ? b.v[3] : z);
    } else {
      update(sa, sb, b.v[0], b.v[1], b.v[2], b.v[3]);
    }
  };
  if constexpr (REFILL) {
    // each buffer is refilled with chunk c + DQR * DQW right after use; the last
    // pass may run past the wave's chunks: those are skipped, their loads (of
    // chunk 0) still issued, so the loads in flight are the same on every path
    for (int c = c_first; c < n_chunks; c += DQR * c_step) {
#pragma unroll
      for (int j = 0; j < DQR; ++j) {
        const int cj = c + j * c_step, cn = cj + DQR * c_step;
        if (j == 0 || cj < n_chunks) step(cj, ring[j]);
        if (sparse) {
          const int cc = clamp_chunk(cn);
          const int e0 = nidx[j][0], e1 = nidx[j][1];
          load_rows(cc, ring[j], [&](int t) { return sparse_row_of(t, (t - cc * KW) < 8 ? e0 : e1); });
          load_entries(clamp_chunk(cn + DQR * c_step), nidx[j]);
        } else {
          load_chunk(clamp_chunk(cn), ring[j]);
        }
      }
    }
  } else {
    // the launch's bound on keys gives every wave at most DQR chunks, all of
    // them in the ring already: one pass and no refill loads
#pragma unroll
    for (int j = 0; j < DQR; ++j) {
      const int cj = c_first + j * c_step;
      if (cj < n_chunks) step(cj, ring[j]);
    }
  }
  // the new key, from LDS: the 8 lanes of key group 0 in wave 0 of split 0
  if (split == 0 && wave == 0 && kg == 0) {
    const u32x4* kn = reinterpret_cast<const u32x4*>(knew);
    const u32x4* vn = reinterpret_cast<const u32x4*>(vnew);
    const u32x4 z = {0u, 0u, 0u, 0u};
    update(score(kn[kp], kn[8 + kp]), -INFINITY, vn[kp], vn[8 + kp], z, z);
  }

  // ---- the lanes 8 apart in a row (same dims) combine: max, rescale, sum
  const float mr = fmaxf(m, dpp<0x128>(m));  // row_ror:8
  const float f = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - mr);
  l *= f;
  l += dpp<0x128>(l);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float v = o[j] * f;
    o[j] = v + dpp<0x128>(v);
  }
  // lanes 0-7 of each row hold the row's partial for their dims
  const int pidx = wave * 4 + (lane >> 4);
  if ((lane & 15) < 8) {
    if (kp == 0) {
      pm[pidx] = mr;
      pl[pidx] = l;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      po[pidx][8 * kp + j] = o[j];
      po[pidx][64 + 8 * kp + j] = o[8 + j];
    }
  }
  __syncthreads();
  // ---- combine the partials (rows that saw no key have m = -inf)
  if (tid < NP) {
    float M = -INFINITY;
#pragma unroll
    for (int q = 0; q < NP; ++q) M = fmaxf(M, pm[q]);
    pf[tid] = (pm[tid] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(pm[tid] - M);
  }
  __syncthreads();
  float L = 0.0f, O = 0.0f;
  if (tid < D) {
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      L += pf[q] * pl[q];
      O += pf[q] * po[q][tid];
    }
  }
  if (S == 1) {
    if (tid < D) a.out[(int64_t)hq * D + tid] = ss::f2bf(O / L);
    release();
    return;
  }
  // ---- S > 1: partial out, count in, the last block of the head merges
  __shared__ int is_last;
  float* rec = a.part + (int64_t)hq * S * DREC;
  if (tid < D) {
    float* dst = rec + (int64_t)split * DREC;
    __hip_atomic_store(dst + 4 + tid, O, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == 0) {
      float M = -INFINITY;
#pragma unroll
      for (int q = 0; q < NP; ++q) M = fmaxf(M, pm[q]);
      __hip_atomic_store(dst, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(dst + 1, L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // the partial's stores complete (reach the agent coherence point) before
  // the block counts itself
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0)
    is_last = __hip_atomic_fetch_add(a.counters + hq, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(S - 1);
  __syncthreads();
  if (!is_last) {
    release();
    return;
  }
  if (tid < D) {
    // the S (<= DQ_MAXSPLITS) partials, 8 loads in flight (indices clamped),
    // merged in split order
    float Ms = -INFINITY, Ls = 0.0f, Os = 0.0f;
    for (int t0 = 0; t0 < S; t0 += 8) {
    float mv[8], lv[8], ov[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float* q = rec + (int64_t)min(t0 + t, S - 1) * DREC;
      mv[t] = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      lv[t] = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ov[t] = __hip_atomic_load(q + 4 + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float mt = mv[t], lt = lv[t], ot = ov[t];
      if (t0 + t >= S || mt == -INFINITY) continue;
      const float Mn = fmaxf(Ms, mt);
      const float fo = (Ms == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(Ms - Mn);
      const float fn = __builtin_amdgcn_exp2f(mt - Mn);
      Ls = Ls * fo + lt * fn;
      Os = Os * fo + ot * fn;
      Ms = Mn;
    }
    }
    a.out[(int64_t)hq * D + tid] = ss::f2bf(Os / Ls);
  }
  if (tid == 0) __hip_atomic_store(a.counters + hq, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  release();
}

}  // namespace

#endif  // SUBSPEC_DRAFT_ATTN_H
