// Small kernels of the path: row RMSNorm and embedding gather for the verify
// pass, workspace fill, and the device-side KV bookkeeping of a cycle
// ("How speculative decoding makes LLMs go brrr", Module 2: after a round the
// K/V of rejected positions are dropped - here by moving kv_len only).
#include "common.h"
#include "internal.h"
#include "profile.h"

namespace {

// Row RMSNorm, optionally after adding fp32 partial sums to the row first:
// h = bf16(h + sum_s part[s]) (split order, written back), then
// out = bf16(h / sqrt(mean(h^2) + eps) * g).  One block of 1024 threads per
// row, one 8-value item per thread (k <= 8192): every load (h, the S split
// partials, the norm weights) is issued before the first is used.  S < 0: any
// number of splits (a loop).
template <int S>
__global__ __launch_bounds__(1024) void rmsnorm_rows_kernel(uint16_t* __restrict__ h,
                                                            const float* __restrict__ part, int splits,
                                                            int rows, const uint16_t* __restrict__ g,
                                                            float eps, int k, uint16_t* __restrict__ out) {
  __shared__ float red[16];
  const int row = blockIdx.x, tid = threadIdx.x;
  uint16_t* x = h + (int64_t)row * k;
  const int items = k / 8;
  const bool act = tid < items;
  const int q = act ? tid : 0;
  u32x4 v = reinterpret_cast<const u32x4*>(x)[q];
  const u32x4 gv = reinterpret_cast<const u32x4*>(g)[q];
  float add[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add_split = [&](int sp) {
    const f32x4_t* p = reinterpret_cast<const f32x4_t*>(part + ((int64_t)sp * rows + row) * k + 8 * q);
    const f32x4_t a0 = p[0], a1 = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      add[i] += a0[i];
      add[4 + i] += a1[i];
    }
  };
  if (S > 0) {
    f32x4_t pa[S > 0 ? S : 1][2];
#pragma unroll
    for (int sp = 0; sp < S; ++sp) {
      const f32x4_t* p = reinterpret_cast<const f32x4_t*>(part + ((int64_t)sp * rows + row) * k + 8 * q);
      pa[sp][0] = p[0];
      pa[sp][1] = p[1];
    }
#pragma unroll
    for (int sp = 0; sp < S; ++sp)  // split order
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        add[i] += pa[sp][0][i];
        add[4 + i] += pa[sp][1][i];
      }
  } else if (S < 0) {
    for (int sp = 0; sp < splits; ++sp) add_split(sp);
  }
  if (S != 0) {
    uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      wv[i] = ss::pack_bf(ss::f2bf(ss::lo_bf(wv[i]) + add[2 * i]), ss::f2bf(ss::hi_bf(wv[i]) + add[2 * i + 1]));
    v = u32x4{wv[0], wv[1], wv[2], wv[3]};
    if (act) reinterpret_cast<u32x4*>(x)[q] = v;
  }
  float ss = 0.0f;
  {
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = ss::lo_bf(wv[i]), hi = ss::hi_bf(wv[i]);
      ss += lo * lo;
      ss += hi * hi;
    }
  }
  ss = act ? ss : 0.0f;
  ss = ss::wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int w = 0; w < 16; ++w) tot += red[w];
  const float inv = 1.0f / sqrtf(tot / (float)k + eps);
  if (!act) return;
  uint16_t* o = out + (int64_t)row * k;
  const uint32_t wv[4] = {v.x, v.y, v.z, v.w}, gw[4] = {gv.x, gv.y, gv.z, gv.w};
  uint32_t ow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint16_t lo = ss::f2bf(ss::lo_bf(wv[i]) * inv * ss::lo_bf(gw[i]));
    const uint16_t hi = ss::f2bf(ss::hi_bf(wv[i]) * inv * ss::hi_bf(gw[i]));
    ow[i] = ss::pack_bf(lo, hi);
  }
  reinterpret_cast<u32x4*>(o)[q] = u32x4{ow[0], ow[1], ow[2], ow[3]};
}

// Out-of-range token ids are clamped into [0, vocab) so a bad id cannot read
// outside the table.  Row r takes tokens[r * stride], or with rows_per_seq
// > 0 tokens[(r / rows_per_seq) * seq_stride + (r % rows_per_seq) * stride].
__global__ __launch_bounds__(256) void embed_rows_kernel(const uint16_t* __restrict__ embed,
                                                         const int32_t* __restrict__ tokens, int stride, int k,
                                                         int vocab, uint16_t* __restrict__ h, int rows_per_seq,
                                                         int64_t seq_stride) {
  const int row = blockIdx.x;
  const int z = rows_per_seq > 0 ? row / rows_per_seq : 0;
  const int j = row - z * rows_per_seq;
  const int tok = min(max(tokens[(int64_t)z * seq_stride + (int64_t)j * stride], 0), vocab - 1);
  const u32x4* src = reinterpret_cast<const u32x4*>(embed + (int64_t)tok * k);
  u32x4* dst = reinterpret_cast<u32x4*>(h + (int64_t)row * k);
  for (int q = threadIdx.x; q < k / 8; q += 256) dst[q] = src[q];
}

// act[r][j] = bf16(silu(g) * u) of the bf16 gate/up outputs g = gu[r][j],
// u = gu[r][F + j] (the 4-bit rows of a tree level; the bf16 GEMM does this
// in its epilogue with the same arithmetic).
__global__ __launch_bounds__(256) void silu_rows_kernel(const uint16_t* __restrict__ gu, int64_t F,
                                                        uint16_t* __restrict__ act) {
  const int row = blockIdx.y;
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= F) return;
  const float g = ss::bf2f(gu[(int64_t)row * 2 * F + j]), u = ss::bf2f(gu[(int64_t)row * 2 * F + F + j]);
  act[(int64_t)row * F + j] = ss::f2bf(g / (1.0f + expf(-g)) * u);
}

// Static tree commit: the accepted chain c's first n nodes (slots
// kv_len + 1 + c D + i - 1, i = 1..n) move to slots kv_len + i, in every
// layer and KV head: grid (layer x KV head), 256 threads, 16 bytes each.
// kv_len itself moves afterwards (kv_rollback), once every block has read it.
__global__ __launch_bounds__(256) void tree_commit_kernel(uint16_t* k_cache, uint16_t* v_cache, int cap, int d,
                                                          const int32_t* kv_len, const int32_t* n_accepted,
                                                          const int32_t* chain, int D) {
  const int n = *n_accepted, c = *chain, kvl = *kv_len;
  if (c <= 0 || n <= 0 || n > D) return;  // chain 0 is already in place
  const int64_t base = (int64_t)blockIdx.x * cap * d;
  const int pieces = d / 8;  // 16-byte pieces per row
  for (int e = threadIdx.x; e < n * pieces; e += 256) {
    const int i = 1 + e / pieces, q = e % pieces;
    const int src = kvl + 1 + c * D + i - 1, dst = kvl + i;
    if (src < 0 || src >= cap || dst < 0 || dst >= cap) continue;
    reinterpret_cast<u32x4*>(k_cache + base + (int64_t)dst * d)[q] =
        reinterpret_cast<const u32x4*>(k_cache + base + (int64_t)src * d)[q];
    reinterpret_cast<u32x4*>(v_cache + base + (int64_t)dst * d)[q] =
        reinterpret_cast<const u32x4*>(v_cache + base + (int64_t)src * d)[q];
  }
}

__global__ __launch_bounds__(256) void zero_kernel(u32x4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}

__global__ void kv_rollback_kernel(int32_t* kv_len, int32_t* tokens, const int32_t* n_accepted,
                                   const int32_t* out_tokens) {
  const int n = *n_accepted;
  *kv_len += n + 1;
  tokens[0] = out_tokens[n];
}

__global__ void kv_advance_kernel(int32_t* kv_len, int32_t delta) { *kv_len += delta; }

// A round's last token appended after its accepted drafts: dst[n] = out[n].
__global__ void token_append_kernel(int32_t* dst, int max_n, const int32_t* n_accepted, const int32_t* out_tokens) {
  const int n = *n_accepted;
  if (n >= 0 && n <= max_n) dst[n] = out_tokens[n];
}

// Batched decoding: sequence b moves by n[b] + 1 and takes its last emitted
// token (tokens [B][ld], out [B][out_ld]); with n NULL every kv_len moves by
// delta.  One thread per sequence.
__global__ void batch_rollback_kernel(int32_t* kv_len, int32_t* tokens, int64_t ld, const int32_t* n_accepted,
                                      const int32_t* out_tokens, int64_t out_ld, int batch, int delta) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  if (!n_accepted) {
    kv_len[b] += delta;
    return;
  }
  const int n = n_accepted[b];
  kv_len[b] += n + 1;
  tokens[(int64_t)b * ld] = out_tokens[(int64_t)b * out_ld + n];
}

// valid = (0 <= kv_len + step < cap) and the input token is a vocabulary id;
// when not, the draft step does nothing but set its output token to -1.
// RoPE angles of position p, pair i < d/2: p * theta^(-2i/d) in float64,
// cos and sin stored as float32 (cs[2i], cs[2i+1]).
__device__ __forceinline__ void rope_angle(int p, int i, int d, float theta, float* cs) {
  const double inv_freq = exp(-(2.0 * i / d) * log((double)theta));
  double sd, cd;
  sincos((double)p * inv_freq, &sd, &cd);
  cs[2 * i] = (float)cd;
  cs[2 * i + 1] = (float)sd;
}

// One draft step's position check, and the RoPE table of its position that
// every layer's attention uses: d/2 threads.
__global__ void pos_guard_kernel(const int32_t* kv_len, const int32_t* token_in, int step, int cap,
                                 int vocab, int32_t* valid, int32_t* token_out, int d, float theta,
                                 float* rope_cs, const int32_t* draft_len) {
  const int pos = *kv_len + step;
  if (threadIdx.x < d / 2) rope_angle(pos, threadIdx.x, d, theta, rope_cs);
  if (threadIdx.x == 0) {
    const int t = *token_in;
    const int ok = pos >= 0 && pos < cap && t >= 0 && t < vocab && (!draft_len || step < *draft_len);
    *valid = ok;
    if (!ok) *token_out = -1;
  }
}

// RoPE table of rows j < m: row j is node t = pos_offset + j * stride, at
// position kv_len + t, or kv_len + its depth in a tree of chains of depth
// tree_d: grid m.
__global__ void rope_table_kernel(const int32_t* kv_len, int pos_offset, int stride, int tree_d, int d, float theta,
                                  float* rope_cs, int rows_per_seq) {
  const int j = blockIdx.x;
  const int z = rows_per_seq > 0 ? j / rows_per_seq : 0;  // the row's sequence
  const int t = pos_offset + (j - z * rows_per_seq) * stride;
  const int dep = tree_d > 0 ? (t == 0 ? 0 : (t - 1) % tree_d + 1) : t;
  if (threadIdx.x < d / 2) rope_angle(kv_len[z] + dep, threadIdx.x, d, theta, rope_cs + (int64_t)j * d);
}

}  // namespace

template <int S>
static void launch_norm(uint16_t* h, const float* part, int splits, const uint16_t* g, float eps, int rows, int k,
                        uint16_t* out, hipStream_t s) {
  SS_LAUNCH(rmsnorm_rows_kernel<S>, dim3(rows), dim3(1024), 0, s, h, part, splits, rows, g, eps, k, out);
}

hipError_t launch_rmsnorm_rows(const uint16_t* h, const uint16_t* g, float eps, int rows, int k,
                               uint16_t* out, hipStream_t s) {
  if (k > 8 * 1024 || k % 8 != 0) return hipErrorInvalidValue;
  launch_norm<0>(const_cast<uint16_t*>(h), nullptr, 0, g, eps, rows, k, out, s);
  return hipGetLastError();
}

hipError_t launch_resid_rmsnorm_rows(uint16_t* h, const float* part, int splits, const uint16_t* g, float eps,
                                     int rows, int k, uint16_t* out, hipStream_t s) {
  if (k > 8 * 1024 || k % 8 != 0) return hipErrorInvalidValue;
  switch (part ? splits : 0) {
    case 0: launch_norm<0>(h, part, splits, g, eps, rows, k, out, s); break;
    case 1: launch_norm<1>(h, part, splits, g, eps, rows, k, out, s); break;
    case 2: launch_norm<2>(h, part, splits, g, eps, rows, k, out, s); break;
    case 3: launch_norm<3>(h, part, splits, g, eps, rows, k, out, s); break;
    case 4: launch_norm<4>(h, part, splits, g, eps, rows, k, out, s); break;
    case 5: launch_norm<5>(h, part, splits, g, eps, rows, k, out, s); break;
    case 6: launch_norm<6>(h, part, splits, g, eps, rows, k, out, s); break;
    case 7: launch_norm<7>(h, part, splits, g, eps, rows, k, out, s); break;
    case 8: launch_norm<8>(h, part, splits, g, eps, rows, k, out, s); break;
    default: launch_norm<-1>(h, part, splits, g, eps, rows, k, out, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_embed_rows(const uint16_t* embed, const int32_t* tokens, int rows, int k,
                             int vocab, uint16_t* h, hipStream_t s, int tok_stride, int rows_per_seq,
                             int64_t seq_stride) {
  SS_LAUNCH(embed_rows_kernel, dim3(rows), dim3(256), 0, s, embed, tokens, tok_stride, k, vocab, h, rows_per_seq,
            seq_stride);
  return hipGetLastError();
}

hipError_t launch_silu_rows(const uint16_t* gu, int64_t F, int rows, uint16_t* act, hipStream_t s) {
  SS_LAUNCH(silu_rows_kernel, dim3((unsigned)((F + 255) / 256), rows), dim3(256), 0, s, gu, F, act);
  return hipGetLastError();
}

hipError_t launch_tree_commit(uint16_t* k_cache, uint16_t* v_cache, int layers_x_kv_heads, int cap, int d,
                              const int32_t* kv_len, const int32_t* n_accepted, const int32_t* chain, int D,
                              hipStream_t s) {
  if (d % 8 != 0) return hipErrorInvalidValue;
  SS_LAUNCH(tree_commit_kernel, dim3(layers_x_kv_heads), dim3(256), 0, s, k_cache, v_cache, cap, d, kv_len,
            n_accepted, chain, D);
  return hipGetLastError();
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  SS_LAUNCH(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (u32x4*)p, n16);
  return hipGetLastError();
}

hipError_t launch_kv_rollback(int32_t* kv_len, int32_t* tokens, const int32_t* n_accepted,
                              const int32_t* out_tokens, hipStream_t s) {
  SS_LAUNCH(kv_rollback_kernel, dim3(1), dim3(1), 0, s, kv_len, tokens, n_accepted,
                     out_tokens);
  return hipGetLastError();
}

hipError_t launch_batch_rollback(int32_t* kv_len, int32_t* tokens, int64_t ld, const int32_t* n_accepted,
                                 const int32_t* out_tokens, int64_t out_ld, int batch, int delta, hipStream_t s) {
  SS_LAUNCH(batch_rollback_kernel, dim3((batch + 63) / 64), dim3(64), 0, s, kv_len, tokens, ld, n_accepted, out_tokens,
            out_ld, batch, delta);
  return hipGetLastError();
}

hipError_t launch_token_append(int32_t* dst, int max_n, const int32_t* n_accepted, const int32_t* out_tokens,
                               hipStream_t s) {
  SS_LAUNCH(token_append_kernel, dim3(1), dim3(1), 0, s, dst, max_n, n_accepted, out_tokens);
  return hipGetLastError();
}

hipError_t launch_kv_advance(int32_t* kv_len, int32_t delta, hipStream_t s) {
  SS_LAUNCH(kv_advance_kernel, dim3(1), dim3(1), 0, s, kv_len, delta);
  return hipGetLastError();
}

hipError_t launch_pos_guard(const int32_t* kv_len, const int32_t* token_in, int step, int cap,
                            int vocab, int32_t* valid, int32_t* token_out, int d, float theta,
                            float* rope_cs, const int32_t* draft_len, hipStream_t s) {
  SS_LAUNCH(pos_guard_kernel, dim3(1), dim3(64), 0, s, kv_len, token_in, step, cap, vocab, valid,
            token_out, d, theta, rope_cs, draft_len);
  return hipGetLastError();
}

hipError_t launch_rope_table(const int32_t* kv_len, int pos_offset, int row_stride, int tree_d, int m, int d,
                             float theta, float* rope_cs, hipStream_t s, int rows_per_seq) {
  SS_LAUNCH(rope_table_kernel, dim3(m), dim3(64), 0, s, kv_len, pos_offset, row_stride < 1 ? 1 : row_stride,
            tree_d, d, theta, rope_cs, rows_per_seq);
  return hipGetLastError();
}
