// The static deep/narrow token tree: drafting its levels and judging its root.
//
// SubSpec keeps SpecInfer's token-tree verification with a static tree that is
// deep and narrow, k = 6 chains of depth D = 48 ("SubSpec" report, sections
// 6.3, 6.4 and 3.7).  Here the tree is k chains sharing the root (the last
// committed token); chain c's node at depth d is node t = 1 + c D + d - 1.
//
//  rows_sample   the tokens of the next level from a level's draft logits:
//                the root's k children (its k largest logits when T_d = 0,
//                else k draws from its distribution) or each chain's next
//                token (argmax or one draw); also each sequence's token of
//                a batched draft step.
//  tree_root     SpecInfer's multi-step speculative sampling at the root:
//                child c is accepted when r_c < p_c(x_c) / q(x_c), with
//                p_{c+1} = norm(max(0, p_c - q)) after a rejection (q one-hot
//                at x_c for greedy children); no child accepted -> one draw
//                from the last p_c.  The accepted chain's own round (the
//                plain rejection round over its depth-1..D rows) already ran
//                for every chain, batched; this kernel picks the accepted
//                chain's result and composes the emitted tokens.
//
// Arithmetic: the integer weights of the plain round (floor(w 2^40) of
// exp((z - M) / T) in float32), 128-bit accept tests, residuals kept below
// 2^41 (the first shifted by bitlength(S_d) - 1, later ones by one bit more),
// inverse CDF in ascending token order.  One block of 1024 threads per row.
// Every pass over the vocabulary is coalesced: the row is cut into chunks of
// 8192 tokens and thread t takes the 8 tokens 8 t .. 8 t + 7 of each chunk,
// so a wave reads 1 KiB of consecutive logits; a draw keeps the per-wave
// weight sums of every chunk (a chunk, then a wave in it, then a lane's 8
// tokens locate the threshold in ascending token order).
#include "common.h"
#include "internal.h"
#include "profile.h"

namespace {

constexpr int kTB = 1024;
constexpr int kTW = kTB / 64;
constexpr int kPiece = 8;                 // tokens per thread and chunk
constexpr int kChunk = kTB * kPiece;      // 8192 tokens
constexpr int kMaxChunks = 64;            // vocabularies up to 524288 tokens

__device__ __forceinline__ unsigned long long wt(float z, float M, float T) { return ss::fixed_weight(z, M, T); }

__device__ ss::ArgMax block_argmax_1k(ss::ArgMax a, float* rv, int* ri) {
  a = ss::wave_argmax(a);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) {
    rv[w] = a.v;
    ri[w] = a.i;
  }
  __syncthreads();
  ss::ArgMax b = {rv[0], ri[0]};
  for (int i = 1; i < kTW; ++i) b = ss::better(b, ss::ArgMax{rv[i], ri[i]});
  return b;
}

__device__ unsigned long long block_sum_1k(unsigned long long v, unsigned long long* red) {
  v = ss::wave_sum_u64(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  unsigned long long t = 0;
  for (int i = 0; i < kTW; ++i) t += red[i];
  return t;
}

// first token of this thread's piece of chunk c
__device__ __forceinline__ int piece0(int c) { return c * kChunk + kPiece * (int)threadIdx.x; }

// Per-wave weight sums of every chunk (wsum[c][wave]) and the row's total.
template <typename W>
__device__ unsigned long long chunk_sums(int V, W weight, unsigned long long* wsum, unsigned long long* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nch = (V + kChunk - 1) / kChunk;
  unsigned long long tot = 0;
  for (int c = 0; c < nch; ++c) {
    const int j0 = piece0(c);
    unsigned long long s = 0;
#pragma unroll
    for (int e = 0; e < kPiece; ++e)
      if (j0 + e < V) s += weight(j0 + e);
    s = ss::wave_sum_u64(s);
    if (lane == 0) wsum[c * kTW + w] = s;
    tot += s;
  }
  return block_sum_1k(lane == 0 ? tot : 0ull, red);
}

// Smallest token whose inclusive prefix weight exceeds th (0 <= th < total),
// from the per-wave chunk sums: thread 0 finds the chunk and the wave, that
// wave scans its lanes' piece sums, the lane holding th walks its 8 tokens.
template <typename W>
__device__ int draw_token(unsigned long long th, int V, W weight, const unsigned long long* wsum, int* s_cw,
                          unsigned long long* s_base, int* s_tok) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nch = (V + kChunk - 1) / kChunk;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long base = 0;
    int cw = nch * kTW - 1;
    for (int i = 0; i < nch * kTW; ++i) {
      if (base + wsum[i] > th) {
        cw = i;
        break;
      }
      base += wsum[i];
    }
    *s_cw = cw;
    *s_base = base;
    *s_tok = V - 1;
  }
  __syncthreads();
  const int cw = *s_cw;
  if (w == cw % kTW) {
    const int j0 = (cw / kTW) * kChunk + kPiece * (int)threadIdx.x;
    unsigned long long mine = 0;
#pragma unroll
    for (int e = 0; e < kPiece; ++e)
      if (j0 + e < V) mine += weight(j0 + e);
    unsigned long long incl = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const unsigned long long t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    const unsigned long long base = *s_base + incl - mine;
    if (mine > 0 && base <= th && th - base < mine) {
      unsigned long long c = base;
      for (int e = 0; e < kPiece && j0 + e < V; ++e) {
        c += weight(j0 + e);
        if (c > th) {
          *s_tok = j0 + e;
          break;
        }
      }
    }
  }
  __syncthreads();
  const int t = *s_tok;
  __syncthreads();  // read by every thread before the shared slots are set again
  return t;
}

// Argmax (and, with prev, the best token after prev in (larger value,
// lower index) order) over a row, coalesced.
__device__ ss::ArgMax row_argmax(const uint16_t* z, int V, const ss::ArgMax* prev, float* rv, int* ri) {
  ss::ArgMax a = {-INFINITY, ss::kNoIndex};
  const int nch = (V + kChunk - 1) / kChunk;
  for (int c = 0; c < nch; ++c) {
    const int j0 = piece0(c);
#pragma unroll
    for (int e = 0; e < kPiece; ++e) {
      const int j = j0 + e;
      if (j >= V) break;
      const ss::ArgMax cj = ss::cand(ss::bf2f(z[j]), j);
      if (prev && !(cj.i != ss::kNoIndex && (cj.v < prev->v || (cj.v == prev->v && cj.i > prev->i)))) continue;
      a = ss::better(a, cj);
    }
  }
  return block_argmax_1k(a, rv, ri);
}

__global__ __launch_bounds__(kTB) void rows_sample_kernel(RowsSampleArgs a) {
  __shared__ float rv[kTW];
  __shared__ int ri[kTW];
  __shared__ unsigned long long red[kTW];
  __shared__ unsigned long long wsum[kMaxChunks * kTW];
  __shared__ int s_cw, s_tok;
  __shared__ unsigned long long s_base;
  const int r = blockIdx.x, tid = threadIdx.x, V = a.V;
  const uint16_t* z = a.logits + (int64_t)r * a.ld;
  const bool fits = a.kv_len[(int64_t)r * a.kv_row] + a.need <= a.cap;
  auto out_slot = [&](int i) { return a.tokens + (int64_t)r * a.t_row + (int64_t)i * a.t_out; };
  if (!fits) {  // past the cache: no candidate (the round skips it)
    if (tid < a.nout) *out_slot(tid) = -1;
    return;
  }
  const ss::ArgMax am = row_argmax(z, V, nullptr, rv, ri);
  if (a.T == 0.0f) {
    if (tid == 0) *out_slot(0) = ss::argmax_token(am);
    ss::ArgMax prev = am;
    for (int c = 1; c < a.nout; ++c) {  // next in (larger value, lower index) order
      ss::ArgMax b = {-INFINITY, ss::kNoIndex};
      if (prev.i != ss::kNoIndex) b = row_argmax(z, V, &prev, rv, ri);
      if (tid == 0) *out_slot(c) = ss::argmax_token(b);
      prev = b;
    }
    return;
  }
  const float M = am.v, T = a.T;
  auto weight = [&](int j) { return wt(ss::bf2f(z[j]), M, T); };
  const unsigned long long S = chunk_sums(V, weight, wsum, red);
  for (int i = 0; i < a.nout; ++i) {
    const uint32_t uc = a.u[(int64_t)r * a.u_row + (int64_t)i * a.u_out];
    int tok = 0;
    if (S > 0) {
      const unsigned long long th = ss::shr128(ss::mul64((unsigned long long)uc, S), 24);
      tok = draw_token(th, V, weight, wsum, &s_cw, &s_base, &s_tok);
    }
    if (tid == 0) *out_slot(i) = tok;
  }
}

__global__ __launch_bounds__(kTB) void tree_root_kernel(const uint16_t* __restrict__ zt, const uint16_t* __restrict__ zd,
                                                        int V, float T, float Td, const int32_t* __restrict__ tokens,
                                                        int k, int D, const uint32_t* __restrict__ r_codes,
                                                        const uint32_t* __restrict__ u_code,
                                                        const int32_t* __restrict__ chain_n,
                                                        const int32_t* __restrict__ chain_out,
                                                        const int32_t* __restrict__ chain_status,
                                                        unsigned long long* resid, int32_t* n_accepted,
                                                        int32_t* chain, int32_t* out_tokens, int32_t* status_out) {
  __shared__ float rv[kTW];
  __shared__ int ri[kTW];
  __shared__ unsigned long long red[kTW];
  __shared__ unsigned long long wsum[kMaxChunks * kTW];
  __shared__ int s_cw, s_tok;
  __shared__ unsigned long long s_base;
  const int tid = threadIdx.x;
  const int nch = (V + kChunk - 1) / kChunk;
  // the root's target and draft rows: max / argmax and non-finite flags
  ss::ArgMax at = {-INFINITY, ss::kNoIndex}, ad = {-INFINITY, ss::kNoIndex};
  int bad = 0;
  for (int c = 0; c < nch; ++c) {
    const int j0 = piece0(c);
#pragma unroll
    for (int e = 0; e < kPiece; ++e) {
      const int j = j0 + e;
      if (j >= V) break;
      const float a = ss::bf2f(zt[j]), b = ss::bf2f(zd[j]);
      bad |= !ss::finite(a) || !ss::finite(b);
      at = ss::better(at, ss::cand(a, j));
      ad = ss::better(ad, ss::cand(b, j));
    }
  }
  at = block_argmax_1k(at, rv, ri);
  ad = block_argmax_1k(ad, rv, ri);
  int status = __syncthreads_or(bad) ? 1 : 0;
  int chosen = -1, y = 0;
  if (T == 0.0f) {  // greedy: the first child equal to the target's argmax
    y = ss::argmax_token(at);
    for (int c = 0; c < k; ++c) {
      const int x = tokens[1 + c * D];
      if (x < 0 || x >= V) {
        status |= 4;
        continue;
      }
      if (x == y) {
        chosen = c;
        break;
      }
    }
  } else {
    const float Mt = at.v, Md = ad.v;
    auto wp = [&](int j) { return wt(ss::bf2f(zt[j]), Mt, T); };
    auto wq = [&](int j) { return wt(ss::bf2f(zd[j]), Md, Td); };
    unsigned long long mine = 0, md = 0;
    for (int c = 0; c < nch; ++c) {
      const int j0 = piece0(c);
#pragma unroll
      for (int e = 0; e < kPiece; ++e) {
        const int j = j0 + e;
        if (j >= V) break;
        mine += wp(j);
        if (Td != 0.0f) md += wq(j);
      }
    }
    const unsigned long long St = block_sum_1k(mine, red);
    const unsigned long long Sd = Td != 0.0f ? block_sum_1k(md, red) : 1ull;
    bool from_p = true;  // the current weights are p's own (else the residual array)
    unsigned long long S = St;
    for (int c = 0; c < k; ++c) {
      const int x = tokens[1 + c * D];
      if (x < 0 || x >= V) {  // not a vocabulary id: skipped
        status |= 4;
        continue;
      }
      const unsigned long long Wdx = Td == 0.0f ? 1ull : wq(x);
      if (Wdx == 0ull) status |= 4;
      const unsigned long long Wx = from_p ? wp(x) : resid[x];
      const ss::U128 lhs = ss::mul64((unsigned long long)r_codes[c] * Wdx, S);
      const ss::U128 rhs = ss::shl128(ss::mul64(Wx, Sd), 24);
      if (ss::lt128(lhs, rhs)) {
        chosen = c;
        break;
      }
      // rejected: the next p is norm(max(0, p - q)), kept below 2^41
      const int shift = ss::bitlen_minus1(Sd) + (from_p ? 0 : 1);
      unsigned long long loc = 0;
      for (int cc = 0; cc < nch; ++cc) {
        const int j0 = piece0(cc);
#pragma unroll
        for (int e = 0; e < kPiece; ++e) {
          const int j = j0 + e;
          if (j >= V) break;
          const unsigned long long Wj = from_p ? wp(j) : resid[j];
          const unsigned long long Wdj = Td == 0.0f ? (j == x ? 1ull : 0ull) : wq(j);
          const unsigned long long w = ss::resid_w(Wj, Sd, Wdj, S, shift);
          resid[j] = w;
          loc += w;
        }
      }
      const unsigned long long Sn = block_sum_1k(loc, red);
      if (Sn == 0ull) {  // no residual mass: back to p
        status |= 2;
        from_p = true;
        S = St;
      } else {
        from_p = false;
        S = Sn;
      }
    }
    if (chosen < 0) {  // every child rejected (or skipped): one draw from the last p
      auto wl = [&](int j) { return from_p ? wp(j) : resid[j]; };
      const unsigned long long tot = chunk_sums(V, wl, wsum, red);
      if (tot > 0ull) {
        const unsigned long long th = ss::shr128(ss::mul64((unsigned long long)*u_code, tot), 24);
        y = draw_token(th, V, wl, wsum, &s_cw, &s_base, &s_tok);
      }
    }
  }
  if (tid == 0) {
    if (chosen >= 0) {
      const int nc = chain_n[chosen];
      out_tokens[0] = tokens[1 + chosen * D];
      for (int i = 0; i <= nc; ++i) out_tokens[1 + i] = chain_out[chosen * D + i];
      *n_accepted = 1 + nc;
      *status_out = status | chain_status[chosen];
    } else {
      out_tokens[0] = y;
      *n_accepted = 0;
      *status_out = status;
    }
    *chain = chosen;
  }
}

}  // namespace

hipError_t launch_rows_sample(const RowsSampleArgs& a, int rows, hipStream_t s) {
  SS_LAUNCH(rows_sample_kernel, dim3(rows), dim3(kTB), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_tree_root(const uint16_t* zt, const uint16_t* zd, int V, float T, float Td, const int32_t* tokens,
                            int k, int D, const uint32_t* r_codes, const uint32_t* u_code, const int32_t* chain_n,
                            const int32_t* chain_out, const int32_t* chain_status, unsigned long long* resid,
                            int32_t* n_accepted, int32_t* chain, int32_t* out_tokens, int32_t* status,
                            hipStream_t s) {
  SS_LAUNCH(tree_root_kernel, dim3(1), dim3(kTB), 0, s, zt, zd, V, T, Td, tokens, k, D, r_codes, u_code, chain_n,
            chain_out, chain_status, resid, n_accepted, chain, out_tokens, status);
  return hipGetLastError();
}
