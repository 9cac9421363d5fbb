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
// inverse CDF in ascending token order.  One block of 1024 threads per row;
// thread i owns the contiguous segment [i s, i s + s) of the vocabulary.
#include "common.h"
#include "internal.h"
#include "profile.h"

namespace {

constexpr int kTB = 1024;
constexpr int kTW = kTB / 64;

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

// Exclusive prefix of the threads' values (thread order) and their total.
__device__ unsigned long long block_excl_1k(unsigned long long v, unsigned long long* red,
                                            unsigned long long* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  unsigned long long incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned long long t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  __syncthreads();
  if (lane == 63) red[w] = incl;
  __syncthreads();
  unsigned long long off = 0, tot = 0;
  for (int i = 0; i < kTW; ++i) {
    if (i < w) off += red[i];
    tot += red[i];
  }
  *total = tot;
  return off + incl - v;
}

// Smallest j whose inclusive prefix weight exceeds th (0 <= th < total):
// the thread whose segment [lo, hi) holds it walks the segment.
template <typename F>
__device__ int seg_pick(unsigned long long th, unsigned long long base, unsigned long long mine, int lo, int hi,
                        F weight, int* s_tok) {
  __syncthreads();
  if (mine > 0 && base <= th && th - base < mine) {
    unsigned long long c = base;
    for (int j = lo; j < hi; ++j) {
      c += weight(j);
      if (c > th) {
        *s_tok = j;
        break;
      }
    }
  }
  __syncthreads();
  const int t = *s_tok;
  __syncthreads();  // read by every thread before s_tok is set again
  return t;
}

__global__ __launch_bounds__(kTB) void rows_sample_kernel(RowsSampleArgs a) {
  __shared__ float rv[kTW];
  __shared__ int ri[kTW];
  __shared__ unsigned long long red[kTW];
  __shared__ int s_tok;
  const int r = blockIdx.x, tid = threadIdx.x, V = a.V;
  const uint16_t* z = a.logits + (int64_t)r * a.ld;
  const int seg = (V + kTB - 1) / kTB;
  const int lo = min(V, tid * seg), hi = min(V, lo + seg);
  const bool fits = a.kv_len[(int64_t)r * a.kv_row] + a.need <= a.cap;
  auto out_slot = [&](int i) { return a.tokens + (int64_t)r * a.t_row + (int64_t)i * a.t_out; };
  if (!fits) {  // past the cache: no candidate (the round skips it)
    if (tid < a.nout) *out_slot(tid) = -1;
    return;
  }
  ss::ArgMax am = {-INFINITY, ss::kNoIndex};
  for (int j = lo; j < hi; ++j) am = ss::better(am, ss::cand(ss::bf2f(z[j]), j));
  am = block_argmax_1k(am, rv, ri);
  if (a.T == 0.0f) {
    if (tid == 0) *out_slot(0) = ss::argmax_token(am);
    ss::ArgMax prev = am;
    for (int c = 1; c < a.nout; ++c) {  // next in (larger value, lower index) order
      ss::ArgMax b = {-INFINITY, ss::kNoIndex};
      if (prev.i != ss::kNoIndex) {
        for (int j = lo; j < hi; ++j) {
          const ss::ArgMax cj = ss::cand(ss::bf2f(z[j]), j);
          if (cj.i != ss::kNoIndex && (cj.v < prev.v || (cj.v == prev.v && cj.i > prev.i))) b = ss::better(b, cj);
        }
      }
      b = block_argmax_1k(b, rv, ri);
      if (tid == 0) *out_slot(c) = ss::argmax_token(b);
      prev = b;
    }
    return;
  }
  const float M = am.v, T = a.T;
  unsigned long long mine = 0;
  for (int j = lo; j < hi; ++j) mine += wt(ss::bf2f(z[j]), M, T);
  unsigned long long S;
  const unsigned long long base = block_excl_1k(mine, red, &S);
  for (int i = 0; i < a.nout; ++i) {
    const uint32_t uc = a.u[(int64_t)r * a.u_row + (int64_t)i * a.u_out];
    int tok = 0;
    if (S > 0) {
      if (tid == 0) s_tok = V - 1;
      const unsigned long long th = ss::shr128(ss::mul64((unsigned long long)uc, S), 24);
      tok = seg_pick(th, base, mine, lo, hi, [&](int j) { return wt(ss::bf2f(z[j]), M, T); }, &s_tok);
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
  __shared__ int s_tok;
  const int tid = threadIdx.x;
  const int seg = (V + kTB - 1) / kTB;
  const int lo = min(V, tid * seg), hi = min(V, lo + seg);
  ss::ArgMax at = {-INFINITY, ss::kNoIndex}, ad = {-INFINITY, ss::kNoIndex};
  int bad = 0;
  for (int j = lo; j < hi; ++j) {
    const float a = ss::bf2f(zt[j]), b = ss::bf2f(zd[j]);
    bad |= !ss::finite(a) || !ss::finite(b);
    at = ss::better(at, ss::cand(a, j));
    ad = ss::better(ad, ss::cand(b, j));
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
    unsigned long long mine = 0;
    for (int j = lo; j < hi; ++j) mine += wp(j);
    const unsigned long long St = block_sum_1k(mine, red);
    unsigned long long Sd = 1;
    if (Td != 0.0f) {
      unsigned long long md = 0;
      for (int j = lo; j < hi; ++j) md += wt(ss::bf2f(zd[j]), Md, Td);
      Sd = block_sum_1k(md, red);
    }
    bool from_p = true;  // the current weights are p's own (else the residual array)
    unsigned long long S = St;
    for (int c = 0; c < k; ++c) {
      const int x = tokens[1 + c * D];
      if (x < 0 || x >= V) {  // not a vocabulary id: skipped
        status |= 4;
        continue;
      }
      const unsigned long long Wdx = Td == 0.0f ? 1ull : wt(ss::bf2f(zd[x]), Md, Td);
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
      for (int j = lo; j < hi; ++j) {
        const unsigned long long Wj = from_p ? wp(j) : resid[j];
        const unsigned long long Wdj = Td == 0.0f ? (j == x ? 1ull : 0ull) : wt(ss::bf2f(zd[j]), Md, Td);
        const unsigned long long w = ss::resid_w(Wj, Sd, Wdj, S, shift);
        resid[j] = w;
        loc += w;
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
      unsigned long long m2 = 0;
      for (int j = lo; j < hi; ++j) m2 += from_p ? wp(j) : resid[j];
      unsigned long long tot;
      const unsigned long long base = block_excl_1k(m2, red, &tot);
      if (tot > 0ull) {
        if (tid == 0) s_tok = V - 1;
        const unsigned long long th = ss::shr128(ss::mul64((unsigned long long)*u_code, tot), 24);
        y = seg_pick(th, base, m2, lo, hi, [&](int j) { return from_p ? wp(j) : resid[j]; }, &s_tok);
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
