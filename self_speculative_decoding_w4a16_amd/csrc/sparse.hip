// Sparse draft index ("The second ledger of speculative decoding", sections
// 3.1-3.2): after each verify the index of every layer and KV head is rebuilt
// from the verify pass's importance scores over the committed positions
// [0, L), L = kv_len: sink = [0, s), recent = [r, L), and the K middle
// positions of [s, r) with the highest scores (score descending, position
// ascending on ties), K = ceil(budget_permille * L / 1000) - s - (L - r)
// clipped to [0, r - s).  The list is ascending.
//
// One block (1024 threads) per list.  Scores are non-negative floats, so
// their bit patterns order like the values: a 4-pass radix select (8 bits a
// pass, histogram in LDS) finds the bits T of the K-th highest score and how
// many positions equal to T must be taken; an ordered compaction over the
// middle then takes every position above T and the first ones equal to T,
// in position order (ballot prefix counts within a wave, wave totals through
// LDS).
#include "common.h"
#include "internal.h"
#include "profile.h"

namespace {

constexpr int kT = 1024;
constexpr int kW = kT / SS_WAVE;

// Exclusive prefix count of `flag` over the block in thread order, and the
// block total.  Every thread calls it.
__device__ __forceinline__ int block_prefix(bool flag, int* wtot, int* total) {
  const int lane = threadIdx.x & (SS_WAVE - 1), wave = threadIdx.x / SS_WAVE;
  const unsigned long long b = __ballot(flag);
  const int in_wave = __popcll(b & ((1ull << lane) - 1ull));
  if (lane == 0) wtot[wave] = __popcll(b);
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < kW; ++w) {
    const int t = wtot[w];
    before += (w < wave) ? t : 0;
    all += t;
  }
  __syncthreads();  // wtot is reused by the next call
  *total = all;
  return before + in_wave;
}

__global__ __launch_bounds__(kT) void kv_select_kernel(const float* score, int cap, const int32_t* kv_len,
                                                       int n_sink, int n_recent, int permille,
                                                       int32_t* index, int index_cap, int32_t* index_len) {
  __shared__ unsigned int hist[256];
  __shared__ unsigned int sel_prefix;
  __shared__ int sel_rem;
  __shared__ int wtot[kW];
  const int tid = threadIdx.x;
  const int64_t list = blockIdx.x;
  const uint32_t* bits = reinterpret_cast<const uint32_t*>(score + list * cap);
  int32_t* out = index + list * index_cap;
  const int L = min(max(*kv_len, 0), cap);
  const int s = min(n_sink, L);
  const int r = max(s, L - n_recent);
  const int64_t total = ((int64_t)permille * L + 999) / 1000;
  const int K = (int)min(max(total - s - (L - r), (int64_t)0), (int64_t)(r - s));
  const int count = s + K + (L - r);
  if (count > index_cap) return;  // the host checked index_cap against capacity
  if (list == 0 && tid == 0) *index_len = count;
  for (int t = tid; t < s; t += kT) out[t] = t;
  for (int t = tid; t < L - r; t += kT) out[s + K + t] = r + t;
  if (K == 0) return;
  if (K == r - s) {
    for (int t = tid; t < K; t += kT) out[s + t] = s + t;
    return;
  }
  // ---- radix select of the K-th highest score bits over [s, r)
  unsigned int prefix = 0, mask = 0;
  int rem = K;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += kT) hist[i] = 0;
    __syncthreads();
    for (int j = s + tid; j < r; j += kT) {
      const unsigned int u = bits[j];
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      int above = 0;
      for (int b = 255; b >= 0; --b) {
        const int h = (int)hist[b];
        if (above + h >= rem) {
          sel_prefix = prefix | ((unsigned int)b << shift);
          sel_rem = rem - above;
          break;
        }
        above += h;
      }
    }
    __syncthreads();
    prefix = sel_prefix;
    rem = sel_rem;
    mask |= 255u << shift;
  }
  // ---- ordered compaction: every score above T, the first `rem` equal to T
  const unsigned int T = prefix;
  int taken = 0, eq_seen = 0;
  for (int c0 = s; c0 < r; c0 += kT) {  // block-uniform trip count
    const int j = c0 + tid;
    const bool ok = j < r;
    const unsigned int u = ok ? bits[j] : 0u;
    const bool gt = ok && u > T, eq = ok && u == T;
    int n_eq = 0, n_take = 0;
    const int eq_rank = block_prefix(eq, wtot, &n_eq);
    const bool take = gt || (eq && eq_seen + eq_rank < rem);
    const int at = block_prefix(take, wtot, &n_take);
    if (take && taken + at < K) out[s + taken + at] = j;
    taken += n_take;
    eq_seen += n_eq;
  }
}

}  // namespace

hipError_t launch_kv_select(const float* score, int cap, const int32_t* kv_len, int n_lists, int n_sink,
                            int n_recent, int budget_permille, int32_t* index, int index_cap,
                            int32_t* index_len, hipStream_t s) {
  SS_LAUNCH(kv_select_kernel, dim3(n_lists), dim3(kT), 0, s, score, cap, kv_len, n_sink, n_recent,
            budget_permille, index, index_cap, index_len);
  return hipGetLastError();
}
