// Entropy-adaptive draft length ("The second ledger of speculative decoding",
// section 3.3): each draft token's output entropy is compared with two
// running class centres - the mean entropy of accepted and of rejected draft
// tokens - which gives it a soft acceptance probability p_i; after token i
// the draft goes on only while some longer length, with the tokens not yet
// drafted expected at p_i, has a higher expected efficiency
//     E(k) = (1 + sum_{m<=k} prod_{i<=m} p_i) / (k C_d / C_v + 1)
// than stopping now.  A confident draft (low entropy) runs long; a spike of
// uncertainty ends it at once.  The draft length lives on the device, so a
// recorded cycle runs unchanged: the draft steps past it skip themselves and
// the rejection round judges only the drafted tokens.
//
// Readings where the page is silent: entropy of softmax(z) at temperature 1;
// p = d_rej / (d_acc + d_rej) with d the distances to the centres (1/2 when
// both are 0; 1 while a centre is unseen); centres by an EMA that starts at
// a class's first entropy; every length 1..gamma_max is a candidate.  The
// controller runs in float64 with no contraction, in a fixed order, so its
// decisions are reproducible from the stored float32 entropies.
#include "common.h"
#include "internal.h"
#include "profile.h"

#pragma clang fp contract(off)

namespace {

constexpr int kT = 256;
constexpr int kChunk = 4096;

// state layout
enum { S_HACC = 0, S_HREJ = 1, S_SEENACC = 2, S_SEENREJ = 3, S_P = 4, S_A = 5, S_LAST = 6 };

__device__ double p_of(const double* st, double h) {
  if (st[S_SEENACC] == 0.0 || st[S_SEENREJ] == 0.0) return 1.0;
  const double da = fabs(h - st[S_HACC]);
  const double dr = fabs(h - st[S_HREJ]);
  if (da + dr == 0.0) return 0.5;
  return dr / (da + dr);
}

// Block partial of the entropy of one row: m = max finite logit of the chunk,
// s = sum exp(z - m), t = sum exp(z - m) (z - m) (float32 terms, float64 sums).
__global__ __launch_bounds__(kT) void draft_control_kernel(ControlArgs c, int step, const uint16_t* __restrict__ z,
                                                           int V, double* part, uint32_t* counter) {
  __shared__ double red[3][kT / 64];
  __shared__ bool s_last;
  if (step >= *c.draft_len) return;  // the step was not drafted (uniform over the grid)
  const int lo = blockIdx.x * kChunk, hi = min(V, lo + kChunk);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float m = -INFINITY;
  for (int j = lo + threadIdx.x; j < hi; j += kT) {
    const float v = ss::bf2f(z[j]);
    if (ss::finite(v)) m = fmaxf(m, v);
  }
  m = ss::wave_max(m);
  if (lane == 0) red[0][w] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  __syncthreads();
  double sa = 0.0, ta = 0.0;
  if (m > -INFINITY) {
    for (int j = lo + threadIdx.x; j < hi; j += kT) {
      const float v = ss::bf2f(z[j]);
      if (ss::finite(v)) {
        const float d = v - m;
        const float e = expf(d);
        sa += (double)e;
        ta += (double)e * (double)d;
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    sa += __shfl_xor(sa, o, 64);
    ta += __shfl_xor(ta, o, 64);
  }
  if (lane == 0) {
    red[1][w] = sa;
    red[2][w] = ta;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    part[3 * blockIdx.x + 0] = (double)m;
    part[3 * blockIdx.x + 1] = red[1][0] + red[1][1] + red[1][2] + red[1][3];
    part[3 * blockIdx.x + 2] = red[2][0] + red[2][1] + red[2][2] + red[2][3];
    __threadfence();
    s_last = atomicAdd(counter, 1u) == gridDim.x - 1;
  }
  __syncthreads();
  if (!s_last || threadIdx.x != 0) return;
  __threadfence();
  *counter = 0u;
  // entropy of the row: combine the chunks in order
  double M = -INFINITY;
  for (unsigned b = 0; b < gridDim.x; ++b) M = fmax(M, __builtin_nontemporal_load(part + 3 * b));
  double S = 0.0, T = 0.0;
  if (M > -INFINITY) {
    for (unsigned b = 0; b < gridDim.x; ++b) {
      const double mb = __builtin_nontemporal_load(part + 3 * b);
      if (!(mb > -INFINITY)) continue;
      const double f = exp(mb - M);
      S += f * __builtin_nontemporal_load(part + 3 * b + 1);
      T += f * (__builtin_nontemporal_load(part + 3 * b + 2) + (mb - M) * __builtin_nontemporal_load(part + 3 * b + 1));
    }
  }
  const float Hf = (M > -INFINITY && S > 0.0) ? (float)(log(S) - T / S) : 0.0f;
  c.entropy[step] = Hf;
  // controller: p of this token, running product and sum, continue or stop
  double* st = c.state;
  const double h = (double)Hf;
  const double p = p_of(st, h);
  double P = st[S_P] * p;
  double A = st[S_A] + P;
  st[S_P] = P;
  st[S_A] = A;
  const int i = step + 1;
  if (i >= c.gamma_max) return;  // the last step: the round drafted gamma_max tokens
  const double e_stop = A / ((double)i * c.c + 1.0);
  bool go = false;
  for (int k = i + 1; k <= c.gamma_max; ++k) {
    P = P * p;
    A = A + P;
    if (A / ((double)k * c.c + 1.0) > e_stop) {
      go = true;
      break;
    }
  }
  if (!go) *c.draft_len = i;
}

__device__ double ema(double centre, double seen, double h, double beta) {
  return seen == 0.0 ? h : centre + beta * (h - centre);
}

// After the rejection round: tokens 1..n update the accepted centre in order,
// token n + 1 (if drafted) the rejected one; then a fresh round.
__global__ void control_update_kernel(ControlArgs c, const int32_t* n_accepted) {
  double* st = c.state;
  const int g = *c.draft_len;
  const int n = *n_accepted;
  for (int i = 0; i < min(n, g); ++i) {
    st[S_HACC] = ema(st[S_HACC], st[S_SEENACC], (double)c.entropy[i], c.beta);
    st[S_SEENACC] = 1.0;
  }
  if (n < g) {
    st[S_HREJ] = ema(st[S_HREJ], st[S_SEENREJ], (double)c.entropy[n], c.beta);
    st[S_SEENREJ] = 1.0;
  }
  st[S_LAST] = (double)g;
  st[S_P] = 1.0;
  st[S_A] = 1.0;
  *c.draft_len = c.gamma_max;
}

__global__ void control_init_kernel(ControlArgs c) {
  double* st = c.state;
  for (int i = 0; i < 8; ++i) st[i] = 0.0;
  st[S_P] = 1.0;
  st[S_A] = 1.0;
  *c.draft_len = c.gamma_max;
}

}  // namespace

int control_chunks(int vocab) { return (vocab + kChunk - 1) / kChunk; }

hipError_t launch_draft_control(const ControlArgs& c, int step, const uint16_t* logits, int vocab, double* part,
                                uint32_t* counter, hipStream_t s) {
  SS_LAUNCH(draft_control_kernel, dim3(control_chunks(vocab)), dim3(kT), 0, s, c, step, logits, vocab, part,
            counter);
  return hipGetLastError();
}

hipError_t launch_control_update(const ControlArgs& c, const int32_t* n_accepted, hipStream_t s) {
  SS_LAUNCH(control_update_kernel, dim3(1), dim3(1), 0, s, c, n_accepted);
  return hipGetLastError();
}

hipError_t launch_control_init(const ControlArgs& c, hipStream_t s) {
  SS_LAUNCH(control_init_kernel, dim3(1), dim3(1), 0, s, c);
  return hipGetLastError();
}
