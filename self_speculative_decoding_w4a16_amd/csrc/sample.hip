// Vocabulary-wide sampling and the rejection round.
//
// Draft sampling: the draft draws each candidate from its own (sharpened)
// distribution and hands it to the verifier ("How speculative decoding makes
// LLMs go brrr", Module 1; temperature 0.2 per the "SubSpec" report, section
// 3.4, Table 5).  Rejection round: accept x_i iff r_i < p_i(x_i)/q_i(x_i),
// else draw from norm(max(0, p_i - q_i)); all accepted -> bonus draw from
// p_{gamma+1} (same digest, Module 3 and its pseudo-code).
//
// Exactness: every weight is exp(fl32(fl32(z - M)/T)) in float32 truncated to
// the integer floor(w * 2^40).  Chunk sums are 64-bit integer sums, so the
// result does not depend on the order blocks finish in; the accept test
// R * Wd_x * St < 2^24 * Wt_x * Sd is evaluated on 128-bit integers, and the
// residual max(0, Wt_j Sd - Wd_j St) is kept to 41 bits.  A draw with code U
// picks the smallest j whose inclusive prefix sum exceeds floor(U*S/2^24).
//
// Each pass reads the logits with all chunks in parallel; the last block to
// finish (arrival counter, reset by that block) does the final, sequential
// part over one chunk.
#include "common.h"
#include "internal.h"
#include "profile.h"

namespace {

constexpr int kT = 256;
constexpr int kRejChunk = 4096;

__device__ __forceinline__ unsigned long long wt(float z, float M, float T) {
  return ss::fixed_weight(z, M, T);  // 0 for non-finite logits
}

using ss::resid_w;
using ss::bitlen_minus1;

// Block-wide (256 threads) sum of unsigned 64-bit values.
__device__ unsigned long long block_sum_u64(unsigned long long v, unsigned long long* red) {
  v = ss::wave_sum_u64(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// Block-wide inclusive scan of unsigned 64-bit values (256 threads).
__device__ unsigned long long block_scan_u64(unsigned long long v, unsigned long long* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    unsigned long long t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  __syncthreads();
  if (lane == 63) red[w] = v;
  __syncthreads();
  unsigned long long off = 0;
  for (int i = 0; i < w; ++i) off += red[i];
  return v + off;
}

// First index j in [lo, hi) with base + prefix_j > th, where prefix is the
// inclusive prefix of weight(j); returns hi - 1 if none (cannot happen when
// the chunk's total crosses th).
template <typename F>
__device__ int scan_pick(int lo, int hi, unsigned long long base, unsigned long long th, F weight,
                         unsigned long long* red, int* s_pick) {
  if (threadIdx.x == 0) *s_pick = hi - 1;
  __syncthreads();
  for (int t0 = lo; t0 < hi; t0 += kT) {
    const int j = t0 + threadIdx.x;
    const unsigned long long w = (j < hi) ? weight(j) : 0ull;
    const unsigned long long incl = block_scan_u64(w, red);
    const bool hit = (j < hi) && (base + incl > th);
    // lowest hitting thread
    const unsigned long long bal = __ballot(hit);
    __shared__ int s_first[4];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    if (lane == 0) s_first[wv] = bal ? (int)__ffsll((long long)bal) - 1 + 64 * wv : 1 << 30;
    __syncthreads();
    int first = min(min(s_first[0], s_first[1]), min(s_first[2], s_first[3]));
    if (first < (1 << 30)) {
      if (threadIdx.x == 0) *s_pick = t0 + first;
      __syncthreads();
      return *s_pick;
    }
    base += red[0] + red[1] + red[2] + red[3];
    __syncthreads();
  }
  return *s_pick;
}

__device__ ss::ArgMax block_argmax(ss::ArgMax a, float* rv, int* ri) {
  a = ss::wave_argmax(a);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) {
    rv[w] = a.v;
    ri[w] = a.i;
  }
  __syncthreads();
  ss::ArgMax b = {rv[0], ri[0]};
  for (int i = 1; i < 4; ++i) b = ss::better(b, ss::ArgMax{rv[i], ri[i]});
  return b;
}

// ------------------------------------------------------------------ draft sampling
__global__ __launch_bounds__(kT) void rowmax_kernel(const uint16_t* __restrict__ z, int V,
                                                    float* part_max, int32_t* part_arg) {
  __shared__ float rv[4];
  __shared__ int ri[4];
  const int cs = (V + gridDim.x - 1) / gridDim.x;
  const int lo = blockIdx.x * cs, hi = min(V, lo + cs);
  ss::ArgMax a = {-INFINITY, 0x7fffffff};
  for (int j = lo + threadIdx.x; j < hi; j += kT) a = ss::better(a, ss::cand(ss::bf2f(z[j]), j));
  a = block_argmax(a, rv, ri);
  if (threadIdx.x == 0) {
    part_max[blockIdx.x] = a.v;
    part_arg[blockIdx.x] = a.i;
  }
}

__global__ __launch_bounds__(kT) void sample_kernel(const uint16_t* __restrict__ z, int V, float T,
                                                    const uint32_t* u_code, const float* pre_max,
                                                    const int32_t* pre_arg, int n_pre,
                                                    int32_t* token, const int32_t* valid,
                                                    SampleWs ws) {
  __shared__ float rv[4];
  __shared__ int ri[4];
  __shared__ unsigned long long red[4];
  __shared__ int s_pick;
  __shared__ bool s_last;
  // the first PRE partials of each thread are loaded before the position flag
  // is tested (indices clamped, masked after)
  constexpr int PRE = 8;
  const int vflag = valid ? *valid : 1;
  float pm[PRE];
  int pa[PRE];
#pragma unroll
  for (int t = 0; t < PRE; ++t) {
    const int i = min((int)threadIdx.x + t * kT, n_pre - 1);
    pm[t] = pre_max[i];
    pa[t] = pre_arg[i];
  }
  if (vflag == 0) return;
  ss::ArgMax a = {-INFINITY, 0x7fffffff};
#pragma unroll
  for (int t = 0; t < PRE; ++t)
    if ((int)threadIdx.x + t * kT < n_pre) a = ss::better(a, ss::ArgMax{pm[t], pa[t]});
  for (int i = threadIdx.x + PRE * kT; i < n_pre; i += kT) a = ss::better(a, ss::ArgMax{pre_max[i], pre_arg[i]});
  a = block_argmax(a, rv, ri);
  if (T == 0.0f) {
    if (blockIdx.x == 0 && threadIdx.x == 0) *token = ss::argmax_token(a);
    return;
  }
  const float M = a.v;
  const int cs = (V + gridDim.x - 1) / gridDim.x;
  const int lo = blockIdx.x * cs, hi = min(V, lo + cs);
  unsigned long long s = 0;
  for (int j = lo + threadIdx.x; j < hi; j += kT) s += wt(ss::bf2f(z[j]), M, T);
  s = block_sum_u64(s, red);
  if (threadIdx.x == 0) {
    ws.chunk_sum[blockIdx.x] = s;
    __threadfence();
    s_last = atomicAdd(ws.counter, 1u) == gridDim.x - 1;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  if (threadIdx.x == 0) *ws.counter = 0u;
  // totals and the chunk holding the threshold (exact integer arithmetic)
  __shared__ unsigned long long s_base, s_th;
  __shared__ int s_chunk;
  if (threadIdx.x == 0) {
    unsigned long long S = 0;
    for (unsigned c = 0; c < gridDim.x; ++c) S += __builtin_nontemporal_load(ws.chunk_sum + c);
    const unsigned long long th = S == 0 ? 0 : ss::shr128(ss::mul64((unsigned long long)*u_code, S), 24);
    unsigned long long base = 0;
    int chunk = gridDim.x - 1;
    for (unsigned c = 0; c < gridDim.x; ++c) {
      const unsigned long long cs_ = __builtin_nontemporal_load(ws.chunk_sum + c);
      if (base + cs_ > th) {
        chunk = c;
        break;
      }
      base += cs_;
    }
    s_base = base;
    s_th = th;
    s_chunk = S == 0 ? -1 : chunk;
  }
  __syncthreads();
  if (s_chunk < 0) {  // no finite logit, no mass: token 0
    if (threadIdx.x == 0) *token = ss::argmax_token(a);
    return;
  }
  const int clo = s_chunk * cs, chi = min(V, clo + cs);
  const int j = scan_pick(clo, chi, s_base, s_th,
                          [&](int jj) { return wt(ss::bf2f(z[jj]), M, T); }, red, &s_pick);
  if (threadIdx.x == 0) *token = j;
}

// ------------------------------------------------------------------ rejection round
// rows: r in [0, gamma]: target row r; r in [gamma+1, 2 gamma]: draft row r-gamma-1
__device__ __forceinline__ const uint16_t* row_ptr(const uint16_t* zt, const uint16_t* zd, int gamma,
                                                   int V, int r) {
  return r <= gamma ? zt + (int64_t)r * V : zd + (int64_t)(r - gamma - 1) * V;
}

// Batch element b = blockIdx.z: its scratch rows (each element has its own
// [rows][C] arrays, [C] residual sums and arrival counter).
__device__ __forceinline__ RejectWs ws_at(RejectWs ws, int b, int rows, int C) {
  const int64_t rc = (int64_t)rows * C;
  ws.row_max += b * rc;
  ws.row_arg += b * rc;
  ws.row_bad += b * rc;
  ws.row_sum += b * rc;
  ws.res_sum += (int64_t)b * C;
  ws.counter += b;
  return ws;
}

__global__ __launch_bounds__(kT) void rej_rowmax_kernel(const uint16_t* zt, const uint16_t* zd,
                                                        int gamma, int V, RejectWs ws) {
  __shared__ float rv[4];
  __shared__ int ri[4];
  __shared__ int s_bad;
  const int c = blockIdx.x, r = blockIdx.y, C = gridDim.x, bz = blockIdx.z;
  zt += (int64_t)bz * (gamma + 1) * V;
  zd += (int64_t)bz * gamma * V;
  ws = ws_at(ws, bz, 2 * gamma + 1, C);
  const uint16_t* z = row_ptr(zt, zd, gamma, V, r);
  const int lo = c * kRejChunk, hi = min(V, lo + kRejChunk);
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  ss::ArgMax a = {-INFINITY, 0x7fffffff};
  int bad = 0;
  for (int j = lo + threadIdx.x; j < hi; j += kT) {
    const float v = ss::bf2f(z[j]);
    bad |= !ss::finite(v);
    a = ss::better(a, ss::cand(v, j));
  }
  if (bad) atomicOr(&s_bad, 1);
  a = block_argmax(a, rv, ri);
  if (threadIdx.x == 0) {
    ws.row_max[r * C + c] = a.v;
    ws.row_arg[r * C + c] = a.i;
    ws.row_bad[r * C + c] = s_bad;
  }
}

__global__ __launch_bounds__(kT) void rej_rowsum_kernel(const uint16_t* zt, const uint16_t* zd,
                                                        int gamma, int V, float T, float Td,
                                                        RejectWs ws) {
  __shared__ unsigned long long red[4];
  const int c = blockIdx.x, r = blockIdx.y, C = gridDim.x, bz = blockIdx.z;
  const float temp = r <= gamma ? T : Td;
  if (temp == 0.0f) return;
  zt += (int64_t)bz * (gamma + 1) * V;
  zd += (int64_t)bz * gamma * V;
  ws = ws_at(ws, bz, 2 * gamma + 1, C);
  float M = -INFINITY;
  for (int i = 0; i < C; ++i) M = fmaxf(M, ws.row_max[r * C + i]);
  const uint16_t* z = row_ptr(zt, zd, gamma, V, r);
  const int lo = c * kRejChunk, hi = min(V, lo + kRejChunk);
  unsigned long long s = 0;
  for (int j = lo + threadIdx.x; j < hi; j += kT) s += wt(ss::bf2f(z[j]), M, temp);
  s = block_sum_u64(s, red);
  if (threadIdx.x == 0) ws.row_sum[r * C + c] = s;
}

struct RowStat {
  float M;
  int A;
  int bad;
  unsigned long long S;
};

__global__ __launch_bounds__(kT) void rej_decide_kernel(const uint16_t* zt, const uint16_t* zd,
                                                        int gamma, int V, float T, float Td,
                                                        const int32_t* toks, const uint32_t* r_codes,
                                                        const uint32_t* u_code, int32_t* n_out,
                                                        int32_t* out_tokens, int32_t* status_out,
                                                        float* probs, RejectWs ws,
                                                        const int32_t* gamma_len, int tok_stride,
                                                        int r_stride, int u_stride) {
  __shared__ RowStat st[129];
  __shared__ int s_n, s_status;
  __shared__ unsigned long long red[4];
  __shared__ int s_pick;
  __shared__ bool s_last;
  const int C = (V + kRejChunk - 1) / kRejChunk;
  const int rows = 2 * gamma + 1;
  {  // batch element blockIdx.z: its logits, tokens, uniforms, outputs and scratch
    const int bz = blockIdx.z;
    zt += (int64_t)bz * (gamma + 1) * V;
    zd += (int64_t)bz * gamma * V;
    toks += (int64_t)bz * tok_stride;
    if (r_codes) r_codes += (int64_t)bz * r_stride;
    if (u_code) u_code += (int64_t)bz * u_stride;
    if (gamma_len) gamma_len += bz;
    n_out += bz;
    out_tokens += (int64_t)bz * (gamma + 1);
    status_out += bz;
    if (probs) probs += (int64_t)bz * 2 * gamma;
    ws = ws_at(ws, bz, rows, C);
  }
  for (int r = threadIdx.x; r < rows; r += kT) {
    RowStat s = {-INFINITY, ss::kNoIndex, 0, 0ull};
    for (int c = 0; c < C; ++c) {
      const ss::ArgMax b = {ws.row_max[r * C + c], ws.row_arg[r * C + c]};
      ss::ArgMax cur = {s.M, s.A};
      cur = ss::better(cur, b);
      s.M = cur.v;
      s.A = cur.i;
      s.bad |= ws.row_bad[r * C + c];
      const float temp = r <= gamma ? T : Td;
      if (temp != 0.0f) s.S += ws.row_sum[r * C + c];
    }
    s.A = ss::argmax_token(ss::ArgMax{s.M, s.A});  // no finite logit: token 0
    st[r] = s;
  }
  __syncthreads();
  const bool writer = (T == 0.0f) ? (blockIdx.x == 0) : false;
  // a draft stopped early: only its first g tokens are judged (g <= gamma)
  const int g = gamma_len ? min(max(*gamma_len, 0), gamma) : gamma;
  if (threadIdx.x == 0) {
    int status = 0, n = g;
    for (int i = 0; i < g; ++i) {
      const int x = toks[i];
      const RowStat& t = st[i];
      const RowStat& d = st[gamma + 1 + i];
      status |= (t.bad | d.bad) ? 1 : 0;
      bool ok;
      float pp, qq;
      if (x < 0 || x >= V) {  // not a vocabulary id: rejected, never read
        ok = false;
        pp = qq = 0.0f;
        status |= 4;
      } else if (T == 0.0f) {
        ok = (x == t.A);
        pp = ok ? 1.0f : 0.0f;
        qq = (Td == 0.0f) ? (x == d.A ? 1.0f : 0.0f)
             : d.S ? (float)((double)wt(ss::bf2f(zd[(int64_t)i * V + x]), d.M, Td) / (double)d.S) : 0.0f;
      } else {
        const unsigned long long Wt = wt(ss::bf2f(zt[(int64_t)i * V + x]), t.M, T);
        unsigned long long Wd, Sd;
        if (Td == 0.0f) {
          Wd = (x == d.A) ? 1ull : 0ull;
          Sd = 1ull;
        } else {
          Wd = wt(ss::bf2f(zd[(int64_t)i * V + x]), d.M, Td);
          Sd = d.S;
        }
        if (Wd == 0ull) status |= 4;
        const ss::U128 lhs = ss::mul64((unsigned long long)r_codes[i] * Wd, t.S);
        const ss::U128 rhs = ss::shl128(ss::mul64(Wt, Sd), 24);
        ok = ss::lt128(lhs, rhs);
        pp = t.S ? (float)((double)Wt / (double)t.S) : 0.0f;
        qq = Sd ? (float)((double)Wd / (double)Sd) : 0.0f;
      }
      if (probs && blockIdx.x == 0) {
        probs[2 * i] = pp;
        probs[2 * i + 1] = qq;
      }
      if (!ok) {
        n = i;
        break;
      }
    }
    status |= st[n].bad ? 1 : 0;
    s_n = n;
    s_status = status;
  }
  __syncthreads();
  const int n = s_n;
  if (T == 0.0f) {
    if (writer && threadIdx.x == 0) {
      for (int i = 0; i < n; ++i) out_tokens[i] = toks[i];
      out_tokens[n] = st[n].A;
      *n_out = n;
      *status_out = s_status;
    }
    return;
  }
  // stochastic: residual (n < gamma) or bonus (n == gamma) draw from row n
  const RowStat t = st[n];
  const bool resid = n < g;
  RowStat d = {0.f, 0, 0, 1ull};
  if (resid) d = st[gamma + 1 + n];
  const bool dgreedy = (Td == 0.0f);
  const unsigned long long Sd = resid ? (dgreedy ? 1ull : d.S) : 1ull;
  const int shift = bitlen_minus1(Sd);
  const uint16_t* zrow_t = zt + (int64_t)n * V;
  const uint16_t* zrow_d = zd + (int64_t)n * V;
  auto wres = [&](int j) -> unsigned long long {
    const unsigned long long Wt = wt(ss::bf2f(zrow_t[j]), t.M, T);
    if (!resid) return Wt;
    const unsigned long long Wd = dgreedy ? (j == d.A ? 1ull : 0ull) : wt(ss::bf2f(zrow_d[j]), d.M, Td);
    return resid_w(Wt, Sd, Wd, t.S, shift);
  };
  const int c = blockIdx.x;
  const int lo = c * kRejChunk, hi = min(V, lo + kRejChunk);
  unsigned long long s = 0;
  if (resid) {
    for (int j = lo + threadIdx.x; j < hi; j += kT) s += wres(j);
    s = block_sum_u64(s, red);
  } else {
    s = ws.row_sum[n * C + c];
  }
  if (threadIdx.x == 0) {
    ws.res_sum[c] = s;
    __threadfence();
    s_last = atomicAdd(ws.counter, 1u) == gridDim.x - 1;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  __shared__ unsigned long long s_base, s_th;
  __shared__ int s_chunk;
  __shared__ bool s_fallback;
  if (threadIdx.x == 0) {
    *ws.counter = 0u;
    unsigned long long S = 0;
    for (int i = 0; i < C; ++i) S += __builtin_nontemporal_load(ws.res_sum + i);
    bool fallback = false;
    if (S == 0ull && resid) {  // no residual mass: draw from p
      fallback = true;
      S = t.S;
    }
    const unsigned long long th = ss::shr128(ss::mul64((unsigned long long)*u_code, S), 24);
    unsigned long long base = 0;
    int chunk = C - 1;
    for (int i = 0; i < C; ++i) {
      const unsigned long long cs_ = fallback ? ws.row_sum[n * C + i] : __builtin_nontemporal_load(ws.res_sum + i);
      if (base + cs_ > th) {
        chunk = i;
        break;
      }
      base += cs_;
    }
    s_base = base;
    s_th = th;
    s_chunk = S == 0ull ? -1 : chunk;  // p without mass (no finite logit): token 0
    s_fallback = fallback;
  }
  __syncthreads();
  const int clo = s_chunk * kRejChunk, chi = min(V, clo + kRejChunk);
  int y;
  if (s_chunk < 0) {
    y = 0;
  } else if (s_fallback) {
    y = scan_pick(clo, chi, s_base, s_th, [&](int j) { return wt(ss::bf2f(zrow_t[j]), t.M, T); }, red,
                  &s_pick);
  } else {
    y = scan_pick(clo, chi, s_base, s_th, wres, red, &s_pick);
  }
  if (threadIdx.x == 0) {
    for (int i = 0; i < n; ++i) out_tokens[i] = toks[i];
    out_tokens[n] = y;
    *n_out = n;
    *status_out = s_status | (s_fallback ? 2 : 0);
  }
}

}  // namespace

int sample_chunks(int vocab) {
  int c = (vocab + 2047) / 2048;
  if (c > 64) c = 64;
  if (c < 1) c = 1;
  return c;
}

hipError_t launch_rowmax(const uint16_t* logits, int vocab, float* part_max, int32_t* part_arg,
                         int n_chunks, hipStream_t s) {
  SS_LAUNCH(rowmax_kernel, dim3(n_chunks), dim3(kT), 0, s, logits, vocab, part_max, part_arg);
  return hipGetLastError();
}

hipError_t launch_sample(const uint16_t* logits, int vocab, float temp, const uint32_t* u_code,
                         const float* pre_max, const int32_t* pre_arg, int n_pre, int32_t* token,
                         const int32_t* valid, const SampleWs& ws, hipStream_t s) {
  SS_LAUNCH(sample_kernel, dim3(sample_chunks(vocab)), dim3(kT), 0, s, logits, vocab, temp,
                     u_code, pre_max, pre_arg, n_pre, token, valid, ws);
  return hipGetLastError();
}

int reject_chunks(int vocab) { return (vocab + kRejChunk - 1) / kRejChunk; }

size_t reject_ws_bytes(int gamma, int vocab) {
  const size_t C = (size_t)reject_chunks(vocab), rows = (size_t)(2 * gamma + 1);
  return rows * C * (4 + 4 + 4 + 8) + C * 8 + 256;
}

hipError_t launch_reject(int gamma, int vocab, float temp, float draft_temp, const uint16_t* zt,
                         const uint16_t* zd, const int32_t* toks, const uint32_t* r_codes,
                         const uint32_t* u_code, int32_t* n_out, int32_t* out_tokens,
                         int32_t* status, float* probs, const RejectWs& ws, hipStream_t s,
                         const int32_t* gamma_len, int batch, int tok_stride, int r_stride, int u_stride) {
  const int C = reject_chunks(vocab), rows = 2 * gamma + 1;
  SS_LAUNCH(rej_rowmax_kernel, dim3(C, rows, batch), dim3(kT), 0, s, zt, zd, gamma, vocab, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (temp != 0.0f || draft_temp != 0.0f) {
    SS_LAUNCH(rej_rowsum_kernel, dim3(C, rows, batch), dim3(kT), 0, s, zt, zd, gamma, vocab, temp,
                       draft_temp, ws);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int blocks = temp == 0.0f ? 1 : C;
  SS_LAUNCH(rej_decide_kernel, dim3(blocks, 1, batch), dim3(kT), 0, s, zt, zd, gamma, vocab, temp,
                     draft_temp, toks, r_codes, u_code, n_out, out_tokens, status, probs, ws, gamma_len,
                     tok_stride < 0 ? gamma : tok_stride, r_stride < 0 ? gamma : r_stride,
                     u_stride < 0 ? 1 : u_stride);
  return hipGetLastError();
}
