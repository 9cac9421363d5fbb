// Batch-1 GEMV of the draft step on 4- or 2-bit substitute weights stored in
// 16-row tiles, on the matrix cores.  Low-batch decode streams the weights
// from memory ("How speculative decoding makes LLMs go brrr", Module 2), so
// the layout and the kernel are built around the weight stream:
//
//  * Tiled layout (subspec_tile_codes): a chunk is 64 bytes of a row (128 k
//    at 4 bits, two 64-groups; 256 k at 2 bits, four groups); the codes of
//    rows 16 tau .. 16 tau + 15 and chunk c are one contiguous KiB, the 16
//    bytes of lane l = 16 g + r at 16 l holding bytes 64 c + 16 g .. + 15 of
//    row 16 tau + r; the scale/min dwords of those rows and groups follow in
//    row order.  Every wave load then reads one contiguous KiB, where the
//    row-major layout needs 16 pieces of 64 bytes from 16 rows.
//  * v_mfma_f32_16x16x32_bf16 with B = 32 k x 16 tile rows as (128 + q) bf16
//    values (one and-or per field pair, exact) and A = the activations on
//    the lanes of one group per A row, every other A value 0: at 4 bits row
//    0 holds x on the lanes of the chunk's first group (g = 0, 1) and row 8
//    on its second's (g = 2, 3); at 2 bits row 4 g holds x on the lanes of
//    group g.  So each D row holds one group's sums per tile row, scaled by
//    that group's own scale and min:
//        sum_k (q s + m) x = s * (sum_k (128 + q) x - 128 X) + m X,
//    X = sum_k x over the group (from LDS).  Four MFMAs per KiB of 4-bit
//    codes (eight at 2 bits) replace the VALU GEMV's v_dot2 and most of its
//    per-chunk scale work; the field extraction (7 VALU per 4-bit code word,
//    15 per 2-bit word) stays.
//  * A block of 8 waves takes units of T tiles (T = 2: a gate tile and its
//    up tile for SiLU * up), persistent over the units; its waves split each
//    unit's chunks (wave w: chunks w, w + 8, ...) and keep P chunks in flight
//    in register slots named statically, the ring running on across units.
//    Each unit's wave partials meet in LDS (double-buffered, one barrier a
//    unit).
//  * x lives in LDS for the whole block in the pair order of the field
//    extraction ((x[k], x[k+4]) at 4 bits, (x[k], x[k+8]) at 2), with its
//    64-group sums; the RMSNorm (and for layer 0 the embedding gather) is
//    computed in the prologue of every block, its loads issued before the
//    first chunks so that their wait covers no weight load.
#include "common.h"
#include "draft_attn.h"
#include "internal.h"
#include "profile.h"

namespace {

constexpr int kW = 8;  // waves per block
constexpr int kNT = kW * SS_WAVE;
constexpr int kBufferWord3 = 0x00020000;  // buffer resource word 3 (CDNA): raw 32-bit data
constexpr int kOutside = 0x40000000;      // offset past every resource: loads zeros
// zeros in LDS for the A operand of the lanes that carry no x: one 16-byte
// slot per MFMA step of a chunk (up to 8 steps, at 2 bits)
constexpr int kZero = 128;

// offset, or one past every resource; kept in a register so the compiler
// issues the load unconditionally instead of branching around it
__device__ __forceinline__ int sel_off(bool in, int off) {
  int o = in ? off : kOutside;
  asm volatile("" : "+v"(o));
  return o;
}

// Per code width WB (4 or 2 bits): k per 64-byte piece of a row (one
// chunk), 64-groups per chunk, MFMA steps per chunk (one per 8 weights of a
// lane's 16 code bytes), the field mask of one (128 + q) bf16 pair.
template <int WB>
struct Width {
  static constexpr int KCH = 512 / WB;
  static constexpr int GPC = 8 / WB;
  static constexpr int NST = 16 / WB;
  static constexpr uint32_t MASK = WB == 4 ? 0x000F000Fu : 0x00030003u;
};

template <int T>
struct TSlot {
  u32x4 pc[T];     // 16 code bytes of the chunk, lane (r, g), each tile
  uint32_t mt[T];  // scale/min of the lane's group, row r, each tile
};

// WB-bit codes, T tiles per unit, P chunks in flight per wave, NX prologue
// items (8 values of x) per thread: K <= 8 * kNT * NX.
//
// DQR > 0: the draft step's QKV projection and its attention in one launch.
// Blocks [0, G) run the GEMV, storing its rows with agent-coherent stores and
// counting each 16-row tile into the count of its 128-row group once those
// stores are
// complete; blocks G + S hq + s run the attention of query head hq over key
// split s (draft_attn.h, DQR chunks in flight per wave), which waits for the
// counts of the rows it reads.  The GEMV blocks come first in the grid and
// wait for nothing.
template <int WB, int T, int P, int NX, int PRO, int EPI, int DQR>
__global__ __launch_bounds__(kNT) void gemv_w4t_kernel(GemvArgs a, int G, AttnArgs at, uint32_t* ready) {
  constexpr bool SIG = DQR > 0;
  static_assert(!SIG || (EPI == EPI_STORE && kNT == DQW * SS_WAVE), "the attention rides on the store epilogue");
  if constexpr (SIG) {
    if ((int)blockIdx.x >= G) {
      const int j = (int)blockIdx.x - G, S = at.head_splits;
      draft_attn_head<false, DQR, false, true>(at, a.valid, j / S, j - (j / S) * S, S, ready);
      return;
    }
  }
  using Wd = Width<WB>;
  extern __shared__ __align__(16) unsigned char smem[];
  const int K = (int)a.k;
  const int chunks = K / Wd::KCH;
  u32x4* xs = reinterpret_cast<u32x4*>(smem);           // K/8 16-byte slots of x pairs
  float* Xs = reinterpret_cast<float*>(smem + 2 * K);   // K/64 group sums
  const int zoff = 2 * K + 4 * (K / 64);                 // kZero bytes of zeros
  float* red = reinterpret_cast<float*>(smem + zoff + kZero);  // [2][kW][16 T]
  float* nred = red + 2 * kW * 16 * T;                    // [kW]

  const int vflag = a.valid ? *a.valid : 1;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  // units: SiLU - F / 16 (gate tile u, up tile F/16 + u); else n / (16 T)
  const int64_t n_phys = EPI == EPI_SILU ? 2 * a.n : a.n;
  const int units = EPI == EPI_SILU ? (int)(a.n / 16) : (int)((a.n + 16 * T - 1) / (16 * T));
  const int b = blockIdx.x;
  const int ntl = b < units ? (units - b + G - 1) / G : 0;
  const int nc = (chunks - w + kW - 1) / kW;  // chunks >= 8 (K >= 1024) or waves past them idle
  const int F = ntl * (nc > 0 ? nc : 0);
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.codes), 0, (int)(n_phys * (K / (8 / WB))), kBufferWord3);
  const __amdgpu_buffer_rsrc_t mrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.meta), 0,
                                                                       (int)(n_phys * (K / 16)), kBufferWord3);
  // first row of tile t of unit index jj of this block
  auto tile_row = [&](int jj, int t) -> int64_t {
    const int64_t u = (int64_t)b + (int64_t)G * jj;
    if (EPI == EPI_SILU) return (t == 0 ? 0 : a.n) + 16 * u;
    return 16 * (T * u + t);
  };

  // ---- prologue loads: x (or h and the norm weights) first, then P chunks
  const uint16_t* src = a.x;
  if (PRO == PRO_NORM) src = a.h;
  if (PRO == PRO_EMBED_NORM) src = a.embed + (int64_t)min(max(*a.token, 0), (int)a.vocab - 1) * K;
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(src), 0, 2 * K, kBufferWord3);
  const __amdgpu_buffer_rsrc_t grs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.norm_w), 0, PRO == PRO_X ? 0 : 2 * K, kBufferWord3);
  u32x4 xv[NX], gv[NX];
#pragma unroll
  for (int j = 0; j < NX; ++j) {
    const int o = tid + kNT * j;
    xv[j] = __builtin_amdgcn_raw_buffer_load_b128(xrs, sel_off(o < K / 8, 16 * o), 0, 0);
    if (PRO != PRO_X) gv[j] = __builtin_amdgcn_raw_buffer_load_b128(grs, sel_off(o < K / 8, 16 * o), 0, 0);
  }

  int ljj = 0, li = 0, lf = 0;  // load cursor: unit index, chunk index, item
  auto load = [&](TSlot<T>& sl) {
    const bool in = lf < F;
    const int c = w + kW * li;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int64_t row = tile_row(ljj, t);
      const bool ok = in && row < n_phys;
      const int tb = (int)(row >> 4) * chunks + c;  // tile-chunk KiB index
      sl.pc[t] = __builtin_amdgcn_raw_buffer_load_b128(crs, sel_off(ok, tb * 1024 + 16 * lane), 0, 0);
      // the lane's group: g >> 1 (4 bits, two groups a chunk) or g (2 bits, four)
      const int e = WB == 4 ? (g >> 1) : g;
      sl.mt[t] = __builtin_amdgcn_raw_buffer_load_b32(mrs, sel_off(ok, 4 * (tb * 16 * Wd::GPC + Wd::GPC * r + e)), 0,
                                                      0);
    }
    ++lf;
    if (++li == nc) {
      li = 0;
      ++ljj;
    }
  };
  TSlot<T> sl[P];
#pragma unroll
  for (int j = 0; j < P; ++j) load(sl[j]);
  if (vflag == 0) return;  // block-uniform: the whole launch is skipped

  // ---- x' in LDS: pair order, group sums
  float inv = 1.0f;
  if (PRO != PRO_X) {
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < NX; ++j) {
      const bool ok = tid + kNT * j < K / 8;
      const uint32_t wv[4] = {xv[j].x, xv[j].y, xv[j].z, xv[j].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = ok ? ss::lo_bf(wv[i]) : 0.0f, hi = ok ? ss::hi_bf(wv[i]) : 0.0f;
        ss += lo * lo;
        ss += hi * hi;
      }
    }
    ss = ss::wave_sum(ss);
    if (lane == 0) nred[w] = ss;
    __syncthreads();
    float tot = 0.0f;
#pragma unroll
    for (int i = 0; i < kW; ++i) tot += nred[i];
    inv = 1.0f / sqrtf(tot / (float)K + a.eps);
  }
#pragma unroll
  for (int j = 0; j < NX; ++j) {
    const int o = tid + kNT * j;
    const bool ok = o < K / 8;
    const uint32_t wv[4] = {xv[j].x, xv[j].y, xv[j].z, xv[j].w};
    if (PRO == PRO_EMBED_NORM && b == 0 && ok) reinterpret_cast<u32x4*>(a.h_out)[o] = xv[j];
    uint32_t xb[8];  // bf16 bits of x'
    if (PRO == PRO_X) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xb[2 * i] = wv[i] & 0xffffu;
        xb[2 * i + 1] = wv[i] >> 16;
      }
    } else {
      const uint32_t gw[4] = {gv[j].x, gv[j].y, gv[j].z, gv[j].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xb[2 * i] = ss::f2bf(ss::lo_bf(wv[i]) * inv * ss::lo_bf(gw[i]));
        xb[2 * i + 1] = ss::f2bf(ss::hi_bf(wv[i]) * inv * ss::hi_bf(gw[i]));
      }
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += ok ? ss::bf2f((uint16_t)xb[i]) : 0.0f;
    // a group's 8 octets sit in 8 consecutive lanes
    s += __shfl_xor(s, 1, SS_WAVE);
    s += __shfl_xor(s, 2, SS_WAVE);
    s += __shfl_xor(s, 4, SS_WAVE);
    u32x4 slot;
    if (WB == 4) {  // the pairs (x[k], x[k+4]) of the 8-weight word at 8 o
      slot = u32x4{xb[0] | (xb[4] << 16), xb[1] | (xb[5] << 16), xb[2] | (xb[6] << 16), xb[3] | (xb[7] << 16)};
    } else {
      // 2 bits: the 16-weight word at 16 (o >> 1) spans items o & ~1 and
      // o | 1 (neighbouring lanes); slot o holds its pairs (x[k], x[k+8]) of
      // k = 4 (o & 1) .. + 3, the fields of MFMA step o & 1 of that word
      uint32_t p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = (uint32_t)__shfl_xor((int)xb[i], 1, SS_WAVE);
      slot = (o & 1) ? u32x4{p[4] | (xb[4] << 16), p[5] | (xb[5] << 16), p[6] | (xb[6] << 16), p[7] | (xb[7] << 16)}
                     : u32x4{xb[0] | (p[0] << 16), xb[1] | (p[1] << 16), xb[2] | (p[2] << 16), xb[3] | (p[3] << 16)};
    }
    if (ok) {
      xs[o] = slot;
      if ((o & 7) == 0) Xs[o >> 3] = s;
    }
  }
  if (tid < kZero / 16) reinterpret_cast<u32x4*>(smem + zoff)[tid] = u32x4{0u, 0u, 0u, 0u};
  // registers of items past the end of x were never read: a use here settles
  // their loads before the loop (else the first reuse waits for every load)
#pragma unroll
  for (int j = 0; j < NX; ++j) {
    asm volatile("" ::"v"(xv[j]));
    if (PRO != PRO_X) asm volatile("" ::"v"(gv[j]));
  }
  __syncthreads();
  if (nc <= 0) {
    // a wave past the chunks (K < 1024) adds zero partials at every unit's
    // barrier, so the block's barrier count matches on every wave
    for (int jj = 0; jj < ntl; ++jj) {
      float* rb = red + (jj & 1) * kW * 16 * T;
#pragma unroll
      for (int t = 0; t < T; ++t)
        if (g == 0) rb[w * 16 * T + 16 * t + r] = 0.0f;
      __syncthreads();
    }
    return;
  }

  // A operand: 4 bits - lanes (r 0, g 0-1) and (r 8, g 2-3) read x (the
  // chunk's two groups in D rows 0 and 8); 2 bits - lanes r = 4 g (its four
  // groups in D rows 0, 4, 8, 12); every other lane reads zeros
  const bool real = WB == 4 ? ((r == 0 && g < 2) || (r == 8 && g >= 2)) : r == 4 * g;
  const uint32_t abase = real ? (uint32_t)(WB == 4 ? 64 * g : 128 * g) : (uint32_t)zoff;
  const uint32_t astride = real ? (uint32_t)(2 * Wd::KCH) : 0u;
  const uint32_t mask = __builtin_amdgcn_readfirstlane(Wd::MASK);
  uint32_t magic = 0x43004300u;
  asm volatile("" : "+v"(magic));

  float acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = 0.0f;
  int cjj = 0, ci = 0;  // compute cursor
  auto compute = [&](const TSlot<T>& s) {
    const int c = w + kW * ci;
    const float xg = Xs[Wd::GPC * c + (WB == 4 ? (g >> 1) : g)];
    const f32x4_t zf = {0.f, 0.f, 0.f, 0.f};
    f32x4_t d[T];
#pragma unroll
    for (int st = 0; st < Wd::NST; ++st) {
      const bf16x8_t av =
          __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(smem + abase + astride * c + 16 * st));
#pragma unroll
      for (int t = 0; t < T; ++t) {
        // 4 bits: code word st, pairs (q_i, q_i+4) at bits 4 i, 16 + 4 i;
        // 2 bits: code word st / 2, pairs (q_e, q_e+8) at bits 2 e, 16 + 2 e
        // for e = 4 (st & 1) + i
        const uint32_t cw = s.pc[t][WB == 4 ? st : st >> 1];
        const int sh0 = WB == 4 ? 0 : 8 * (st & 1), sh = WB == 4 ? 4 : 2;
        const bf16x8_t bv = __builtin_bit_cast(
            bf16x8_t, u32x4{((cw >> sh0) & mask) | magic, ((cw >> (sh0 + sh)) & mask) | magic,
                            ((cw >> (sh0 + 2 * sh)) & mask) | magic, ((cw >> (sh0 + 3 * sh)) & mask) | magic});
        d[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, st == 0 ? zf : d[t], 0, 0, 0);
      }
    }
    // the lane's own group sums sit in component 0 (D row 4 g); for 4 bits
    // only lanes g = 0 and 2 hold one (rows 0 and 8)
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float sc = ss::h2f((uint16_t)(s.mt[t] & 0xffffu)), mn = ss::h2f((uint16_t)(s.mt[t] >> 16));
      acc[t] += sc * (d[t][0] - 128.0f * xg) + mn * xg;
    }
    if (++ci == nc) {  // the wave's last chunk of unit cjj: the waves' partials meet in LDS
      float* rb = red + (cjj & 1) * kW * 16 * T;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        float v = acc[t];  // the groups of the chunk, summed into lanes g = 0
        if (WB == 2) v += __shfl_xor(v, 16, SS_WAVE);
        v += __shfl_xor(v, 32, SS_WAVE);
        if (g == 0) rb[w * 16 * T + 16 * t + r] = v;
        acc[t] = 0.0f;
      }
      __syncthreads();
      if (EPI == EPI_SILU) {
        if (tid < 16) {
          float gt = 0.0f, up = 0.0f;
#pragma unroll
          for (int q = 0; q < kW; ++q) {
            gt += rb[q * 16 * T + tid];
            up += rb[q * 16 * T + 16 + tid];
          }
          gt = ss::bf2f(ss::f2bf(gt));
          up = ss::bf2f(ss::f2bf(up));
          a.y[tile_row(cjj, 0) + tid] = ss::f2bf(gt / (1.0f + expf(-gt)) * up);
        }
      } else if (tid < 16 * T) {
        const int64_t row = tile_row(cjj, tid >> 4) + (tid & 15);
        if (row < a.n) {
          float v = 0.0f;
#pragma unroll
          for (int q = 0; q < kW; ++q) v += rb[q * 16 * T + tid];
          if (EPI == EPI_RESID) v = ss::bf2f(a.resid[row]) + v;
          if constexpr (SIG)
            __hip_atomic_store(a.y + row, ss::f2bf(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          else
            a.y[row] = ss::f2bf(v);
        }
      }
      if constexpr (SIG) {
        // the unit's rows are stored by wave 0: once they are complete at the
        // agent coherence point, each tile's 16 rows are counted in
        if (w == 0) {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          if (lane < 16 * T && (lane & 15) == 0) {
            const int64_t row = tile_row(cjj, lane >> 4);
            if (row < a.n)
              __hip_atomic_fetch_add(ready + kReadyStride * (int)(row / D), 16u, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
      ci = 0;
      ++cjj;
    }
  };
  int f = 0;
  for (; f + P <= F; f += P) {
#pragma unroll
    for (int j = 0; j < P; ++j) {
      __builtin_amdgcn_sched_barrier(0);
      compute(sl[j]);
      load(sl[j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int j = 0; j < P - 1; ++j)
    if (f + j < F) compute(sl[j]);
}

// Repack of row-major BITS-bit codes and meta into 16-row tiles: thread i
// writes the 16 code bytes of item i = (tile, chunk, lane l = 16 g + r) and,
// for g < GPC (the chunk's groups), the meta dword of row r and group g.
template <int BITS>
__global__ __launch_bounds__(256) void tile_codes_kernel(const uint8_t* __restrict__ codes,
                                                         const uint16_t* __restrict__ meta, int64_t n, int64_t k,
                                                         uint8_t* __restrict__ tcodes, uint16_t* __restrict__ tmeta) {
  using Wd = Width<BITS>;
  const int64_t chunks = k / Wd::KCH;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (n / 16) * chunks * 64) return;
  const int l = (int)(i & 63), r = l & 15, g = l >> 4;
  const int64_t tc = i >> 6;  // tile * chunks + chunk
  const int64_t tau = tc / chunks, c = tc - tau * chunks;
  const int64_t row = 16 * tau + r;
  *reinterpret_cast<u32x4*>(tcodes + tc * 1024 + 16 * l) =
      *reinterpret_cast<const u32x4*>(codes + row * (k / (8 / BITS)) + 64 * c + 16 * g);
  if (g < Wd::GPC) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(meta) + row * (k / 64) + Wd::GPC * c + g;
    reinterpret_cast<uint32_t*>(tmeta)[tc * 16 * Wd::GPC + Wd::GPC * r + g] = *src;
  }
}

int w4t_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
  }
  return cus;
}

template <int WB, int T, int P, int NX, int PRO, int EPI>
hipError_t launch_t(const GemvArgs& a, hipStream_t s) {
  const int K = (int)a.k;
  const size_t lds = (size_t)(2 * K + 4 * (K / 64) + kZero) + 4 * (2 * kW * 16 * T + kW);
  const int units = EPI == EPI_SILU ? (int)(a.n / 16) : (int)((a.n + 16 * T - 1) / (16 * T));
  // two blocks per compute unit: 16 waves of at most 128 VGPRs
  const int G = std::max(1, std::min(units, 2 * w4t_cus()));
  SS_LAUNCH((gemv_w4t_kernel<WB, T, P, NX, PRO, EPI, 0>), dim3((unsigned)G), dim3(kNT), lds, s, a, G, AttnArgs{},
            nullptr);
  return hipGetLastError();
}

// Store and SiLU sites take two tiles a unit (one x read per two MFMAs),
// with three chunks in flight (store: the narrow QKV projection, 5.6 against
// 5.8 us for two and 6.1 for four at the 7B shape) or two (SiLU: gate/up);
// residual sites (the narrow O and down projections) one tile with four
// chunks in flight (more waves per row of tiles).
template <int WB, int NX, int PRO, int EPI>
hipError_t launch_pe(const GemvArgs& a, hipStream_t s) {
  if constexpr (EPI == EPI_RESID) return launch_t<WB, 1, 4, NX, PRO, EPI>(a, s);
  else if constexpr (EPI == EPI_STORE) return launch_t<WB, 2, 3, NX, PRO, EPI>(a, s);
  else return launch_t<WB, 2, 2, NX, PRO, EPI>(a, s);
}

template <int WB, int NX>
hipError_t launch_nx(int pro, int epi, const GemvArgs& a, hipStream_t s) {
  if (pro == PRO_X && epi == EPI_STORE) return launch_pe<WB, NX, PRO_X, EPI_STORE>(a, s);
  if (pro == PRO_X && epi == EPI_RESID) return launch_pe<WB, NX, PRO_X, EPI_RESID>(a, s);
  if (pro == PRO_NORM && epi == EPI_STORE) return launch_pe<WB, NX, PRO_NORM, EPI_STORE>(a, s);
  if (pro == PRO_NORM && epi == EPI_SILU) return launch_pe<WB, NX, PRO_NORM, EPI_SILU>(a, s);
  if (pro == PRO_EMBED_NORM && epi == EPI_STORE) return launch_pe<WB, NX, PRO_EMBED_NORM, EPI_STORE>(a, s);
  return hipErrorInvalidValue;
}

template <int WB>
hipError_t launch_w(int pro, int epi, const GemvArgs& a, hipStream_t s) {
  const int items = (int)(a.k / 8);
  const int nx = (items + kNT - 1) / kNT;
  if (nx <= 1) return launch_nx<WB, 1>(pro, epi, a, s);
  if (nx <= 2) return launch_nx<WB, 2>(pro, epi, a, s);
  if (nx <= 3) return launch_nx<WB, 3>(pro, epi, a, s);
  if (nx <= 5) return launch_nx<WB, 5>(pro, epi, a, s);
  return launch_nx<WB, 7>(pro, epi, a, s);
}

template <int WB, int NX, int PRO>
hipError_t launch_qa(int dqr, const GemvArgs& a, const AttnArgs& at, uint32_t* ready, hipStream_t s) {
  constexpr int T = 2;
  const int K = (int)a.k;
  const size_t lds = (size_t)(2 * K + 4 * (K / 64) + kZero) + 4 * (2 * kW * 16 * T + kW);
  const int units = (int)((a.n + 16 * T - 1) / (16 * T));
  const int G = std::max(1, std::min(units, 2 * w4t_cus()));
  const dim3 grid((unsigned)(G + at.n_q * at.head_splits)), block(kNT);
  if (dqr == 1) SS_LAUNCH((gemv_w4t_kernel<WB, T, 3, NX, PRO, EPI_STORE, 1>), grid, block, lds, s, a, G, at, ready);
  else SS_LAUNCH((gemv_w4t_kernel<WB, T, 3, NX, PRO, EPI_STORE, 2>), grid, block, lds, s, a, G, at, ready);
  return hipGetLastError();
}

template <int WB, int NX>
hipError_t launch_qa_pro(int pro, int dqr, const GemvArgs& a, const AttnArgs& at, uint32_t* ready, hipStream_t s) {
  if (pro == PRO_NORM) return launch_qa<WB, NX, PRO_NORM>(dqr, a, at, ready, s);
  if (pro == PRO_EMBED_NORM) return launch_qa<WB, NX, PRO_EMBED_NORM>(dqr, a, at, ready, s);
  return hipErrorInvalidValue;
}

}  // namespace

bool qkv_attn_supported(int wb, int pro, int64_t n, int64_t k) {
  const int kch = tile_chunk_k(wb);
  return (wb == 4 || wb == 2) && (pro == PRO_NORM || pro == PRO_EMBED_NORM) && k % kch == 0 && n % D == 0 &&
         (k / 8 + kNT - 1) / kNT <= 2;
}

hipError_t launch_qkv_attn(int wb, int pro, const GemvArgs& a, const AttnArgs& at, int dqr, uint32_t* ready,
                           hipStream_t s) {
  if (!a.tiled || !qkv_attn_supported(wb, pro, a.n, a.k) || (dqr != 1 && dqr != 2) || at.head_splits < 1 ||
      a.n != (int64_t)(at.n_q + 2 * at.n_kv) * D)
    return hipErrorInvalidValue;
  const int nx = (int)((a.k / 8 + kNT - 1) / kNT);
  if (wb == 4) return nx <= 1 ? launch_qa_pro<4, 1>(pro, dqr, a, at, ready, s) : launch_qa_pro<4, 2>(pro, dqr, a, at, ready, s);
  return nx <= 1 ? launch_qa_pro<2, 1>(pro, dqr, a, at, ready, s) : launch_qa_pro<2, 2>(pro, dqr, a, at, ready, s);
}

bool gemv_w4t_supported(int pro, int epi) {
  return (pro == PRO_X && (epi == EPI_STORE || epi == EPI_RESID)) ||
         (pro == PRO_NORM && (epi == EPI_STORE || epi == EPI_SILU)) ||
         (pro == PRO_EMBED_NORM && epi == EPI_STORE);
}

int tile_chunk_k(int bits) { return bits == 4 ? Width<4>::KCH : (bits == 2 ? Width<2>::KCH : 0); }

hipError_t launch_gemv_w4t(int wb, int pro, int epi, const GemvArgs& a, hipStream_t s) {
  const int kch = tile_chunk_k(wb);
  if (kch == 0 || a.k % kch != 0 || a.n % 16 != 0 || a.k > 8 * kNT * 7) return hipErrorInvalidValue;
  return wb == 4 ? launch_w<4>(pro, epi, a, s) : launch_w<2>(pro, epi, a, s);
}

hipError_t launch_tile_codes(const uint8_t* codes, const uint16_t* meta, int64_t n, int64_t k, int bits,
                             uint8_t* tcodes, uint16_t* tmeta, hipStream_t s) {
  const int kch = tile_chunk_k(bits);
  if (kch == 0 || k % kch != 0 || n % 16 != 0) return hipErrorInvalidValue;
  const int64_t items = (n / 16) * (k / kch) * 64;
  if (items == 0) return hipSuccess;
  const dim3 grid((unsigned)((items + 255) / 256)), block(256);
  if (bits == 4) SS_LAUNCH(tile_codes_kernel<4>, grid, block, 0, s, codes, meta, n, k, tcodes, tmeta);
  else SS_LAUNCH(tile_codes_kernel<2>, grid, block, 0, s, codes, meta, n, k, tcodes, tmeta);
  return hipGetLastError();
}
