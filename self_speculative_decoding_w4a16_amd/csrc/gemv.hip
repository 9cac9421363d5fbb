// Batch-1 GEMV for the draft step: y = W x with W either bf16 or the 4-bit
// substitute (codes + fp16 {scale, min} per 64-group).  Low-batch decode is
// bound by streaming the weights from memory ("How speculative decoding makes
// LLMs go brrr", Module 2), so the kernel is built around HBM bandwidth:
//
//  * x lives in LDS for the whole block.  For W4 it is stored as bf16 pairs
//    (x[k], x[k+4]) in the order the nibble extraction produces, and laid out
//    so that the 64 lanes of a wave read consecutive 16-byte slots (no bank
//    conflicts).  An RMSNorm (and, for layer 0, the embedding gather) is
//    computed in the prologue of every block, so it costs no extra launch.
//  * Every lane streams 16-byte chunks of R rows (R = 1, 2, 4); a wave covers
//    whole rows, lane c takes chunks c, c+64, ...  Rows are contiguous, so
//    each wave load reads R fully used, contiguous 1 KiB segments, for bf16
//    rows (8 weights a chunk) and W4 code rows (32 weights a chunk) alike.
//    A wave's steps alternate between two register slots, so one step's
//    loads are in flight for the whole time the other is consumed.
//  * W4 dequantisation happens in registers: a nibble pair becomes the bf16
//    pair (128+q_a, 128+q_b) with one and-or, and v_dot2_f32_bf16 multiplies
//    it by the x pair.  Per chunk (32 weights of one 64-group)
//        sum_k (q_k s + m) x_k = s * sum_k (128+q_k) x_k + (m - 128 s) * sum_k x_k
//    so the scale and min are applied once per 32 weights; sum_k x_k comes
//    from LDS.
//  * 2- and 3-bit substitutes (the paper note's low-bit substitute layers)
//    take the same path with 16-byte units of 64 weights (one group): two-bit
//    fields become (128 + q) bf16 pairs with one and-or each, x pairs
//    (x[e], x[e+8]) of every 16-weight word; a 3-bit code is the 2-bit plane
//    plus 4 x a 1-bit plane, whose byte order makes its fields pair the same
//    x, so sum q x = d_lo + 4 d_hi - 640 sum x.
//  * Epilogues: store, residual add (bf16(resid + acc)), SiLU(gate)*up with
//    gate row n and up row F+n in the same wave, and logits with a per-block
//    (max, argmax) partial for the sampler.
#include "common.h"
#include "internal.h"
#include "profile.h"

#include <stdlib.h>

#include <mutex>

namespace {

constexpr int kThreads = 256;  // block size; 1024 for long inputs (see launch_one)

// (128 + q_a, 128 + q_b) bf16 pair of nibbles a, a+4 of a code word, dotted
// with the matching x pair.  `mask` (0x000F000F) sits in an SGPR and `magic`
// (0x43004300) in a VGPR so that each extraction is a single v_and_or_b32.
__device__ __forceinline__ float w4_word_dot(uint32_t cw, u32x4 xq, float d, uint32_t mask,
                                             uint32_t magic) {
  d = ss::dot2((cw & mask) | magic, xq.x, d);
  d = ss::dot2(((cw >> 4) & mask) | magic, xq.y, d);
  d = ss::dot2(((cw >> 8) & mask) | magic, xq.z, d);
  d = ss::dot2(((cw >> 12) & mask) | magic, xq.w, d);
  return d;
}

// 2-bit word: fields e and e+8 (bits 2e, 16+2e) of a 16-weight word, dotted
// with x pairs (x[e], x[e+8]) held in two slots (e < 4, e >= 4).
__device__ __forceinline__ float w2_word_dot(uint32_t cw, u32x4 xa, u32x4 xb, float d, uint32_t mask,
                                             uint32_t magic) {
  d = ss::dot2((cw & mask) | magic, xa.x, d);
  d = ss::dot2(((cw >> 2) & mask) | magic, xa.y, d);
  d = ss::dot2(((cw >> 4) & mask) | magic, xa.z, d);
  d = ss::dot2(((cw >> 6) & mask) | magic, xa.w, d);
  d = ss::dot2(((cw >> 8) & mask) | magic, xb.x, d);
  d = ss::dot2(((cw >> 10) & mask) | magic, xb.y, d);
  d = ss::dot2(((cw >> 12) & mask) | magic, xb.z, d);
  d = ss::dot2(((cw >> 14) & mask) | magic, xb.w, d);
  return d;
}

// 1-bit word (the third bit of 3-bit codes) of 32 weights: its bytes hold
// weights 0-7, 16-23, 8-15, 24-31, so fields j and j+16 (j < 8) are weights
// j and j+8 of the first 16-weight word and fields 8+j, 24+j those of the
// second: the pairs of the 2-bit plane's slots xs[0..3].
__device__ __forceinline__ float w1_word_dot(uint32_t hw, const u32x4* xs, float d, uint32_t mask,
                                             uint32_t magic) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    d = ss::dot2(((hw >> (4 * j)) & mask) | magic, xs[j].x, d);
    d = ss::dot2(((hw >> (4 * j + 1)) & mask) | magic, xs[j].y, d);
    d = ss::dot2(((hw >> (4 * j + 2)) & mask) | magic, xs[j].z, d);
    d = ss::dot2(((hw >> (4 * j + 3)) & mask) | magic, xs[j].w, d);
  }
  return d;
}

__device__ __forceinline__ float bf16_chunk_dot(u32x4 w, u32x4 xq, float d) {
  d = ss::dot2(w.x, xq.x, d);
  d = ss::dot2(w.y, xq.y, d);
  d = ss::dot2(w.z, xq.z, d);
  d = ss::dot2(w.w, xq.w, d);
  return d;
}

// Weight widths: WB = 16 (bf16), 4, 3 or 2 bits.  Quantised units are 16
// bytes of codes: 32 weights at 4 bits, 64 (one group) at 2 and 3 bits.
template <int WB>
__host__ __device__ constexpr int unit_weights() {
  return WB == 16 ? 8 : (WB == 4 ? 32 : 64);
}
// 16-byte LDS slots of x per unit: 4 (4-bit: pairs (x[k], x[k+4]) of each
// 8-weight word), 8 (2- and 3-bit: pairs (x[e], x[e+8]) of each 16-weight
// word; the 3-bit third-bit plane reads the same slots).
template <int WB>
__host__ __device__ constexpr int slots_per_unit() {
  return WB == 4 ? 4 : 8;
}
// Slot w of unit c: lanes of a wave reading the same slot of consecutive
// units hit consecutive 16-byte slots (no bank conflicts).
template <int WB>
__host__ __device__ __forceinline__ int xslot(int c, int w) {
  return ((c >> 6) * 64 * slots_per_unit<WB>()) + (w << 6) + (c & 63);
}
template <int WB>
__host__ __device__ __forceinline__ int xslots(int K) {
  return ((K / unit_weights<WB>() + 63) / 64) * 64 * slots_per_unit<WB>();
}
// Bytes of one row of codes (the 3-bit third-bit plane follows the 2-bit
// plane of the row, at byte K/4).
template <int WB>
__host__ __device__ __forceinline__ int code_row_bytes(int K) {
  return WB == 4 ? K / 2 : (WB == 2 ? K / 4 : 3 * K / 8);
}

// Physical rows of row group g (R rows; in SiLU mode R/2 gate rows + the
// matching R/2 up rows).  Rows past the end are clamped to row 0 (always a
// valid address) and flagged invalid.
template <int R, int EPI>
__device__ __forceinline__ void group_rows(int64_t g, int64_t n, int64_t (&prow)[R], bool (&rv)[R],
                                           int64_t& out0) {
  constexpr int RO = (EPI == EPI_SILU) ? R / 2 : R;
  out0 = g * RO;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (EPI == EPI_SILU) {
      const int64_t o = out0 + (r % RO);
      rv[r] = o < n;
      prow[r] = rv[r] ? ((r < RO) ? o : n + o) : 0;
    } else {
      prow[r] = out0 + r;
      rv[r] = prow[r] < n;
      if (!rv[r]) prow[r] = 0;
    }
  }
}

// Weight rows are read through buffer resources: a row's resource covers
// exactly its bytes (none for rows past the end and for steps past the
// wave's last group), so chunks outside it read as zeros without touching
// memory and every step issues the same loads (no branch around them, which
// would make the compiler wait for all loads in flight where the paths meet).
typedef __amdgpu_buffer_rsrc_t Res;
constexpr int kBufferWord3 = 0x00020000;  // buffer resource word 3 (CDNA): raw 32-bit data
constexpr int kNonTemporal = 2;           // buffer load cache policy: nt (streamed weights)

// One step: unit u of row r is the 16-byte chunk (base + lane + 64u) of the
// row; for W4 also the fp16 {scale, min} of its 64-group.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <int R, int U, int WB>
struct Step {
  u32x4 v[U][R];
  uint32_t m[U][R];
  u32x2 h[U][R];  // 3-bit: the unit's 8 bytes of the third-bit plane
};

template <int R, int U, int WB>
__device__ __forceinline__ void load_step(Step<R, U, WB>& b, const Res (&wr)[R], const Res (&mr)[R], int base,
                                          int lane, int hoff) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = base + lane + u * SS_WAVE;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      b.v[u][r] = __builtin_amdgcn_raw_buffer_load_b128(wr[r], 16 * i, 0, kNonTemporal);
      if (WB != 16) b.m[u][r] = __builtin_amdgcn_raw_buffer_load_b32(mr[r], 4 * (WB == 4 ? i >> 1 : i), 0, 0);
      if (WB == 3) b.h[u][r] = __builtin_amdgcn_raw_buffer_load_b64(wr[r], hoff + 8 * i, 0, kNonTemporal);
    }
  }
}

template <int R, int WB>
__device__ __forceinline__ void row_res(const GemvArgs& a, const int64_t (&prow)[R], const bool (&live)[R], int K,
                                        Res (&wr)[R], Res (&mr)[R]) {
  constexpr bool W4 = WB != 16;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (W4) {
      const int rb = code_row_bytes<WB>(K);
      wr[r] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.codes) + prow[r] * rb, 0,
                                                live[r] ? rb : 0, kBufferWord3);
      mr[r] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.meta) + prow[r] * (K / 32), 0,
                                                live[r] ? K / 16 : 0, kBufferWord3);
    } else {
      wr[r] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.w) + prow[r] * K, 0, live[r] ? 2 * K : 0,
                                                kBufferWord3);
      mr[r] = wr[r];
    }
  }
}

// Position of a wave in its walk over (row group, step): group g, first unit
// `base` of the step, the group's physical rows, validity, first output row,
// weight and meta resources and (residual epilogue) residual inputs.
template <int R>
struct Cursor {
  int64_t g, out0;
  int base;
  int64_t prow[R];
  bool rv[R];
  Res wr[R], mr[R];
  float rres[R];
};

template <int R, int WB, int EPI>
__device__ __forceinline__ void cursor_at(Cursor<R>& c, const GemvArgs& a, int64_t g, int64_t n_groups, int K) {
  c.g = g;
  c.base = 0;
  group_rows<R, EPI>(g < n_groups ? g : 0, a.n, c.prow, c.rv, c.out0);
  // past the wave's last group no row is valid: such steps read zeros and
  // store nothing
#pragma unroll
  for (int r = 0; r < R; ++r) c.rv[r] = c.rv[r] && g < n_groups;
  row_res<R, WB>(a, c.prow, c.rv, K, c.wr, c.mr);
}

// Residual inputs of the cursor's rows, loaded (through the vector memory
// path, in order with the weights) for every step, so that no load depends on
// a branch.
template <int R, int EPI>
__device__ __forceinline__ void load_rres(Cursor<R>& c, Res rr) {
#pragma unroll
  for (int r = 0; r < R; ++r)
    c.rres[r] = (EPI == EPI_RESID)
                    ? ss::bf2f(__builtin_amdgcn_raw_buffer_load_b16(rr, 2 * (int)c.prow[r], 0, 0))
                    : 0.0f;
}

// The step after c: the next unit block of the same group, else the first of
// the wave's next group.
template <int R, int U, int WB, int EPI>
__device__ __forceinline__ Cursor<R> cursor_next(const Cursor<R>& c, const GemvArgs& a, Res rr,
                                                 int64_t wave_stride, int64_t n_groups, int K, int n_units) {
  Cursor<R> d;
  d.g = c.g;
  d.out0 = c.out0;
  d.base = c.base + U * SS_WAVE;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    d.prow[r] = c.prow[r];
    d.rv[r] = c.rv[r];
    d.wr[r] = c.wr[r];
    d.mr[r] = c.mr[r];
  }
  if (d.base >= n_units) cursor_at<R, WB, EPI>(d, a, c.g + wave_stride, n_groups, K);
  load_rres<R, EPI>(d, rr);
  return d;
}

// Sums each of a wave's R per-lane row accumulators over the 64 lanes in one
// butterfly: at xor 32 (and 16 for R = 4) the lanes trade half of their rows,
// so R rows cost 6 + log2(R) lane swaps instead of 6 R.  Row r's total ends in
// lanes [64 r / R, 64 (r + 1) / R).  Partners are added in the same xor order
// as ss::wave_sum, so the sums are bit-identical to it.
template <int R>
__device__ __forceinline__ float reduce_rows(const float (&acc)[R], int lane) {
  if constexpr (R == 4) {
    const bool hi = lane & 32;
    const float k0 = (hi ? acc[2] : acc[0]) + __shfl_xor(hi ? acc[0] : acc[2], 32, SS_WAVE);
    const float k1 = (hi ? acc[3] : acc[1]) + __shfl_xor(hi ? acc[1] : acc[3], 32, SS_WAVE);
    const bool h16 = lane & 16;
    float v = (h16 ? k1 : k0) + __shfl_xor(h16 ? k0 : k1, 16, SS_WAVE);
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) v += __shfl_xor(v, o, SS_WAVE);
    return v;
  } else if constexpr (R == 2) {
    const bool hi = lane & 32;
    float v = (hi ? acc[1] : acc[0]) + __shfl_xor(hi ? acc[0] : acc[1], 32, SS_WAVE);
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) v += __shfl_xor(v, o, SS_WAVE);
    return v;
  } else {
    return ss::wave_sum(acc[0]);
  }
}

// Stores item `it` (x[8it .. 8it+7], bf16) into LDS: as consecutive pairs
// for bf16 weights; for 4-bit as the pairs (x0,x4),(x1,x5),(x2,x6),(x3,x7)
// in slot xslot(it/4, it%4); for 2- and 3-bit as the pairs of the unit's
// slots (the partner item's values from the neighbouring lane); plus the sum of the
// unit's values, reduced over the lanes that hold the unit.  Every lane of
// the wave calls it (the lane exchanges need all of them).
template <int WB>
__device__ __forceinline__ void put_x(u32x4* smem4, float* xsum, int it, bool ok, const uint16_t (&xb)[8]) {
  if (WB == 16) {
    if (ok)
      smem4[it] = u32x4{ss::pack_bf(xb[0], xb[1]), ss::pack_bf(xb[2], xb[3]), ss::pack_bf(xb[4], xb[5]),
                        ss::pack_bf(xb[6], xb[7])};
    return;
  }
  float xs = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) xs += ss::bf2f(xb[i]);
  xs += __shfl_xor(xs, 1, SS_WAVE);
  xs += __shfl_xor(xs, 2, SS_WAVE);
  if (WB == 4) {
    if (ok) {
      smem4[xslot<4>(it >> 2, it & 3)] = u32x4{ss::pack_bf(xb[0], xb[4]), ss::pack_bf(xb[1], xb[5]),
                                               ss::pack_bf(xb[2], xb[6]), ss::pack_bf(xb[3], xb[7])};
      if ((it & 3) == 0) xsum[it >> 2] = xs;
    }
    return;
  }
  xs += __shfl_xor(xs, 4, SS_WAVE);
  // 2-bit plane: item 2w holds x[16w .. +7], item 2w+1 x[16w+8 .. +15] of the
  // unit; slot 2w takes pairs e = 0..3 (written by the even item), slot
  // 2w+1 pairs e = 4..7 (the odd item)
  const uint32_t w0 = ss::pack_bf(xb[0], xb[1]), w1 = ss::pack_bf(xb[2], xb[3]);
  const uint32_t w2 = ss::pack_bf(xb[4], xb[5]), w3 = ss::pack_bf(xb[6], xb[7]);
  uint16_t p[8];
  {
    const uint32_t q0 = __shfl_xor(w0, 1, SS_WAVE), q1 = __shfl_xor(w1, 1, SS_WAVE);
    const uint32_t q2 = __shfl_xor(w2, 1, SS_WAVE), q3 = __shfl_xor(w3, 1, SS_WAVE);
    p[0] = (uint16_t)q0; p[1] = (uint16_t)(q0 >> 16); p[2] = (uint16_t)q1; p[3] = (uint16_t)(q1 >> 16);
    p[4] = (uint16_t)q2; p[5] = (uint16_t)(q2 >> 16); p[6] = (uint16_t)q3; p[7] = (uint16_t)(q3 >> 16);
  }
  const int c = it >> 3, a = it & 7;
  if (ok) {
    const bool odd = a & 1;
    u32x4 v;
    if (!odd) v = u32x4{ss::pack_bf(xb[0], p[0]), ss::pack_bf(xb[1], p[1]), ss::pack_bf(xb[2], p[2]),
                        ss::pack_bf(xb[3], p[3])};
    else v = u32x4{ss::pack_bf(p[4], xb[4]), ss::pack_bf(p[5], xb[5]), ss::pack_bf(p[6], xb[6]),
                   ss::pack_bf(p[7], xb[7])};
    smem4[xslot<WB>(c, a)] = v;
    if (a == 0) xsum[c] = xs;
  }
}

// Consumes one step: its dot products into the per-lane accumulators and, on
// the group's last step, the row sums and the epilogue.
template <int R, int U, int WB, int EPI>
__device__ __forceinline__ void consume(const GemvArgs& a, const Cursor<R>& c, const Step<R, U, WB>& cur,
                                        float (&acc)[R], ss::ArgMax& best, const u32x4* smem4,
                                        const float* xsum, int lane, int n_units, uint32_t mask,
                                        uint32_t magic, uint32_t mask2, uint32_t mask1) {
  constexpr int RO = (EPI == EPI_SILU) ? R / 2 : R;
  // compute the current step
#pragma unroll
  for (int u = 0; u < U; ++u) {
    // chunks past the row end (zeros) are computed on x of chunk 0 and their
    // result dropped: no branch, so no wait is placed where paths meet
    const int i0 = c.base + lane + u * SS_WAVE;
    const bool ok = i0 < n_units;
    const int i = ok ? i0 : 0;
    if (WB == 2 || WB == 3) {
      const float xs = xsum[i];
      u32x4 xl[8];
#pragma unroll
      for (int w = 0; w < 8; ++w) xl[w] = smem4[xslot<WB>(i, w)];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const u32x4 cw = cur.v[u][r];
        float d0 = w2_word_dot(cw.x, xl[0], xl[1], 0.0f, mask2, magic);
        float d1 = w2_word_dot(cw.y, xl[2], xl[3], 0.0f, mask2, magic);
        d0 = w2_word_dot(cw.z, xl[4], xl[5], d0, mask2, magic);
        d1 = w2_word_dot(cw.w, xl[6], xl[7], d1, mask2, magic);
        const float sc = ss::h2f((uint16_t)(cur.m[u][r] & 0xffffu));
        const float mn = ss::h2f((uint16_t)(cur.m[u][r] >> 16));
        float t;
        if (WB == 3) {
          float e0 = w1_word_dot(cur.h[u][r].x, xl, 0.0f, mask1, magic);
          float e1 = w1_word_dot(cur.h[u][r].y, xl + 4, 0.0f, mask1, magic);
          t = sc * ((d0 + d1) + 4.0f * (e0 + e1)) + (mn - 640.0f * sc) * xs;
        } else {
          t = sc * (d0 + d1) + (mn - 128.0f * sc) * xs;
        }
        acc[r] += ok ? t : 0.0f;
      }
    } else if (WB == 4) {
      const float xs = xsum[i];
      const u32x4 x0 = smem4[xslot<4>(i, 0)], x1 = smem4[xslot<4>(i, 1)];
      const u32x4 x2 = smem4[xslot<4>(i, 2)], x3 = smem4[xslot<4>(i, 3)];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const u32x4 cw = cur.v[u][r];
        float d0 = w4_word_dot(cw.x, x0, 0.0f, mask, magic);
        float d1 = w4_word_dot(cw.y, x1, 0.0f, mask, magic);
        d0 = w4_word_dot(cw.z, x2, d0, mask, magic);
        d1 = w4_word_dot(cw.w, x3, d1, mask, magic);
        const float sc = ss::h2f((uint16_t)(cur.m[u][r] & 0xffffu));
        const float mn = ss::h2f((uint16_t)(cur.m[u][r] >> 16));
        const float t = sc * (d0 + d1) + (mn - 128.0f * sc) * xs;
        acc[r] += ok ? t : 0.0f;
      }
    } else {
      const u32x4 xq = smem4[i];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float t = bf16_chunk_dot(cur.v[u][r], xq, acc[r]);
        acc[r] = ok ? t : acc[r];
      }
    }
  }

  if (c.base + U * SS_WAVE >= n_units) {  // last step of the group
    constexpr int LPR = SS_WAVE / R;  // lanes per row after the butterfly
    const float tot = reduce_rows<R>(acc, lane);
    if (EPI == EPI_SILU) {
      const float up_tot = __shfl_xor(tot, 32, SS_WAVE);  // up row r + R/2 sits 32 lanes away
#pragma unroll
      for (int r = 0; r < RO; ++r) {
        if (lane == LPR * r && c.rv[r]) {
          const float gt = ss::bf2f(ss::f2bf(tot));
          const float up = ss::bf2f(ss::f2bf(up_tot));
          a.y[c.out0 + r] = ss::f2bf(gt / (1.0f + expf(-gt)) * up);
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (lane == LPR * r && c.rv[r]) {
          float v = tot;
          if (EPI == EPI_RESID) v = c.rres[r] + v;
          const uint16_t b = ss::f2bf(v);
          a.y[c.prow[r]] = b;
          if (EPI == EPI_LOGITS) best = ss::better(best, ss::cand(ss::bf2f(b), (int)c.prow[r]));
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0f;
  }
}

template <int R, int WB, int PRO, int EPI, int NT>
__global__ __launch_bounds__(NT) void gemv_kernel(GemvArgs a, int64_t n_groups, uint32_t mask_arg,
                                                        uint32_t magic_arg, uint32_t mask2_arg, uint32_t mask1_arg) {
  constexpr bool W4 = WB != 16;  // quantised weights (4, 3 or 2 bits)
  extern __shared__ u32x4 smem4[];
  constexpr int kWaves = NT / SS_WAVE;
  __shared__ float red[kWaves];
  __shared__ float red_v[kWaves];
  __shared__ int red_i[kWaves];

  // the draft step's position flag: read first, tested after this wave's
  // first loads are issued (so its latency overlaps theirs; nothing is
  // stored before the test)
  const int vflag = a.valid ? *a.valid : 1;
  const int tid = threadIdx.x, lane = tid & (SS_WAVE - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / SS_WAVE);  // wave-uniform: rows in SGPRs
  const int K = (int)a.k;
  const int n_units = K / unit_weights<WB>();  // 16-byte chunks of codes per row
  // 16-byte chunks per lane and row in one step: W4 chunks carry 4x the VALU
  // work of bf16 chunks, so W4 steps are shorter (better overlap); 2/3-bit
  // units hold a whole group (twice the weights of a 4-bit unit)
  constexpr int U = WB == 16 ? ((R >= 4) ? 2 : (R == 2 ? 4 : 8)) : (WB == 4 ? ((R >= 4) ? 1 : 2) : 1);
  const int hoff = K / 4;  // 3-bit: byte offset of the third-bit plane in a row
  const uint32_t mask2 = __builtin_amdgcn_readfirstlane(mask2_arg);  // 0x00030003: 2-bit fields
  const uint32_t mask1 = __builtin_amdgcn_readfirstlane(mask1_arg);  // 0x00010001: 1-bit fields
  const int64_t wave_stride = (int64_t)gridDim.x * kWaves;
  const uint32_t mask = __builtin_amdgcn_readfirstlane(mask_arg);
  uint32_t magic = magic_arg;
  asm volatile("" : "+v"(magic));

  // ------------------------------------------------ prologue inputs and first weights
  // Loads complete in issue order.  A plain input x is issued before the
  // first weights, so waiting for it does not wait for the weight burst of
  // every wave at once; with the norm prologue (h and the norm weights,
  // L2-resident) issuing the weights first measured faster.  Indices are
  // clamped (every load issued), out-of-range items masked at use.
  const uint16_t* src = a.x;
  if (PRO == PRO_NORM) src = a.h;
  if (PRO == PRO_EMBED_NORM) src = a.embed + (int64_t)min(max(*a.token, 0), a.vocab - 1) * K;
  const u32x4* src4 = reinterpret_cast<const u32x4*>(src);
  const u32x4* g4 = reinterpret_cast<const u32x4*>(a.norm_w);
  float* xsum = reinterpret_cast<float*>(smem4 + (W4 ? xslots<WB>(K) : K / 8));
  // items: 8 consecutive values of x (one 16-byte quad); for W4 the four
  // items of a 32-value chunk sit in four consecutive lanes
  constexpr int NI = (3 * kThreads + NT - 1) / NT;  // items per thread held when normalising
  constexpr int XB = (PRO == PRO_X) ? 4 : NI;        // items per thread loaded up front
  const int n_items = K / 8;
  u32x4 hv[XB], gv[XB];
  auto load_prologue = [&]() {
#pragma unroll
    for (int t = 0; t < XB; ++t) {
      const int it = min(tid + t * NT, n_items - 1);
      hv[t] = src4[it];
      if (PRO != PRO_X) gv[t] = g4[it];
    }
  };
  if (PRO == PRO_X) load_prologue();

  // Two step slots, A and B, alternate without register copies (a copy of a
  // slot whose loads are in flight would wait for them): while one is
  // consumed the other's loads are in flight.  The wave's step count T is
  // known up front, so the loop runs only while both refills are real steps
  // and the last one or two steps are consumed after it; no load is issued
  // for a step past the end, and none sits behind a branch inside the loop.
  const int64_t g0 = (int64_t)blockIdx.x * kWaves + wave;
  const int spg = (n_units + U * SS_WAVE - 1) / (U * SS_WAVE);  // steps per group
  const int64_t T = g0 < n_groups ? ((n_groups - 1 - g0) / wave_stride + 1) * spg : 0;
  const Res rr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(EPI == EPI_RESID ? a.resid : a.y), 0,
                                                    EPI == EPI_RESID ? (int)(2 * a.n) : 0, kBufferWord3);
  Cursor<R> ca, cb;
  Step<R, U, WB> sa, sb;
  cursor_at<R, WB, EPI>(ca, a, g0, n_groups, K);
  load_rres<R, EPI>(ca, rr);
  load_step<R, U, WB>(sa, ca.wr, ca.mr, 0, lane, hoff);
  if (PRO != PRO_X) {
    load_prologue();
  } else {
    // keep the prologue's arithmetic (and its wait) after the weight loads
    __builtin_amdgcn_sched_barrier(0);
  }
  if (vflag == 0) return;  // block-uniform: the whole launch is skipped

  // ------------------------------------------------ prologue: x (and group sums) in LDS
  if (PRO != PRO_X) {
    float ss = 0.0f;
#pragma unroll
    for (int t = 0; t < NI; ++t) {
      const bool ok = tid + t * NT < n_items;
      const uint32_t wv[4] = {hv[t].x, hv[t].y, hv[t].z, hv[t].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = ok ? ss::lo_bf(wv[i]) : 0.0f, hi = ok ? ss::hi_bf(wv[i]) : 0.0f;
        ss += lo * lo;
        ss += hi * hi;
      }
    }
    ss = ss::wave_sum(ss);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    float tot = 0.0f;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) tot += red[i];
    const float inv = 1.0f / sqrtf(tot / (float)K + a.eps);
    if (PRO == PRO_EMBED_NORM && blockIdx.x == 0) {
      for (int q = tid; q < n_items; q += NT) reinterpret_cast<u32x4*>(a.h_out)[q] = src4[q];
    }
#pragma unroll
    for (int t = 0; t < NI; ++t) {
      const int it = tid + t * NT;
      if (t * NT >= n_items) break;  // block-uniform
      const bool ok = it < n_items;
      const uint32_t wv[4] = {hv[t].x, hv[t].y, hv[t].z, hv[t].w};
      const uint32_t gw[4] = {gv[t].x, gv[t].y, gv[t].z, gv[t].w};
      uint16_t xb[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xb[2 * i] = ss::f2bf(ss::lo_bf(wv[i]) * inv * ss::lo_bf(gw[i]));
        xb[2 * i + 1] = ss::f2bf(ss::hi_bf(wv[i]) * inv * ss::hi_bf(gw[i]));
      }
      put_x<WB>(smem4, xsum, it, ok, xb);
    }
  } else {
    // the first XB items per thread are the ones loaded up front (all of x up
    // to 8 XB NT values); any further batch is loaded here
    for (int b0 = 0; b0 < n_items; b0 += XB * NT) {  // block-uniform trip count
      if (b0 > 0) {
#pragma unroll
        for (int t = 0; t < XB; ++t) hv[t] = src4[min(b0 + t * NT + tid, n_items - 1)];
      }
#pragma unroll
      for (int t = 0; t < XB; ++t) {
        if (b0 + t * NT >= n_items) break;  // block-uniform
        const int it = b0 + t * NT + tid;
        const uint32_t wv[4] = {hv[t].x, hv[t].y, hv[t].z, hv[t].w};
        uint16_t xb[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xb[2 * i] = (uint16_t)(wv[i] & 0xffffu);
          xb[2 * i + 1] = (uint16_t)(wv[i] >> 16);
        }
        put_x<WB>(smem4, xsum, it, it < n_items, xb);
      }
    }
  }
  // Prologue registers whose items lie past the end of x were never read; a
  // use of every one here settles their loads before the loop, where the
  // compiler would otherwise wait for all loads in flight (each step's
  // included) before it reuses those registers.
#pragma unroll
  for (int t = 0; t < XB; ++t) {
    asm volatile("" ::"v"(hv[t]));
    if (PRO != PRO_X) asm volatile("" ::"v"(gv[t]));
  }
  __syncthreads();

  // ------------------------------------------------ main loop over (row group, step)
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;
  ss::ArgMax best = {-INFINITY, ss::kNoIndex};
  // steps t (in A) and t+1 (in B) per iteration, refilling B with t+1 and A
  // with t+2 (both < T)
  int64_t t = 0;
  while (t + 2 < T) {
    cb = cursor_next<R, U, WB, EPI>(ca, a, rr, wave_stride, n_groups, K, n_units);
    load_step<R, U, WB>(sb, cb.wr, cb.mr, cb.base, lane, hoff);
    consume<R, U, WB, EPI>(a, ca, sa, acc, best, smem4, xsum, lane, n_units, mask, magic, mask2, mask1);
    ca = cursor_next<R, U, WB, EPI>(cb, a, rr, wave_stride, n_groups, K, n_units);
    load_step<R, U, WB>(sa, ca.wr, ca.mr, ca.base, lane, hoff);
    consume<R, U, WB, EPI>(a, cb, sb, acc, best, smem4, xsum, lane, n_units, mask, magic, mask2, mask1);
    t += 2;
  }
  if (t + 2 == T) {  // steps T-2 (in A) and T-1
    cb = cursor_next<R, U, WB, EPI>(ca, a, rr, wave_stride, n_groups, K, n_units);
    load_step<R, U, WB>(sb, cb.wr, cb.mr, cb.base, lane, hoff);
    consume<R, U, WB, EPI>(a, ca, sa, acc, best, smem4, xsum, lane, n_units, mask, magic, mask2, mask1);
    consume<R, U, WB, EPI>(a, cb, sb, acc, best, smem4, xsum, lane, n_units, mask, magic, mask2, mask1);
  } else if (t + 1 == T) {  // step T-1 (in A)
    consume<R, U, WB, EPI>(a, ca, sa, acc, best, smem4, xsum, lane, n_units, mask, magic, mask2, mask1);
  }
  if (EPI == EPI_LOGITS) {
    best = ss::wave_argmax(best);
    if (lane == 0) {
      red_v[wave] = best.v;
      red_i[wave] = best.i;
    }
    __syncthreads();
    if (tid == 0) {
      ss::ArgMax b = {red_v[0], red_i[0]};
      for (int i = 1; i < kWaves; ++i) b = ss::better(b, ss::ArgMax{red_v[i], red_i[i]});
      a.part_max[blockIdx.x] = b.v;
      a.part_arg[blockIdx.x] = b.i;
    }
  }
}

int device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
  }
  return cus;
}

// Resident blocks per compute unit of one kernel at one LDS size, from the
// runtime's occupancy calculator (register and LDS limits), cached.
struct Occupancy {
  std::mutex mu;
  size_t lds[8];
  int fit[8];
  int n = 0;
  int get(const void* fn, int threads, size_t l) {
    std::lock_guard<std::mutex> g(mu);
    for (int i = 0; i < n; ++i)
      if (lds[i] == l) return fit[i];
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, threads, l) != hipSuccess || nb < 1) nb = 1;
    if (n < 8) {
      lds[n] = l;
      fit[n] = nb;
      ++n;
    }
    return nb;
  }
};

// Blocks of a persistent launch: a few per compute unit, no more than fit on
// a compute unit at once (so the grid runs in one round), fewer when the
// matrix has fewer row groups.  `site_per_cu` (> 0) overrides the default
// for a site measured faster with another count.
int64_t gemv_blocks(int64_t n_groups, bool w4, int fit, int threads, int site_per_cu = 0) {
  const int waves = threads / SS_WAVE;
  int want = threads == kThreads ? 4 * (w4 ? 1 : 2) : 1;
  if (threads == kThreads && site_per_cu > 0) want = site_per_cu;
  if (fit > 0 && want > fit) want = fit;
  const int64_t cap = (int64_t)device_cus() * want;
  const int64_t need = (n_groups + waves - 1) / waves;
  return need < cap ? need : cap;
}

template <int WB>
size_t gemv_lds(int64_t k) {
  return WB != 16 ? (size_t)xslots<WB>((int)k) * 16 + (size_t)(k / unit_weights<WB>()) * 4 : (size_t)k * 2;
}

template <int R, int WB, int PRO, int EPI, int NT>
hipError_t launch_nt(const GemvArgs& a, hipStream_t s, int* blocks_out) {
  constexpr bool W4 = WB != 16;
  constexpr int RO = (EPI == EPI_SILU) ? R / 2 : R;
  static Occupancy occ;
  const int64_t n_groups = (a.n + RO - 1) / RO;
  const size_t lds = gemv_lds<WB>(a.k);
  const int fit = occ.get(reinterpret_cast<const void*>(&gemv_kernel<R, WB, PRO, EPI, NT>), NT, lds);
  // the narrow QKV and O projections (n <= 8192) of bf16 layers, and the W4
  // QKV projection, run faster with two blocks per compute unit than with
  // the default 8 (bf16) or 4 (W4): at the 7B shape bf16 QKV 8.2 against
  // 8.6 us, bf16 O 6.3 against 6.7, W4 QKV 5.9 against 6.2 (W4 O is best
  // with 4)
  const bool narrow = (EPI == EPI_STORE || EPI == EPI_RESID) && a.n <= 8192 && (!W4 || EPI == EPI_STORE);
  const int64_t blocks = gemv_blocks(n_groups, W4, fit, NT, narrow ? 2 : 0);
  if (blocks_out) *blocks_out = (int)blocks;
  SS_LAUNCH((gemv_kernel<R, WB, PRO, EPI, NT>), dim3((unsigned)blocks), dim3(NT), lds, s, a, n_groups,
            0x000F000Fu, 0x43004300u, 0x00030003u, 0x00010001u);
  return hipGetLastError();
}

// Long inputs (the down projection) use 1024-thread blocks, one per compute
// unit: x is staged in LDS once per 16 waves instead of once per 4.
constexpr int64_t kLongK = 8192;

template <int R, int WB, int PRO, int EPI>
hipError_t launch_one(const GemvArgs& a, hipStream_t s, int* blocks_out) {
  if constexpr (PRO == PRO_X && EPI != EPI_LOGITS) {
    if (a.k > kLongK) return launch_nt<R, WB, PRO, EPI, 1024>(a, s, blocks_out);
  }
  return launch_nt<R, WB, PRO, EPI, kThreads>(a, s, blocks_out);
}

template <int WB, int PRO, int EPI>
hipError_t launch_r(int R, const GemvArgs& a, hipStream_t s, int* b) {
  if constexpr (EPI == EPI_SILU) {
    (void)R;  // always one gate and one up row per wave
    return launch_one<2, WB, PRO, EPI>(a, s, b);
  } else {
    if (R >= 4) return launch_one<4, WB, PRO, EPI>(a, s, b);
    if (R == 2) return launch_one<2, WB, PRO, EPI>(a, s, b);
    return launch_one<1, WB, PRO, EPI>(a, s, b);
  }
}

template <int WB>
hipError_t launch_w(int R, int pro, int epi, const GemvArgs& a, hipStream_t s, int* b) {
  if (pro == PRO_X && epi == EPI_STORE) return launch_r<WB, PRO_X, EPI_STORE>(R, a, s, b);
  if (pro == PRO_X && epi == EPI_RESID) return launch_r<WB, PRO_X, EPI_RESID>(R, a, s, b);
  if (pro == PRO_NORM && epi == EPI_STORE) return launch_r<WB, PRO_NORM, EPI_STORE>(R, a, s, b);
  if (pro == PRO_EMBED_NORM && epi == EPI_STORE) return launch_r<WB, PRO_EMBED_NORM, EPI_STORE>(R, a, s, b);
  if (pro == PRO_NORM && epi == EPI_SILU) return launch_r<WB, PRO_NORM, EPI_SILU>(R, a, s, b);
  if constexpr (WB == 16 || WB == 4) {
    if (pro == PRO_NORM && epi == EPI_LOGITS) return launch_r<WB, PRO_NORM, EPI_LOGITS>(R, a, s, b);
  }
  return hipErrorInvalidValue;
}

}  // namespace

// Rows per wave: enough blocks to fill 256 CUs several times over, and as
// many rows per lane as that allows (more bytes in flight per lane).  The
// gate/up GEMVs take one gate and one up row per wave: at the 7B shape that
// measured faster than two of each (W4: 3 %, bf16: 3 %), as the row groups
// then spread more evenly over the waves of the persistent grid.
static int pick_r(int64_t n, int epi) {
  if (epi == EPI_SILU) return 2;
  if (n >= 16384) return 4;
  if (n >= 4096) return 2;
  return 1;
}

// Upper bound on the blocks of a launch (sizes per-block partial buffers).
int gemv_max_blocks(bool w4, int64_t n, int epi) {
  const int R = pick_r(n, epi);
  const int RO = (epi == EPI_SILU) ? R / 2 : R;
  return (int)gemv_blocks((n + RO - 1) / RO, w4, 0, kThreads);
}

hipError_t launch_gemv(int wb, int pro, int epi, const GemvArgs& a, hipStream_t s, int* blocks_out) {
  if (a.tiled) {
    if ((wb != 4 && wb != 2) || !gemv_w4t_supported(pro, epi)) return hipErrorInvalidValue;
    if (blocks_out) *blocks_out = 0;
    return launch_gemv_w4t(wb, pro, epi, a, s);
  }
  const int R = pick_r(a.n, epi);
  switch (wb) {
    case 16: return launch_w<16>(R, pro, epi, a, s, blocks_out);
    case 4: return launch_w<4>(R, pro, epi, a, s, blocks_out);
    case 3: return launch_w<3>(R, pro, epi, a, s, blocks_out);
    case 2: return launch_w<2>(R, pro, epi, a, s, blocks_out);
  }
  return hipErrorInvalidValue;
}
