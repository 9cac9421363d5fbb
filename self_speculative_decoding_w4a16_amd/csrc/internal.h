// Host-side declarations shared by the translation units of libsubspec.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// ------------------------------------------------------------------ GEMV (batch 1)
// Prologue: where the input vector x comes from.
enum GemvPro { PRO_X = 0, PRO_NORM = 1, PRO_EMBED_NORM = 2 };
// Epilogue: what is written.
enum GemvEpi { EPI_STORE = 0, EPI_RESID = 1, EPI_SILU = 2, EPI_LOGITS = 3 };

struct GemvArgs {
  // weights: bf16 w, or W4 codes + meta
  const uint16_t* w;
  const uint8_t* codes;
  const uint16_t* meta;
  int64_t n;  // output rows (F in EPI_SILU mode: physical rows are 2F)
  int64_t k;
  // prologue inputs
  const uint16_t* x;         // PRO_X
  const uint16_t* h;         // PRO_NORM: residual stream [k]
  const uint16_t* norm_w;    // PRO_NORM / PRO_EMBED_NORM
  float eps;
  const uint16_t* embed;     // PRO_EMBED_NORM: embed table [V][k]
  const int32_t* token;      // PRO_EMBED_NORM: device token id (clamped to [0, vocab))
  int64_t vocab;             // PRO_EMBED_NORM: rows of the embed table
  uint16_t* h_out;           // PRO_EMBED_NORM: block 0 stores the embedded row here
  // epilogue outputs
  uint16_t* y;               // output [n]
  const uint16_t* resid;     // EPI_RESID: y = bf16(resid + acc) (may alias y)
  float* part_max;           // EPI_LOGITS: per-block max
  int32_t* part_arg;         // EPI_LOGITS: per-block argmax
  const int32_t* valid;      // optional device flag: skip everything if *valid == 0
  int tiled;                 // codes + meta in 16-row tiles (subspec_tile_codes)
};

int gemv_max_blocks(bool w4, int64_t n, int epi);  // blocks of one launch (logits partials)
// wb: weight width, 16 (bf16 w), 4, 3 or 2 (codes + meta; see subspec_quantize)
hipError_t launch_gemv(int wb, int pro, int epi, const GemvArgs& a, hipStream_t s, int* blocks_out);
// 4- or 2-bit GEMV on 16-row tiles (a.tiled; matrix cores): prologue/epilogue
// pairs it takes, and the launch (a.n % 16 == 0, a.k a multiple of the
// width's chunk (tile_chunk_k), a.k <= 28672)
bool gemv_w4t_supported(int pro, int epi);
int tile_chunk_k(int bits);  // k per 64-byte row piece of a tile: 128 (4 bits), 256 (2 bits), 0 otherwise
hipError_t launch_gemv_w4t(int wb, int pro, int epi, const GemvArgs& a, hipStream_t s);
// row-major codes + meta -> 16-row tiles (bits 4 or 2; n % 16 == 0, k % tile_chunk_k(bits) == 0)
hipError_t launch_tile_codes(const uint8_t* codes, const uint16_t* meta, int64_t n, int64_t k, int bits,
                             uint8_t* tcodes, uint16_t* tmeta, hipStream_t s);

// ------------------------------------------------------------------ GEMM (verify)
// GEPI_PARTIAL: fp32 partial sums [split][m][n] for the caller to reduce
enum GemmEpi { GEPI_STORE = 0, GEPI_RESID = 1, GEPI_SILU = 2, GEPI_PARTIAL = 3 };
struct GemmArgs {
  const uint16_t* w;  // bf16 [N][K]
  int64_t n;          // output columns (F in GEPI_SILU mode)
  int64_t k;
  const uint16_t* x;  // bf16 [m][K]
  int m;
  uint16_t* y;        // bf16 [m][ldy]
  int64_t ldy;
  const uint16_t* resid;  // GEPI_RESID: [m][ldy]
  float* partials;        // split-k partial sums [splits][m][n] (when splits > 1)
};
// k splits the GEMM of this shape uses (1: the epilogue runs in the kernel).
int gemm_splits(int64_t n, int64_t k, int m, int epi);
size_t gemm_partials_bytes(int64_t n, int64_t k, int m, int epi);
// Launches the GEMM; with more than one split it writes a.partials instead
// of running `epi`, and the caller reduces them (splits in *splits_out).
hipError_t launch_gemm(int epi, const GemmArgs& a, hipStream_t s, int* splits_out);
// y[t][c] = bf16(sum over splits of part[s][t][c]), splits in order.
hipError_t launch_gemm_reduce(const float* part, int splits, int m, int64_t n, uint16_t* y, int64_t ldy,
                              hipStream_t s);

// Skinny GEMM on 4-bit weights (matrix cores): Y[t][n] = bf16(sum_k X[t][k] w[n][k])
// for t < m <= 16; k % 128 == 0; codes + meta row-major, or in 16-row tiles
// (tiled; n % 16 == 0).  With k split over blocks it writes fp32
// partials (gemm_w4_splits x m x n floats at part) and reduces them in order.
// With splits_out set it always writes the partials ([splits][m][n], also
// for one split), reduces nothing and returns the count: the consumer adds
// them (the rows forward's RoPE and residual + RMSNorm kernels).
int gemm_w4_splits(int64_t n, int64_t k);
hipError_t launch_gemm_w4(const uint8_t* codes, const uint16_t* meta, int64_t n, int64_t k, const uint16_t* x, int m,
                          uint16_t* y, float* part, hipStream_t s, int* splits_out, bool tiled);
// The gate/up projection (2F rows: gate rows, then up rows) ending in
// act[t][j] = bf16(SiLU(gate) * up); only while it needs no k split
// (gemm_w4_splits(2F, k) == 1), else hipErrorInvalidValue.
hipError_t launch_gemm_w4_silu(const uint8_t* codes, const uint16_t* meta, int64_t F, int64_t k, const uint16_t* x,
                               int m, uint16_t* act, hipStream_t s, bool tiled);

// ------------------------------------------------------------------ quantise
hipError_t launch_quantize(const uint16_t* w, int64_t n, int64_t k, int bits, uint8_t* codes,
                           uint16_t* meta, hipStream_t s);

// ------------------------------------------------------------------ attention
struct AttnArgs {
  const uint16_t* qkv;  // [m][(Hq+2Hkv) d] raw projections (pre-RoPE)
  const float* qkv_part;  // or, when set: their fp32 partial sums [qkv_splits][m][(Hq+2Hkv) d]
  int qkv_splits;
  uint16_t* q_rot;      // [m][Hq d] rotated queries (bf16)
  uint16_t* k_cache;    // [Hkv][cap][d] of this layer
  uint16_t* v_cache;
  const int32_t* kv_len;
  int pos_offset;       // node of row 0; row j is node t = pos_offset + j * row_stride
  int row_stride;       // 0 or 1: consecutive nodes
  // tree_d = 0: a chain - node t at slot and position kv_len + t, seeing
  // slots [0, kv_len + t].  tree_d = D > 0: the static tree of chains of
  // depth D - node t (t >= 1 in chain (t - 1) / D at depth (t - 1) % D + 1)
  // at slot kv_len + t and position kv_len + depth, seeing slots
  // [0, kv_len] and its own chain's slots up to its own.
  int tree_d;
  int m;                // query rows (of each sequence)
  // seqs > 1: a batch of independent sequences, rows [z m, z m + m) of every
  // per-row buffer belong to sequence z, whose kv_len is kv_len[z] and whose
  // cache heads are z n_kv .. z n_kv + n_kv - 1 of the layer (the cache is
  // [seqs][n_kv][cap][d] per layer); partials [seqs][n_kv][splits][m][G][d + 4]
  int seqs;
  int n_q, n_kv, d, cap;
  float theta;
  const float* rope_cs;  // [m][d/2][2] (cos, sin) of each row's position
  float* part;          // split partials [Hkv][splits][m][G][d + 4]
  int splits;           // grid splits over keys (128 keys each)
  int split_keys;       // verify: keys per split block (0: 128; more: one block walks several 128-key tiles)
  uint16_t* out;        // [m][Hq d]
  float* ml;            // optional [m][Hq][2]: softmax (max, sum) of each row and head
  // sparse draft (draft step only; index == nullptr: dense): keys are
  // index[hk][0 .. *n_index) followed by positions kv_len .. kv_len + pos_offset
  const int32_t* index;  // [Hkv][index_cap] of this layer
  const int32_t* n_index;
  int index_cap;
  int max_keys;  // draft step: bound on the keys of the launch (picks the kernel)
  // draft step, per-head kernel: key splits per query head (1: no partials);
  // with more, the head's partials go to part[hq][split][d + 4] and the last
  // block of the head to arrive (counters[hq], zero between launches) merges
  int head_splits;
  uint32_t* counters;
};
hipError_t launch_rope_append(const AttnArgs& a, hipStream_t s);
// One query position (the draft step): RoPE + KV append + attention into
// out [Hq d] (bf16).  Up to 8192 keys (a.max_keys) a.head_splits blocks per
// query head do it all (the last one to finish merges); beyond, per-split
// partials (m, l, o[d]) in part[kv head][split][group head][d + 4] are merged
// by a second launch.
hipError_t launch_decode_attention(const AttnArgs& a, const int32_t* valid, hipStream_t s);
int decode_attn_keys_per_split();  // verify rows
// Keys per split block of the verify attention for a launch over `cap` keys,
// `n_kv` KV heads and `rows_x_group` = query rows x GQA group.
int verify_attn_split_keys(int cap, int n_kv, int rows_x_group);
int draft_attn_keys_per_split();   // draft step
int draft_head_splits(int max_keys);  // key splits per query head of the per-head kernel
// Chunks of 16 keys per wave the per-head draft attention keeps in flight
// (1-3) for a launch, or 0 if the launch does not take the per-head form.
int draft_head_ring(const AttnArgs& a);
// The draft step's QKV GEMV on 4- or 2-bit tiles (prologue PRO_NORM or
// PRO_EMBED_NORM, store epilogue; a.n = (n_q + 2 n_kv) 128) and the
// per-head draft attention over dense keys (ring dqr 1 or 2) in one launch;
// qkv_attn_supported tells the GEMV shapes it takes (k up to 8192).  ready:
// kReadyLines 128-byte lines, the count of 128-row group g of the QKV output
// (g < n_q + 2 n_kv < kReadyLines) at word kReadyStride g, zero on entry and
// left zero; bit 0 of the last line's first word is set if a wait of the
// attention blocks gave up.  (Counts sharing a line made the launch 21 us
// instead of 11.8 at the 7B shape: the pollers and the GEMV's atomics meet
// on one line.)
constexpr int kReadyStride = 32;  // words: one count per 128-byte line
constexpr int kReadyLines = 128;
bool qkv_attn_supported(int wb, int pro, int64_t n, int64_t k);
hipError_t launch_qkv_attn(int wb, int pro, const GemvArgs& a, const AttnArgs& at, int dqr, uint32_t* ready,
                           hipStream_t s);
// m query rows at positions kv_len + pos_offset + j (q_rot and the cache already
// written by rope_append): per-row split partials, then a merge into out.
hipError_t launch_rows_attention(const AttnArgs& a, hipStream_t s);
// Importance scores of one layer after launch_rows_attention (a.ml set):
// score[hk][j] for j < kv_len + m, over the last `window` rows.
hipError_t launch_attn_scores(const AttnArgs& a, float* score, int window, hipStream_t s);
int attn_scores_max_pairs();
// Sparse index of every (layer, KV head) list from the scores.
hipError_t launch_kv_select(const float* score, int cap, const int32_t* kv_len, int n_lists, int n_sink,
                            int n_recent, int budget_permille, int32_t* index, int index_cap,
                            int32_t* index_len, hipStream_t s);

// ------------------------------------------------------------------ misc kernels
hipError_t launch_rmsnorm_rows(const uint16_t* h, const uint16_t* g, float eps, int rows, int k,
                               uint16_t* out, hipStream_t s);
// h[r] = bf16(h[r] + sum over splits of part[s][r]) in place (splits in
// order; skipped when part is null), then out[r] = RMSNorm(h[r]) * g.  k <= 8192.
hipError_t launch_resid_rmsnorm_rows(uint16_t* h, const float* part, int splits, const uint16_t* g, float eps,
                                     int rows, int k, uint16_t* out, hipStream_t s);
// h[r] = embed[tokens[r * tok_stride]] (ids clamped into [0, vocab)); with
// rows_per_seq > 0 the token of row r is
// tokens[(r / rows_per_seq) * seq_stride + (r % rows_per_seq) * tok_stride].
hipError_t launch_embed_rows(const uint16_t* embed, const int32_t* tokens, int rows, int k,
                             int vocab, uint16_t* h, hipStream_t s, int tok_stride = 1, int rows_per_seq = 0,
                             int64_t seq_stride = 0);
// Batched decoding: kv_len[b] += n[b] + 1, tokens[b ld] = out[b out_ld + n[b]]
// (or, with n_accepted NULL, kv_len[b] += delta).
hipError_t launch_batch_rollback(int32_t* kv_len, int32_t* tokens, int64_t ld, const int32_t* n_accepted,
                                 const int32_t* out_tokens, int64_t out_ld, int batch, int delta, hipStream_t s);
// act[r][j] = bf16(silu(gu[r][j]) * gu[r][F + j]) for r < rows, j < F.
hipError_t launch_silu_rows(const uint16_t* gu, int64_t F, int rows, uint16_t* act, hipStream_t s);
// Static tree: move the accepted chain's K/V next to the prefix (every layer
// and KV head of a [layers x KV heads][cap][d] cache); kv_len is not changed.
hipError_t launch_tree_commit(uint16_t* k_cache, uint16_t* v_cache, int layers_x_kv_heads, int cap, int d,
                              const int32_t* kv_len, const int32_t* n_accepted, const int32_t* chain, int D,
                              hipStream_t s);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_kv_rollback(int32_t* kv_len, int32_t* tokens, const int32_t* n_accepted,
                              const int32_t* out_tokens, hipStream_t s);
hipError_t launch_kv_advance(int32_t* kv_len, int32_t delta, hipStream_t s);
// dst[n] = out_tokens[n] for n = *n_accepted in [0, max_n] (one thread)
hipError_t launch_token_append(int32_t* dst, int max_n, const int32_t* n_accepted, const int32_t* out_tokens,
                               hipStream_t s);
// Draft step: position check (valid, token_out = -1 when out of range, or
// when step >= *draft_len with draft_len set) and the RoPE table (cos, sin)
// [d/2][2] of position kv_len + step.
hipError_t launch_pos_guard(const int32_t* kv_len, const int32_t* token_in, int step, int cap,
                            int vocab, int32_t* valid, int32_t* token_out, int d, float theta,
                            float* rope_cs, const int32_t* draft_len, hipStream_t s);
// RoPE table [m][d/2][2] of the rows' positions: row j is node
// t = pos_offset + j * row_stride at position kv_len + t (tree_d = 0) or
// kv_len + depth(t) in the static tree of chains of depth tree_d.
// rows_per_seq > 0: row j belongs to sequence j / rows_per_seq, whose kv_len
// is kv_len[j / rows_per_seq], and is node (j % rows_per_seq) of it.
hipError_t launch_rope_table(const int32_t* kv_len, int pos_offset, int row_stride, int tree_d, int m, int d,
                             float theta, float* rope_cs, hipStream_t s, int rows_per_seq = 0);

// ------------------------------------------------------------------ sampling / rejection
struct SampleWs {
  float* part_max;
  int32_t* part_arg;
  unsigned long long* chunk_sum;
  uint32_t* counter;
};
int sample_chunks(int vocab);
hipError_t launch_sample(const uint16_t* logits, int vocab, float temp, const uint32_t* u_code,
                         const float* pre_max, const int32_t* pre_arg, int n_pre,
                         int32_t* token, const int32_t* valid, const SampleWs& ws, hipStream_t s);
hipError_t launch_rowmax(const uint16_t* logits, int vocab, float* part_max, int32_t* part_arg,
                         int n_chunks, hipStream_t s);

struct RejectWs {                    // per batch element b, at offset b x the one-element size:
  float* row_max;                    // [batch][rows][chunks]
  int32_t* row_arg;                  // [batch][rows][chunks]
  int32_t* row_bad;                  // [batch][rows][chunks] non-finite flags
  unsigned long long* row_sum;       // [batch][rows][chunks]
  unsigned long long* res_sum;       // [batch][chunks]
  uint32_t* counter;                 // [batch] arrival counters (zero between launches)
};
int reject_chunks(int vocab);
size_t reject_ws_bytes(int gamma, int vocab);
// gamma_len (optional, device [batch]): each round judges only the first
// min(*gamma_len, gamma) draft tokens (a draft stopped early).  batch
// independent rounds (grid z): every pointer argument is [batch] x its
// one-round extent, consecutive - except that the draft tokens, r codes and
// u codes of round b may start at b x tok_stride, r_stride, u_stride
// (defaults gamma, gamma, 1; 0 shares one set: the chains of a tree).
hipError_t launch_reject(int gamma, int vocab, float temp, float draft_temp, const uint16_t* zt,
                         const uint16_t* zd, const int32_t* toks, const uint32_t* r_codes,
                         const uint32_t* u_code, int32_t* n_out, int32_t* out_tokens,
                         int32_t* status, float* probs, const RejectWs& ws, hipStream_t s,
                         const int32_t* gamma_len = nullptr, int batch = 1, int tok_stride = -1,
                         int r_stride = -1, int u_stride = -1);

// ------------------------------------------------------------------ adaptive draft length
struct ControlArgs {
  int32_t* draft_len;   // device: draft length of the round (gamma_max at its start)
  double* state;        // device [8]: h_acc, h_rej, seen_acc, seen_rej, P, A, last length, spare
  float* entropy;       // device [gamma_max]: entropy of each drafted token
  double c, beta;       // C_d / C_v, EMA rate
  int gamma_max;
};
int control_chunks(int vocab);
// After draft step `step`: entropy of the step's logits and the controller's
// continue/stop decision (may lower *draft_len to step + 1); nothing when the
// step was not drafted (step >= *draft_len).
hipError_t launch_draft_control(const ControlArgs& c, int step, const uint16_t* logits, int vocab,
                                double* part, uint32_t* counter, hipStream_t s);
// After the rejection round: EMA updates from n accepted, then a fresh round.
hipError_t launch_control_update(const ControlArgs& c, const int32_t* n_accepted, hipStream_t s);
hipError_t launch_control_init(const ControlArgs& c, hipStream_t s);

// ------------------------------------------------------------------ static token tree
// k chains of depth D share the root; chain c's depth-d node is node
// 1 + c D + d - 1 (node 0: the root).
// Tokens from rows of logits (one 1024-thread block per row): row r writes
// nout tokens tokens[r t_row + i t_out] - its nout largest logits (T = 0;
// larger first, lower index first on ties, token 0 past the finite ones) or
// nout inverse-CDF draws with u[r u_row + i u_out] (T > 0) - or -1 tokens
// when kv_len[r kv_row] + need > cap (no room in the cache).  Static tree:
// level 0 is one row with nout = k children at tokens[1 + c D]; level
// d >= 1 is k rows (chains) writing tokens[1 + c D + d].
struct RowsSampleArgs {
  const uint16_t* logits;
  int64_t ld;
  int V;
  float T;
  const uint32_t* u;
  int64_t u_row, u_out;
  int32_t* tokens;
  int64_t t_row, t_out;
  int nout;
  const int32_t* kv_len;
  int64_t kv_row;
  int need, cap;
};
hipError_t launch_rows_sample(const RowsSampleArgs& a, int rows, hipStream_t s);
// The root's multi-step rejection and the round's result, from the root's
// target and draft rows and every chain's own round (chain_n [k],
// chain_out [k][D], chain_status [k]); resid: [V] 64-bit scratch.
hipError_t launch_tree_root(const uint16_t* zt, const uint16_t* zd, int V, float T, float Td, const int32_t* tokens,
                            int k, int D, const uint32_t* r_codes, const uint32_t* u_code, const int32_t* chain_n,
                            const int32_t* chain_out, const int32_t* chain_status, unsigned long long* resid,
                            int32_t* n_accepted, int32_t* chain, int32_t* out_tokens, int32_t* status,
                            hipStream_t s);
