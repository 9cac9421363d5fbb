/*
 * subspec.h - C ABI of libsubspec.so: the hot path of self-speculative decoding
 * with a 4-bit (W4A16) substitute draft, for one AMD Instinct MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *   [SD]  "How speculative decoding makes LLMs go brrr" (digest): overall flow
 *         and pseudo-code of one speculative step; Module 1 (drafter returns
 *         gamma candidates and q(x)); Module 2 (one causal target forward over
 *         gamma+1 positions, KV rollback); Module 3 (rejection sampling).
 *   [SSN] "SubSpec: Speculate Deep and Accurate" (paper note), Method details:
 *         substitute layers are the target's own layers quantised without
 *         calibration data; resident layers and the KV cache are shared.
 *   [SSR] "SubSpec: the target's own low-bit shadow as the draft" (report),
 *         section 2.2 (4-bit substitutes, sharpened draft), section 3.2
 *         (greedy verification, Table 1).
 *         Sections 6.3, 6.4, 3.7: SubSpec's static deep/narrow token tree
 *         (k = 6, D = 48) verified the SpecInfer way.
 *   [SSL] "The second ledger of speculative decoding" (SparseSpec-L blog),
 *         section 3.1 (the draft reads a ~10% index of sink, recent and
 *         important positions, gathered from the dense cache) and section
 *         3.2 (importance = attention of the last W = 16 query positions of
 *         the verify pass; the index is rebuilt after every verify).
 *
 * Conventions shared by every entry point
 *   - All buffer pointers are DEVICE pointers unless stated otherwise; the
 *     caller allocates and frees them.  The library allocates nothing.
 *   - bf16 values are passed as uint16_t bit patterns, fp16 as uint16_t.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it and returns; outputs are valid after the stream
 *     has been synchronised.
 *   - Return value: SUBSPEC_OK (0) or a negative error code.  On an argument,
 *     shape, capacity or workspace error NOTHING is enqueued and
 *     subspec_last_error() describes the problem.  A HIP launch failure
 *     returns SUBSPEC_EHIP (work enqueued before it is not rolled back).
 *   - Scratch memory comes from the caller's workspace `ws` of `ws_bytes`
 *     bytes (see subspec_workspace_bytes).  It must be zero-filled once with
 *     subspec_workspace_init before first use; kernels leave the counters in
 *     it at zero again.  Calls that share one workspace must be ordered on
 *     one stream.
 *   - Uniform random numbers are passed as integer codes U in [0, 2^24),
 *     meaning u = U / 2^24.
 */
#ifndef SUBSPEC_H
#define SUBSPEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SUBSPEC_ABI_VERSION 7

enum {
  SUBSPEC_OK = 0,
  SUBSPEC_EINVAL = -1,       /* NULL pointer or out-of-range scalar          */
  SUBSPEC_ESHAPE = -2,       /* dimensions the kernels do not support        */
  SUBSPEC_ECAPACITY = -3,    /* KV capacity or token buffer too small         */
  SUBSPEC_EHIP = -4,         /* a HIP runtime call failed                     */
  SUBSPEC_EUNSUPPORTED = -5, /* a parameter value the library does not handle */
  SUBSPEC_EWORKSPACE = -6    /* workspace NULL or smaller than required       */
};

/* Byte offset in a workspace of the device word whose bit 0 records a
 * bounded cross-block wait that gave up (see subspec_draft_step). */
#define SUBSPEC_WS_WAIT_FAULT_OFFSET 65408

/* status bits written by subspec_reject */
enum {
  SUBSPEC_STATUS_NONFINITE = 1,     /* a non-finite logit in a row that was read  */
  SUBSPEC_STATUS_ZERO_RESIDUAL = 2, /* max(0,p-q) had no mass; drew from p        */
  SUBSPEC_STATUS_Q_ZERO = 4         /* a draft token had q(x) = 0                  */
};

/* Library ABI version (SUBSPEC_ABI_VERSION of the build). */
int subspec_abi_version(void);

/* Message of the last failing call made by this host thread ("" if none). */
const char *subspec_last_error(void);

/* ------------------------------------------------------------------------ */
/* Model description (host structs holding device pointers)                 */
/* ------------------------------------------------------------------------ */

/* One linear layer y = W x with W of shape [n][k] (row n = output n).
 * Exactly one of the two forms is set:
 *   bf16:  w     = bf16 [n][k] row-major, codes = meta = NULL;
 *   low-bit: codes = uint8 rows of `bits`-bit codes in the layout of
 *          subspec_quantize ([n][k/2] at 4 bits, [n][k/4] at 2, [n][3k/8]
 *          at 3), meta = fp16 [n][k/64][2] = {scale, min} of each 64-group
 *          along k; the weight is q * scale + min; w = NULL.
 *   bits:  4, 3 or 2 for the low-bit form (0 reads as 4); ignored for bf16.
 *   layout: 0 for the row-major codes and meta above; 1 for 4- or 2-bit
 *          codes and meta in the 16-row tiles of subspec_tile_codes (n % 16
 *          == 0, k % 128 == 0 at 4 bits and k % 256 == 0 at 2, k <= 28672;
 *          the draft step's GEMV then runs on the matrix cores; the skinny
 *          GEMM of subspec_w4_gemm and the row paths take 4 bits only).
 *          Ignored for bf16. */
typedef struct {
  const uint16_t *w;
  const uint8_t *codes;
  const uint16_t *meta;
  int64_t n, k;
  int32_t bits;
  int32_t layout;
} subspec_linear;

/* One decoder layer ([SSN] Method details: a substitute keeps the layer's
 * structure).  The target (verify) weights are always bf16.  The draft
 * weights are the W4 substitutes, or the same bf16 pointers for a layer the
 * draft shares with the target.
 *   qkv     [(Hq + 2 Hkv) d][H]  rows: all q heads, then k heads, then v heads
 *   o       [H][Hq d]
 *   gate_up [2 F][H]             rows 0..F-1 gate, rows F..2F-1 up
 *   down    [H][F]                                                         */
typedef struct {
  const uint16_t *attn_norm, *ffn_norm; /* bf16 [H] RMSNorm weights */
  subspec_linear qkv, o, gate_up, down;
  subspec_linear qkv_d, o_d, gate_up_d, down_d;
} subspec_layer;

/* Model description.  Supported: head_dim 128; hidden and ffn multiples of
 * 128, hidden <= 6144, ffn <= 28672; n_q_heads a multiple of n_kv_heads
 * with a group n_q_heads / n_kv_heads <= 8; vocab <= 2^24
 * (SUBSPEC_EUNSUPPORTED / SUBSPEC_ESHAPE otherwise). */
typedef struct {
  int32_t n_layers, hidden, ffn, n_q_heads, n_kv_heads, head_dim, vocab;
  float rope_theta, rms_eps;
  const uint16_t *embed;      /* bf16 [vocab][hidden]  */
  const uint16_t *final_norm; /* bf16 [hidden]         */
  const uint16_t *lm_head;    /* bf16 [vocab][hidden]  */
  const subspec_layer *layers; /* HOST array [n_layers] */
} subspec_model;

/* Decode state shared by draft and verify ([SSN]: one KV cache).
 *   k_cache, v_cache  bf16 [n_layers][Hkv][capacity][head_dim]
 *   kv_len            device int32: positions [0, kv_len) hold committed
 *                     target K/V; the last committed token is tokens[0] and
 *                     has not been run yet (kv_len = committed - 1)
 *   tokens            device int32 [gamma_max + 1]: [0] last committed token,
 *                     [1..gamma] the draft tokens of the current cycle
 *   draft_logits      device bf16 [gamma_max][vocab]: row i = logits the
 *                     draft produced at step i (the distribution of tokens[i+1])
 * Sparse-KV drafting ([SSL] sections 3.1-3.2; leave kv_score and kv_index
 * NULL for dense drafting):
 *   kv_score          device fp32 [n_layers][Hkv][capacity]: written by every
 *                     verify call: score[l][hk][j] = sum over the call's last
 *                     min(score_window, n_tokens) rows r and the query heads
 *                     h of KV head hk of the attention probability row r,
 *                     head h gave position j (0 where j is past row r)
 *   kv_index          device int32 [n_layers][Hkv][index_cap]: ascending
 *                     positions, written by subspec_kv_select
 *   kv_index_len      device int32 scalar: entries of every list
 *   index_cap         capacity of each list; must be >= the count for
 *                     kv_len = capacity (see subspec_kv_select)
 *   use_index         host flag: nonzero -> draft_step attends, per layer and
 *                     KV head, to the index plus the speculative positions
 *                     [kv_len, kv_len + step]; zero -> dense (first cycle)
 *   n_sink, n_recent  positions always kept at the start and the end
 *   score_window      verify rows that feed the scores, 1..16
 *   budget_permille   index size ceil(budget_permille * kv_len / 1000), in
 *                     thousandths so that the count is exact integer math */
typedef struct {
  uint16_t *k_cache, *v_cache;
  int32_t capacity;
  int32_t *kv_len;
  int32_t *tokens;
  uint16_t *draft_logits;
  int32_t gamma_max;
  float *kv_score;
  int32_t *kv_index;
  int32_t *kv_index_len;
  int32_t index_cap;
  int32_t use_index;
  int32_t n_sink, n_recent, score_window, budget_permille;
  const int32_t *draft_len; /* device int32 or NULL: with the entropy-adaptive
                               draft length (subspec_control), draft steps
                               with step >= *draft_len are skipped (token -1) */
  int32_t attn_own_launch;  /* host flag: 0 -> a draft step runs a layer's
                               attention in the QKV projection's launch where
                               it can (see subspec_draft_step); nonzero -> in
                               a launch of its own (same results, bit for bit) */
} subspec_state;

/* Bytes of workspace needed for calls on `m` with at most `max_tokens`
 * positions per verify call and a KV capacity of `capacity`.  Returns 0 if
 * the model description is invalid (see subspec_last_error). */
size_t subspec_workspace_bytes(const subspec_model *m, int32_t max_tokens, int32_t capacity);

/* Zero-fill a workspace (a fill kernel; safe inside stream capture). */
int subspec_workspace_init(void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------ */
/* Substitute construction  ([SSN] Method details; [SSR] section 2.2)        */
/* ------------------------------------------------------------------------ */

/* Quantise a bf16 [n][k] matrix to `bits`-bit uniform asymmetric codes
 * (bits = 4, 3 or 2; L = 2^bits - 1), groups of `group` = 64 consecutive
 * weights along k ([SSN]: substitutes at 2/3 bits; [SSR] section 2.2: 4).
 * Per group: lo/hi = min/max, scale = the smallest fp16 value s with
 * L s >= fl32(hi - lo), found as fp16(fl32(fl32(hi-lo)/L)) raised by one fp16
 * step when L s falls short (1 if it is 0; saturating at the fp16 maximum),
 * min = fp16(lo) (saturating), code = clamp(rint_even(fl32(fl32(x-min)/
 * scale)), 0, L) using the stored fp16 values, no fused multiply-add; every
 * weight in the fp16 range is then within scale/2 of its level.
 * Outputs: meta fp16 [n][k/64][2] = {scale, min}; codes uint8, per row:
 *   4 bits: k/2 bytes, byte j = q[2j] | q[2j+1] << 4;
 *   2 bits: k/4 bytes, byte j = q[4j] | q[4j+1] << 2 | q[4j+2] << 4 | q[4j+3] << 6;
 *   3 bits: 3k/8 bytes: the low two bits of every code in the 2-bit layout
 *           (k/4 bytes), then the third bits (k/8 bytes) in 4-byte words of
 *           32 weights whose bytes hold weights 0-7, 16-23, 8-15, 24-31 of
 *           the word (bit t of a byte: its t-th weight).
 * k % 64 == 0 (k % 128 == 0 at 3 bits, so rows stay 16-byte aligned),
 * group == 64; otherwise SUBSPEC_EUNSUPPORTED / SUBSPEC_ESHAPE. */
int subspec_quantize(const uint16_t *w, int64_t n, int64_t k, int32_t group, int32_t bits,
                     uint8_t *codes, uint16_t *meta, void *stream);

/* The same 4- or 2-bit codes and meta in 16-row tiles
 * (subspec_linear.layout = 1), the storage order of the batch-1 draft GEMV
 * on the matrix cores: a storage choice of this library, not of the method
 * (the substitute is the [SSR] section 2.2 / [SSN] low-bit quantisation
 * either way; the values are moved, not changed).  A chunk is 64 bytes of a
 * row: c_k = 512 / bits weights (128 at 4 bits, 256 at 2), e = 8 / bits
 * 64-groups.  For tile t (rows 16t .. 16t + 15) and chunk c, with c_n =
 * k / c_k chunks a row and b = (t c_n + c):
 *   tcodes[1024 b + 16 (16 g + r) + j] = codes[(16t + r) R + 64 c + 16 g + j]
 *       for r < 16, g < 4, j < 16, R = k bits / 8 code bytes a row;
 *   tmeta dword 16 e b + e r + f = meta dword (16t + r) k/64 + e c + f, f < e
 *       (meta dword = {scale, min} of one 64-group).
 * codes, meta: the subspec_quantize output at `bits` = 4 or 2 (device; not
 * modified); tcodes (n R bytes), tmeta (n k/64 dwords): device outputs
 * owned by the caller, not overlapping the inputs.  n % 16 == 0 and
 * k % c_k == 0 (SUBSPEC_ESHAPE otherwise); other widths:
 * SUBSPEC_EUNSUPPORTED; NULL pointers: SUBSPEC_EINVAL. */
int subspec_tile_codes(const uint8_t *codes, const uint16_t *meta, int64_t n, int64_t k, int32_t bits,
                       uint8_t *tcodes, uint16_t *tmeta, void *stream);

/* ------------------------------------------------------------------------ */
/* The speculative cycle  ([SD] pseudo-code)                                 */
/* ------------------------------------------------------------------------ */

/* Draft step `step` (0 <= step < gamma_max): run tokens[step] at position
 * kv_len + step through the draft (substitute and shared layers), write its
 * K/V into the shared cache at that position, store the logits in
 * draft_logits[step] and the drawn token in tokens[step + 1].  The token is
 * the argmax (lowest index on ties) when draft_temp == 0, else the inverse
 * CDF of softmax(logits / draft_temp) at u = u_codes[step] / 2^24
 * ([SSR] section 3.4: sharpened draft).  u_codes: device uint32 [> step].
 * Needs kv_len + step < capacity (checked on the device: out-of-range
 * positions are skipped and tokens[step+1] is set to -1).
 * On a layer whose QKV substitute is 4- or 2-bit in 16-row tiles, with dense
 * keys (use_index == 0), hidden size <= 8192 and capacity <= 256 keys per
 * key split of the per-head attention (two 16-key chunks a wave; 2048 keys
 * at 8 splits), the attention runs in the QKV GEMV's launch unless
 * st->attn_own_launch is set:
 * extra blocks wait for the counts the GEMV blocks leave in the workspace
 * once a head's q/k/v rows are stored.  Those waits are bounded (0.2 s); a
 * wait that gives up sets bit 0 of the workspace word at byte offset
 * SUBSPEC_WS_WAIT_FAULT_OFFSET (the step's results are then undefined and
 * the workspace must be re-initialised with subspec_workspace_init). */
int subspec_draft_step(const subspec_model *m, const subspec_state *st, int32_t step,
                       float draft_temp, const uint32_t *u_codes, void *ws, size_t ws_bytes,
                       void *stream);

/* Verify ([SD] Module 2): run `n_tokens` tokens (device int32 [n_tokens]) at
 * positions kv_len .. kv_len + n_tokens - 1 through the bf16 target in one
 * causal pass (row j attends to [0, kv_len + j]); overwrite those K/V
 * entries with the target's; write logits bf16 [n_tokens][vocab] unless
 * `logits` is NULL (prefill).  1 <= n_tokens <= max_tokens of the workspace. */
int subspec_verify(const subspec_model *m, const subspec_state *st, int32_t n_tokens,
                   const int32_t *tokens, uint16_t *logits, void *ws, size_t ws_bytes,
                   void *stream);

/* One rejection round ([SD] Module 3; [SSR] section 3.2 for T = 0).
 *   target_logits bf16 [gamma+1][vocab]; draft_logits bf16 [gamma][vocab];
 *   draft_tokens int32 [gamma]; r_codes uint32 [gamma]; u_code uint32 [1].
 * For i = 0..gamma-1 draft_tokens[i] is accepted iff r_i < p_i(x)/q_i(x),
 * with p_i = softmax(target_logits[i]/temp) (one-hot argmax if temp == 0)
 * and q_i = softmax(draft_logits[i]/draft_temp) (one-hot argmax if
 * draft_temp == 0).  At the first rejection n = i and one token is drawn
 * from norm(max(0, p_i - q_i)); if all are accepted n = gamma and the bonus
 * token is drawn from p_gamma.  Weights are exp((z - max)/T) in float32,
 * truncated to integers floor(w * 2^40) so that every sum and comparison is
 * exact; draws use the inverse CDF at u_code.
 * Outputs (device): n_accepted int32 [1]; out_tokens int32 [gamma+1], first
 * n+1 valid; status int32 [1] (SUBSPEC_STATUS_* bits); probs float [gamma][2]
 * = (p_i(x_i), q_i(x_i)) for i <= n (optional, may be NULL).
 * 0 <= gamma <= 64, 1 <= vocab <= 2^24. */
int subspec_reject(int32_t gamma, int32_t vocab, float temp, float draft_temp,
                   const uint16_t *target_logits, const uint16_t *draft_logits,
                   const int32_t *draft_tokens, const uint32_t *r_codes, const uint32_t *u_code,
                   int32_t *n_accepted, int32_t *out_tokens, int32_t *status, float *probs,
                   void *ws, size_t ws_bytes, void *stream);

/* `batch` independent rejection rounds in one launch set (the rounds of B
 * sequences decoded together with shared substitutes; [SSR] section 10.3,
 * batch > 1).  Each round is exactly subspec_reject_len on its slice: every
 * pointer is [batch] x its one-round extent, consecutive:
 *   target_logits [B][gamma+1][vocab], draft_logits [B][gamma][vocab],
 *   draft_tokens and r_codes [B][gamma], u_codes [B], gamma_len [B] (device;
 *   NULL = gamma for every round), n_accepted and status [B], out_tokens
 *   [B][gamma+1], probs [B][gamma][2] (optional).
 * 1 <= batch <= 4096; workspace of subspec_reject_workspace_bytes(batch, gamma,
 * vocab) bytes (zero-filled once, like every workspace). */
int subspec_reject_batch(int32_t batch, int32_t gamma, int32_t vocab, float temp, float draft_temp,
                         const uint16_t *target_logits, const uint16_t *draft_logits,
                         const int32_t *draft_tokens, const uint32_t *r_codes, const uint32_t *u_codes,
                         const int32_t *gamma_len, int32_t *n_accepted, int32_t *out_tokens, int32_t *status,
                         float *probs, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes subspec_reject_batch needs (0 on invalid arguments). */
size_t subspec_reject_workspace_bytes(int32_t batch, int32_t gamma, int32_t vocab);

/* subspec_reject without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, kernels and results as
 * subspec_reject, minus ws / ws_bytes: the scratch (per-row partial maxima,
 * flags and fixed-point sums, residual chunk sums, the arrival counter) is a
 * static 1 MiB device array per GPU, held until the process ends; its device
 * address is looked up once per device (hipGetSymbolAddress).  The call
 * allocates nothing and clears the counter itself with a fill kernel.
 * Limit: 1024 + 20 (2 gamma + 1) ceil(vocab / 4096) bytes (each array rounded
 * up to 256 bytes) must fit in 1 MiB, else SUBSPEC_ECAPACITY and nothing is
 * enqueued (gamma 64 fits vocab up to ~1.6M; gamma 16 up to 2^24 does not).
 * Every call on one GPU uses that GPU's one array: calls that overlap on one
 * GPU (two streams, or two threads) race and must be serialised by the
 * caller. */
int subspec_reject_noalloc(int32_t gamma, int32_t vocab, float temp, float draft_temp,
                           const uint16_t *target_logits, const uint16_t *draft_logits,
                           const int32_t *draft_tokens, const uint32_t *r_codes, const uint32_t *u_code,
                           int32_t *n_accepted, int32_t *out_tokens, int32_t *status, float *probs,
                           void *stream);

/* The rejection round of a draft that may have stopped early: as
 * subspec_reject, but only the first min(*gamma_len, gamma) draft tokens are
 * judged (gamma_len: device int32, the round's draft length); if they are all
 * accepted the bonus token is drawn from target row *gamma_len.  Used with
 * the entropy-adaptive draft length ([SSL] section 3.3). */
int subspec_reject_len(int32_t gamma, int32_t vocab, float temp, float draft_temp,
                       const uint16_t *target_logits, const uint16_t *draft_logits,
                       const int32_t *draft_tokens, const uint32_t *r_codes, const uint32_t *u_code,
                       const int32_t *gamma_len, int32_t *n_accepted, int32_t *out_tokens, int32_t *status,
                       float *probs, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------ */
/* Multi-level substitutes  ([SSR] §10.3 item 9)                             */
/* ------------------------------------------------------------------------ */

/* A 2-bit substitute drafts for the 4-bit draft, which drafts for the bf16
 * target.  Reading: nested speculation - the 4-bit draft's gamma tokens come
 * from inner rounds: draft steps of a model with 2-bit substitutes (the same
 * shared layers and cache), one pass of the 4-bit draft over the drafted
 * positions (subspec_draft_verify), the plain round (subspec_reject with
 * p = 4-bit, q = 2-bit), and the round's last token appended after its
 * accepted drafts (subspec_draft_append); the outer round then judges the
 * gamma tokens against the target with q = the 4-bit logits those passes
 * computed. */

/* The draft weights' pass over n_tokens (<= 16) positions: tokens[j] at
 * position kv_len + pos_offset + j (causal), bf16 shared layers and 4-bit
 * substitutes; writes their K/V (slots past the capacity are skipped on the
 * device) and, unless NULL, logits [n_tokens][vocab].  Errors: EINVAL for a
 * NULL tokens or n_tokens outside [1, 16], ECAPACITY when pos_offset +
 * n_tokens exceeds the capacity, EWORKSPACE for a short workspace. */
int subspec_draft_verify(const subspec_model *m, const subspec_state *st, int32_t pos_offset, int32_t n_tokens,
                         const int32_t *tokens, uint16_t *logits, void *ws, size_t ws_bytes, void *stream);

/* tokens[at + n] = out_tokens[n] with n = *n_accepted (device): a round's
 * last token placed after its accepted drafts.  A device n outside
 * [0, max_n] writes nothing.  Errors: EINVAL for NULL buffers, at < 0,
 * max_n < 0 or at + max_n > gamma_max (the tokens buffer holds gamma_max + 1
 * entries). */
int subspec_draft_append(const subspec_state *st, int32_t at, int32_t max_n, const int32_t *n_accepted,
                         const int32_t *out_tokens,
                         void *stream);

/* ------------------------------------------------------------------------ */
/* Batched decoding: B sequences share the substitutes ([SSR] §10.3 item 11)  */
/* ------------------------------------------------------------------------ */

/* B independent sequences decoded together, so that every weight (bf16 or
 * 4-bit) streams once per step for all of them: each has its own KV cache
 * region, length and tokens.  Buffers (device): k_cache / v_cache bf16
 * [L][batch][Hkv][capacity][d]; kv_len [batch]; tokens [batch][gamma_max + 1]
 * ([b][0] the last committed token, [b][1..] drafts); draft_logits
 * [batch][gamma_max][vocab].  1 <= batch <= 16 (the draft step's rows);
 * the draft step takes vocab <= 524288. */
typedef struct {
  uint16_t *k_cache, *v_cache;
  int32_t capacity;
  int32_t batch;
  int32_t *kv_len;
  int32_t *tokens;
  uint16_t *draft_logits;
  int32_t gamma_max;
} subspec_batch_state;

/* Workspace bytes for batch_draft_step / batch_verify of up to max_tokens
 * positions per sequence and batch_reject with gamma = max_tokens - 1. */
size_t subspec_batch_workspace_bytes(const subspec_model *m, int32_t batch, int32_t max_tokens, int32_t capacity);

/* Draft step `step` of every sequence at once: row b runs tokens[b][step]
 * at position kv_len[b] + step through the draft, writes its K/V there and
 * draft_logits[b][step], and draws tokens[b][step + 1] (argmax, or the
 * inverse CDF with u_codes[b gamma_max + step]); a sequence whose position
 * is past its capacity gets token -1.  Draft weights bf16 or 4-bit.  With
 * batch = 1 this is subspec_draft_step on the same buffers. */
int subspec_batch_draft_step(const subspec_model *m, const subspec_batch_state *st, int32_t step, float draft_temp,
                             const uint32_t *u_codes, void *ws, size_t ws_bytes, void *stream);

/* The target pass over n_tokens positions of every sequence: row j of
 * sequence b runs tokens[b ld_tokens + j] at kv_len[b] + j (causal within the
 * sequence), writes its K/V and, unless logits is NULL, logits
 * [batch][n_tokens][vocab].  batch x n_tokens <= 512, n_tokens <= 64. */
int subspec_batch_verify(const subspec_model *m, const subspec_batch_state *st, int32_t n_tokens,
                         const int32_t *tokens, int64_t ld_tokens, uint16_t *logits, void *ws, size_t ws_bytes,
                         void *stream);

/* Every sequence's rejection round (subspec_reject's rule and arithmetic)
 * over gamma = gamma_max drafts: target_logits [batch][gamma + 1][vocab],
 * the state's draft logits and tokens, r_codes [batch][gamma], u_codes
 * [batch]; outputs n_accepted [batch], out_tokens [batch][gamma + 1],
 * status [batch]. */
int subspec_batch_reject(const subspec_model *m, const subspec_batch_state *st, float temp, float draft_temp,
                         const uint16_t *target_logits, const uint32_t *r_codes, const uint32_t *u_codes,
                         int32_t *n_accepted, int32_t *out_tokens, int32_t *status, void *ws, size_t ws_bytes,
                         void *stream);

/* kv_len[b] += n_accepted[b] + 1 and tokens[b][0] = out_tokens[b][n] for
 * every sequence (out_tokens [batch][gamma_max + 1]); with n_accepted NULL,
 * kv_len[b] += delta (prefill). */
int subspec_batch_rollback(const subspec_batch_state *st, const int32_t *n_accepted, const int32_t *out_tokens,
                           int32_t delta, void *stream);

/* ------------------------------------------------------------------------ */
/* The static token tree  ([SSR] sections 6.3, 6.4 and 3.7)                  */
/* ------------------------------------------------------------------------ */

/* SubSpec drafts a static tree, deep and narrow (k = 6, D = 48), and verifies
 * every path in one target pass (SpecInfer's tree verification).  Reading
 * (the pages name only k and D): k chains of depth D share the root, the last
 * committed token tokens[0].  Node t = 1 + c D + d - 1 is chain c's node at
 * depth d (1 <= d <= D): cache slot kv_len + t, position kv_len + d; it
 * attends to slots [0, kv_len] and to its own chain's slots up to its own.
 * The state's buffers hold the tree: tokens [1 + k D] (node order),
 * draft_logits [1 + k (D - 1)][vocab] (row 0 the root, row
 * 1 + c (D - 1) + d - 1 chain c's depth-d node).  kv_len + 1 + k D must not
 * exceed the capacity (checked on the device: a tree that does not fit gets
 * -1 children, and its round emits one token).  1 <= k <= 16, 1 <= D <= 64,
 * 1 + k D <= 512; vocab <= 524288; draft weights bf16 or 4-bit.  One cycle: tree_draft for
 * level 0 .. D - 1, tree_verify, tree_reject, tree_commit. */

/* Workspace bytes of the four calls below (0 on invalid arguments). */
size_t subspec_tree_workspace_bytes(const subspec_model *m, int32_t k, int32_t depth, int32_t capacity);

/* One draft pass over a level, all chains at once (the 4-bit GEMMs take the
 * k rows in one weight stream).  Level 0 runs the root and writes its k
 * children tokens[1 + c D]: its k largest logits when draft_temp == 0
 * (larger first, lower index first on ties, token 0 past the finite ones),
 * else k draws with u_codes[c] (inverse CDF, [SD] Module 1, as
 * subspec_draft_step).  Level d >= 1 runs the depth-d nodes and writes chain
 * c's next token tokens[1 + c D + d] (argmax, or a draw with
 * u_codes[k + c (D - 1) + d - 1]).  u_codes: device uint32 [k D]. */
int subspec_tree_draft(const subspec_model *m, const subspec_state *st, int32_t k, int32_t depth, int32_t level,
                       float draft_temp, const uint32_t *u_codes, void *ws, size_t ws_bytes, void *stream);

/* The target pass over all 1 + k D nodes (bf16 target weights, tree
 * visibility); writes their K/V and logits bf16 [1 + k D][vocab]. */
int subspec_tree_verify(const subspec_model *m, const subspec_state *st, int32_t k, int32_t depth, uint16_t *logits,
                        void *ws, size_t ws_bytes, void *stream);

/* Judge one tree.  The root: SpecInfer's multi-step rejection over the k
 * children in chain order - child c accepted when
 * r_codes[c] / 2^24 < p_c(x_c) / q(x_c), p_0 = softmax(target row 0 / T),
 * after a rejection p_{c+1} = norm(max(0, p_c - q)), q = softmax(draft row 0
 * / T_d) (one-hot at x_c when draft_temp == 0); T = 0: the first child equal
 * to the target's argmax.  No child accepted: one token drawn from the last
 * p_c with u_code (n = 0).  Child c accepted: chain c's depth-2..D tokens are
 * judged by the plain round (subspec_reject) over its depth-1..D target rows
 * and depth-1..D-1 draft rows with r_codes[k ..] and u_code, and
 * n = 1 + that round's n.  Outputs (device): n_accepted, chain (c, or -1),
 * out_tokens [n + 1] (room for D + 1), status (subspec_reject's bits; a
 * child outside the vocabulary is skipped with bit 4).  Integer arithmetic
 * as subspec_reject; residuals after the first kept below 2^41 by one more
 * bit of shift.  r_codes: [k + D - 1] (needed when temp > 0). */
int subspec_tree_reject(int32_t k, int32_t depth, int32_t vocab, float temp, float draft_temp,
                        const uint16_t *target_logits, const uint16_t *draft_logits, const int32_t *tokens,
                        const uint32_t *r_codes, const uint32_t *u_code, int32_t *n_accepted, int32_t *chain,
                        int32_t *out_tokens, int32_t *status, void *ws, size_t ws_bytes, void *stream);

/* Commit a judged tree: the accepted chain's first n nodes' K/V move to
 * slots kv_len + 1 .. kv_len + n (every layer and KV head), then
 * kv_len += n + 1 and tokens[0] = out_tokens[n] (as subspec_kv_rollback). */
int subspec_tree_commit(const subspec_model *m, const subspec_state *st, int32_t k, int32_t depth,
                        const int32_t *n_accepted, const int32_t *chain, const int32_t *out_tokens, void *stream);

/* ------------------------------------------------------------------------ */
/* Entropy-adaptive draft length  ([SSL] section 3.3)                        */
/* ------------------------------------------------------------------------ */

/* Controller state (device buffers owned by the caller).  Each draft token's
 * entropy H_i (of softmax(logits) at temperature 1) is compared with two EMA
 * centres - the mean entropy of accepted and of rejected draft tokens -
 * giving p_i = d_rej / (d_acc + d_rej) (d: distance to a centre; 1/2 if both
 * are 0; 1 while a centre is unseen); after token i the draft goes on only
 * if some longer length k, with the undrafted tokens at p_i, has
 * E(k) = (1 + sum_{m<=k} prod_{j<=m} p_j) / (k c + 1) > E(i).
 *   draft_len  device int32: the round's draft length (gamma_max at its start)
 *   state      device double [8]: h_acc, h_rej, seen_acc, seen_rej, running
 *              product, running 1 + sum, last round's length, spare
 *   entropy    device float [gamma_max]: entropies of the round's tokens
 *   c          C_d / C_v, draft-step cost over verify-pass cost (> 0)
 *   beta       EMA rate in (0, 1]
 *   gamma_max  longest draft (>= 1)                                         */
typedef struct {
  int32_t *draft_len;
  double *state;
  float *entropy;
  double c, beta;
  int32_t gamma_max;
} subspec_control;

/* Zero the centres and start a round (a fill kernel; capture-safe). */
int subspec_control_init(const subspec_control *ctl, void *stream);

/* After draft step `step`: the entropy of draft_logits[step] and the
 * controller's decision; lowers *draft_len to step + 1 when the draft should
 * stop.  Does nothing for a step that was not drafted (step >= *draft_len).
 * Needs st->draft_len == ctl->draft_len; workspace as for draft steps. */
int subspec_draft_control(const subspec_model *m, const subspec_state *st, int32_t step,
                          const subspec_control *ctl, void *ws, size_t ws_bytes, void *stream);

/* After the rejection round (n = *n_accepted, device): tokens 1..n update the
 * accepted centre in order, token n + 1 (if drafted) the rejected centre;
 * records the round's length in state[6] and starts the next round. */
int subspec_control_update(const subspec_control *ctl, const int32_t *n_accepted, void *stream);

/* Commit a round ([SD] Module 2: discard the K/V of rejected positions):
 * kv_len += n + 1 and tokens[0] = out_tokens[n], n = *n_accepted (device). */
int subspec_kv_rollback(const subspec_state *st, const int32_t *n_accepted,
                        const int32_t *out_tokens, void *stream);

/* Rebuild the sparse draft index ([SSL] sections 3.1-3.2) from the scores
 * of the last verify, after the rollback, over the committed positions
 * [0, L), L = kv_len (device).  For every layer and KV head the list is
 * sink = [0, min(n_sink, L)), recent = [max(sink end, L - n_recent), L), and
 * the K middle positions of highest score (score descending, position
 * ascending on ties), K = ceil(budget_permille * L / 1000) - |sink| -
 * |recent| clipped to [0, middle size]; i.e. min(L, max(ceil(budget * L),
 * |sink| + |recent|)) entries, ascending, count in kv_index_len.  Needs
 * kv_score, kv_index, kv_index_len set and index_cap >= that count at
 * L = capacity (SUBSPEC_ECAPACITY otherwise). */
int subspec_kv_select(const subspec_model *m, const subspec_state *st, void *stream);

/* Entries of every sparse index list that subspec_kv_select builds at
 * kv_len = L ([SSL] section 3.1: sink + recent + important positions, about
 * budget_permille / 1000 of the context): min(L, max(ceil(budget_permille *
 * L / 1000), |sink| + |recent|)) with |sink| = min(n_sink, L) and |recent| =
 * min(n_recent, L - |sink|).  Host-side arithmetic only (no device work);
 * callers size kv_index with it (index_cap = the count at L = capacity).
 * Returns -1 for L < 0, negative n_sink / n_recent or a budget outside
 * [0, 1000]. */
int64_t subspec_index_count(int64_t L, int32_t n_sink, int32_t n_recent, int32_t budget_permille);

/* kv_len += delta (device), e.g. after a prefill chunk run through verify. */
int subspec_kv_advance(const subspec_state *st, int32_t delta, void *stream);

/* ------------------------------------------------------------------------ */
/* Kernel-level entry points (single operations of the path)                 */
/* ------------------------------------------------------------------------ */

/* y[n] = bf16( sum_k (q[n][k] * scale + min) * x[k] ) at batch 1 (the draft's
 * W4A16 GEMV, 4-bit codes; subspec_gemv takes every width).  x bf16 [k],
 * y bf16 [n]; k % 64 == 0. */
int subspec_w4_gemv(const uint8_t *codes, const uint16_t *meta, int64_t n, int64_t k,
                    const uint16_t *x, uint16_t *y, void *stream);

/* Y[t][n] = bf16( sum_k X[t][k] (q[n][k] * scale + min) ) for t < m <= 16 on
 * the matrix cores: the draft of up to 16 sequences decoded together, which
 * share the 4-bit substitutes ([SSR] section 10.3, item 11; the weights
 * stream once for all m).  w: 4-bit codes + meta [n][k]; X bf16 [m][k], Y bf16
 * [m][n]; k % 128 == 0.  Workspace: subspec_w4_gemm_workspace_bytes(n, k, m)
 * (fp32 split-k partials). */
int subspec_w4_gemm(const subspec_linear *w, const uint16_t *x, int32_t m, uint16_t *y, void *ws,
                    size_t ws_bytes, void *stream);
size_t subspec_w4_gemm_workspace_bytes(int64_t n, int64_t k, int32_t m);

/* y[n] = bf16( sum_k w[n][k] x[k] ), bf16 weights at batch 1; k % 8 == 0. */
int subspec_bf16_gemv(const uint16_t *w, int64_t n, int64_t k, const uint16_t *x, uint16_t *y,
                      void *stream);

/* The draft step's fused GEMV, one launch (the kernels draft_step runs, at
 * kernel level):
 *   x' = norm_w ? bf16( x * rsqrt(mean(x^2) + eps) * norm_w ) : x   (RMSNorm)
 *   epilogue 0: y[n] = bf16( W x' )[n]                 for n < w->n
 *   epilogue 1: y[n] = bf16( resid[n] + (W x')[n] )    for n < w->n
 *   epilogue 2: y[n] = bf16( SiLU(g) * u ), g = bf16((W x')[n]),
 *               u = bf16((W x')[F + n]), for n < F = w->n / 2 (gate rows
 *               first, then the up rows)
 * w: bf16 (w set) or low-bit (codes + meta + bits) weights [n][k]; x, norm_w bf16 [k];
 * resid, y bf16.  k % 64 == 0, k <= 28672 (k <= 6144 with norm_w).  Errors:
 * EINVAL for bad pointers, epilogue or linear; ESHAPE / EUNSUPPORTED for k. */
int subspec_gemv(const subspec_linear *w, const uint16_t *x, const uint16_t *norm_w, float eps,
                 int32_t epilogue, const uint16_t *resid, uint16_t *y, void *stream);

/* Y[t][n] = bf16( sum_k X[t][k] W[n][k] ) for t < m <= 512 (the verify GEMM
 * on matrix cores: slices of 64 positions, or of 128 past 64, each streaming
 * the weights once).  X bf16 [m][k], Y bf16 [m][n]; k % 128 == 0. */
int subspec_bf16_gemm(const uint16_t *w, int64_t n, int64_t k, const uint16_t *x, int32_t m,
                      uint16_t *y, void *ws, size_t ws_bytes, void *stream);

/* Draw one token from bf16 logits [vocab] as subspec_draft_step does
 * (argmax if temp == 0, else inverse CDF at u_code/2^24); token int32 [1]. */
int subspec_sample(const uint16_t *logits, int32_t vocab, float temp, const uint32_t *u_code,
                   int32_t *token, void *ws, size_t ws_bytes, void *stream);

/* Measurement helper: one streaming read of buf (bytes, a positive multiple
 * of 16, 16-byte aligned device memory) by a read-only kernel, the HBM read
 * ceiling that the weight-streaming kernels of the draft and verify passes
 * are measured against (low-batch decode is bound by streaming weights from
 * memory: "How speculative decoding makes LLMs go brrr", Module 2).  The
 * device word *sink is XORed with every 32-bit word of buf (the caller zeroes
 * it first to read the fold); nothing else is written.  Errors: EINVAL for
 * null pointers, ESHAPE for bytes. */
int subspec_hbm_read(const void *buf, int64_t bytes, uint32_t *sink, void *stream);

/* ------------------------------------------------------------------------ */
/* Profiling (host side; off by default)                                     */
/* ------------------------------------------------------------------------ */

/* Launch sites timed by the profiler: one class per kernel and shape role, so
 * that a class average is the average of one kernel at one shape. */
enum {
  SUBSPEC_K_W4_QKV = 0,        /* draft QKV GEMV, 4-bit substitute layer           */
  SUBSPEC_K_W4_O = 1,          /* draft O GEMV + residual, 4-bit                   */
  SUBSPEC_K_W4_GATE_UP = 2,    /* draft gate/up GEMV with SiLU*up, 4-bit           */
  SUBSPEC_K_W4_DOWN = 3,       /* draft down GEMV + residual, 4-bit                */
  SUBSPEC_K_BF16_QKV = 4,      /* the same four on shared bf16 layers              */
  SUBSPEC_K_BF16_O = 5,
  SUBSPEC_K_BF16_GATE_UP = 6,
  SUBSPEC_K_BF16_DOWN = 7,
  SUBSPEC_K_LM_HEAD = 8,       /* draft lm_head GEMV (+ per-block max/argmax)      */
  SUBSPEC_K_GEMM_QKV = 9,      /* verify GEMMs on the matrix cores                 */
  SUBSPEC_K_GEMM_O = 10,
  SUBSPEC_K_GEMM_GATE_UP = 11,
  SUBSPEC_K_GEMM_DOWN = 12,
  SUBSPEC_K_GEMM_LM_HEAD = 13,
  SUBSPEC_K_ATTN_DRAFT = 14,   /* draft RoPE + KV append + split attention         */
  SUBSPEC_K_ATTN_VERIFY = 15,  /* verify RoPE + KV append + causal attention       */
  SUBSPEC_K_SAMPLE = 16,       /* draft token draw                                 */
  SUBSPEC_K_REJECT = 17,       /* rejection round                                  */
  SUBSPEC_K_MISC = 18,         /* norms, embedding, KV bookkeeping                 */
  SUBSPEC_K_SCORES = 19,       /* verify importance scores (sparse drafting)       */
  SUBSPEC_K_SELECT = 20,       /* sparse index rebuild                             */
  SUBSPEC_K_QKV_ATTN = 21,     /* draft QKV GEMV on low-bit tiles with the layer's
                                  attention in the same launch                      */
  SUBSPEC_K_CLASSES = 22
};

/* Start recording: from now on every kernel this library launches, on any
 * stream, is launched with a pair of HIP events that take the dispatch's own
 * start and end timestamps (hipExtLaunchKernel), up to `max_records` records
 * (one per launch, or one per API step that makes several launches; later
 * launches are not recorded).  Creates the events (host-side objects; no
 * device memory).  Returns SUBSPEC_EHIP if event creation fails. */
int subspec_profile_start(int32_t max_records);

/* Stop recording (events already recorded stay readable). */
int subspec_profile_stop(void);

/* Synchronise the recorded events and report, for kernel class `cls`, the
 * number of records, their summed duration in milliseconds and their summed
 * algorithmic bytes (weights, activations and KV each counted once; 0 where
 * the host does not know them, as for attention, whose KV length lives on
 * the device).  A record's duration runs from the end of the previous record
 * on the same stream (or from its own start stamp, if later) to its end. */
int subspec_profile_read(int32_t cls, int64_t *launches, double *total_ms, double *bytes);

#ifdef __cplusplus
}
#endif
#endif /* SUBSPEC_H */
