// Host side of libsubspec: argument validation, workspace carving and the
// launch sequence of each entry point declared in include/subspec.h.
//
// Workspace layout (every entry point): a fixed 64 KiB block of arrival
// counters at offset 0 (zero-filled once by subspec_workspace_init, left at
// zero by every kernel that uses it), followed by call-local scratch whose
// layout depends on the call (nothing in it survives between calls).
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <string>

#include "../../include/subspec.h"
#include "internal.h"
#include "profile.h"

// HBM read ceiling (stream.hip): *sink ^= XOR of the buffer's 32-bit words
hipError_t launch_hbm_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t s);

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return SUBSPEC_OK;
}

#define HIPCHK(expr)                                                                   \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess) return fail(SUBSPEC_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

constexpr size_t kCounterBytes = 64 * 1024;
constexpr size_t kSampleCounterOff = 16 * 1024;
constexpr size_t kRejectCounterOff = 16 * 1024 + 256;
constexpr size_t kRejectBatchCounterOff = 32 * 1024;  // batched rejection: one per element
constexpr int kMaxRejectBatch = 4096;                   // its counters fill [32 KiB, 48 KiB)
constexpr size_t kAttnCounterOff = 20 * 1024;  // draft attention: one per query head (<= 224)
constexpr size_t kControlCounterOff = 16 * 1024 + 512;  // draft-length controller
// draft step, QKV GEMV and attention in one launch: a count per 128-row group
// of the QKV output, one a 128-byte line, the give-up word in the last line,
// [48 KiB, 64 KiB)
constexpr size_t kQkvReadyOff = 48 * 1024;
static_assert(kQkvReadyOff + 4 * kReadyStride * kReadyLines == kCounterBytes, "ready lines");
static_assert(kQkvReadyOff + 4 * kReadyStride * (kReadyLines - 1) == SUBSPEC_WS_WAIT_FAULT_OFFSET, "give-up word");
constexpr int kMaxTokens = 64;
constexpr int kMaxTreeK = 16;       // chains of a static tree (rows of a draft level: the 4-bit GEMM's m)
constexpr int kMaxTreeD = 64;       // depth of a static tree
constexpr int kMaxTreeRows = 512;   // nodes of one tree's verify pass (1 + k D)
constexpr int kMaxGemvK = 28672;  // x (2 B) + half-group sums in 64 KiB of LDS
constexpr int kMaxGamma = 64;
constexpr int kMaxNormK = 6144;  // 3 items of 8 values per thread, 256 threads

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Carver {
  char* base;
  size_t off;
  void* take(size_t bytes) {
    void* p = base ? base + off : nullptr;
    off = align256(off + bytes);
    return p;
  }
};

hipStream_t hs(void* s) { return reinterpret_cast<hipStream_t>(s); }

// compute units of the current device (queried once)
int compute_units() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cus = n;
    else
      cus = 256;
  }
  return cus;
}

// ------------------------------------------------------------------ validation
bool lin_is_bf16(const subspec_linear& l) { return l.w && !l.codes && !l.meta; }
bool lin_is_w4(const subspec_linear& l) {  // any low-bit form (4, 3 or 2 bits)
  return !l.w && l.codes && l.meta && (l.bits == 0 || l.bits == 2 || l.bits == 3 || l.bits == 4);
}
// weight width the GEMV kernels take: 16 (bf16), 4, 3 or 2
int lin_bits(const subspec_linear& l) { return lin_is_w4(l) ? (l.bits == 0 ? 4 : l.bits) : 16; }
// bytes of one row of codes
double code_row_bytes(int bits, double k) { return bits == 4 ? k / 2 : (bits == 2 ? k / 4 : 3 * k / 8); }

// layout 1 (16-row tiles of subspec_tile_codes): 4- or 2-bit codes, n % 16 == 0,
// k a multiple of the width's chunk (128 or 256), k within the tiled GEMV's
// prologue (kMaxTiledK)
constexpr int64_t kMaxTiledK = 28672;
int check_layout(const subspec_linear& l, const char* what, int layer) {
  if (lin_is_bf16(l) || l.layout == 0) return SUBSPEC_OK;
  if (l.layout != 1) return fail(SUBSPEC_EINVAL, "layer %d %s: layout must be 0 or 1", layer, what);
  const int kch = tile_chunk_k(lin_bits(l));
  if (kch == 0) return fail(SUBSPEC_EINVAL, "layer %d %s: layout 1 needs 4- or 2-bit codes", layer, what);
  if (l.n % 16 != 0 || l.k % kch != 0 || l.k > kMaxTiledK)
    return fail(SUBSPEC_ESHAPE, "layer %d %s: layout 1 needs n %% 16 == 0, k %% %d == 0 and k <= %lld", layer, what,
                kch, (long long)kMaxTiledK);
  return SUBSPEC_OK;
}

int check_linear(const subspec_linear& l, int64_t n, int64_t k, bool allow_w4, const char* what,
                 int layer) {
  if (l.n != n || l.k != k)
    return fail(SUBSPEC_ESHAPE, "layer %d %s: shape [%lld][%lld], expected [%lld][%lld]", layer,
                what, (long long)l.n, (long long)l.k, (long long)n, (long long)k);
  if (lin_is_bf16(l)) return SUBSPEC_OK;
  if (allow_w4 && lin_is_w4(l)) {
    if (lin_bits(l) == 3 && k % 128 != 0)
      return fail(SUBSPEC_ESHAPE, "layer %d %s: 3-bit codes need k %% 128 == 0", layer, what);
    return check_layout(l, what, layer);
  }
  return fail(SUBSPEC_EINVAL, "layer %d %s: set exactly one of w (bf16)%s", layer, what,
              allow_w4 ? " or codes+meta with bits 4, 3 or 2" : "");
}

int check_model(const subspec_model* m) {
  if (!m) return fail(SUBSPEC_EINVAL, "model is NULL");
  if (m->n_layers < 1 || m->hidden <= 0 || m->ffn <= 0 || m->vocab <= 0 || m->n_q_heads <= 0 ||
      m->n_kv_heads <= 0)
    return fail(SUBSPEC_EINVAL, "model dimensions must be positive");
  if (m->head_dim != 128) return fail(SUBSPEC_EUNSUPPORTED, "head_dim must be 128");
  if (m->n_q_heads % m->n_kv_heads != 0)
    return fail(SUBSPEC_ESHAPE, "n_q_heads must be a multiple of n_kv_heads");
  if (m->n_q_heads / m->n_kv_heads > 8 || m->n_kv_heads > 1024)
    return fail(SUBSPEC_EUNSUPPORTED, "GQA group above 8 or more than 1024 kv heads");
  if (m->hidden % 128 != 0 || m->ffn % 128 != 0)
    return fail(SUBSPEC_ESHAPE, "hidden and ffn must be multiples of 128");
  if (m->hidden > kMaxGemvK || m->ffn > kMaxGemvK ||
      (int64_t)m->n_q_heads * m->head_dim > kMaxGemvK)
    return fail(SUBSPEC_EUNSUPPORTED, "GEMV input width above %d", kMaxGemvK);
  if (m->hidden > kMaxNormK)
    return fail(SUBSPEC_EUNSUPPORTED, "hidden above %d (norm-fused GEMV prologue)", kMaxNormK);
  if (m->vocab > (1 << 24)) return fail(SUBSPEC_EUNSUPPORTED, "vocab above 2^24");
  if (!(m->rms_eps > 0.0f) || !(m->rope_theta > 1.0f))
    return fail(SUBSPEC_EINVAL, "rms_eps must be > 0 and rope_theta > 1");
  if (!m->embed || !m->final_norm || !m->lm_head || !m->layers)
    return fail(SUBSPEC_EINVAL, "embed, final_norm, lm_head and layers must be set");
  const int64_t H = m->hidden, F = m->ffn, qd = (int64_t)m->n_q_heads * m->head_dim;
  const int64_t qkv = (int64_t)(m->n_q_heads + 2 * m->n_kv_heads) * m->head_dim;
  for (int l = 0; l < m->n_layers; ++l) {
    const subspec_layer& L = m->layers[l];
    if (!L.attn_norm || !L.ffn_norm) return fail(SUBSPEC_EINVAL, "layer %d: norm weights NULL", l);
    int r;
    if ((r = check_linear(L.qkv, qkv, H, false, "qkv", l)) ||
        (r = check_linear(L.o, H, qd, false, "o", l)) ||
        (r = check_linear(L.gate_up, 2 * F, H, false, "gate_up", l)) ||
        (r = check_linear(L.down, H, F, false, "down", l)) ||
        (r = check_linear(L.qkv_d, qkv, H, true, "qkv_d", l)) ||
        (r = check_linear(L.o_d, H, qd, true, "o_d", l)) ||
        (r = check_linear(L.gate_up_d, 2 * F, H, true, "gate_up_d", l)) ||
        (r = check_linear(L.down_d, H, F, true, "down_d", l)))
      return r;
  }
  return SUBSPEC_OK;
}

// Entries of every sparse index list at kv_len = L: min(L, max(ceil(budget
// * L), |sink| + |recent|)), non-decreasing in L.
int64_t index_count_of(int64_t L, int64_t n_sink, int64_t n_recent, int64_t budget_permille) {
  const int64_t sk = std::min<int64_t>(n_sink, L);
  const int64_t rec = std::min<int64_t>(n_recent, L - sk);
  const int64_t total = (budget_permille * L + 999) / 1000;
  return std::min<int64_t>(L, std::max<int64_t>(total, sk + rec));
}
int64_t index_count(int64_t L, const subspec_state* st) {
  return index_count_of(L, st->n_sink, st->n_recent, st->budget_permille);
}

int check_state(const subspec_model* m, const subspec_state* st) {
  if (!st) return fail(SUBSPEC_EINVAL, "state is NULL");
  if (!st->k_cache || !st->v_cache || !st->kv_len || !st->tokens)
    return fail(SUBSPEC_EINVAL, "state buffers k_cache, v_cache, kv_len, tokens must be set");
  if (st->capacity < 1) return fail(SUBSPEC_ECAPACITY, "capacity must be >= 1");
  if (st->kv_score || st->kv_index || st->use_index) {
    if (!st->kv_score || !st->kv_index || !st->kv_index_len)
      return fail(SUBSPEC_EINVAL, "sparse drafting needs kv_score, kv_index and kv_index_len");
    if (st->n_sink < 0 || st->n_recent < 0) return fail(SUBSPEC_EINVAL, "n_sink and n_recent must be >= 0");
    if (st->score_window < 1 || st->score_window > 16)
      return fail(SUBSPEC_EINVAL, "score_window must be in [1, 16]");
    if (st->budget_permille < 0 || st->budget_permille > 1000)
      return fail(SUBSPEC_EINVAL, "budget_permille must be in [0, 1000]");
    if (st->score_window * (m->n_q_heads / m->n_kv_heads) > attn_scores_max_pairs())
      return fail(SUBSPEC_EUNSUPPORTED, "score_window x GQA group above %d", attn_scores_max_pairs());
    const int64_t need = index_count(st->capacity, st);
    if (st->index_cap < need)
      return fail(SUBSPEC_ECAPACITY, "index_cap %d below the %lld entries of kv_len = capacity",
                  st->index_cap, (long long)need);
  }
  return SUBSPEC_OK;
}

// ------------------------------------------------------------------ layouts
struct FwdWs {
  uint32_t* sample_counter;
  uint32_t* attn_counters;
  uint32_t* qkv_ready;  // kReadyLines lines: the n_q + 2 n_kv counts, the give-up word last
  uint16_t *h, *xn, *qkv, *qrot, *attn, *act;
  uint16_t* gu;  // rows forward on 4-bit weights: gate/up outputs [mt][2F] before SiLU*up
  float* attn_part;
  int part_recs;  // partial records per query head in attn_part
  float* attn_ml;
  float* rope_cs;
  float* gemm_part;
  float* logit_max;
  int32_t* logit_arg;
  unsigned long long* sample_sums;
  int32_t* valid;
};

size_t max_gemm_partials(const subspec_model* m, int mt) {
  const int64_t H = m->hidden, F = m->ffn, qd = (int64_t)m->n_q_heads * m->head_dim;
  const int64_t qkv = (int64_t)(m->n_q_heads + 2 * m->n_kv_heads) * m->head_dim;
  size_t b = 0;
  b = std::max(b, gemm_partials_bytes(qkv, H, mt, GEPI_STORE));
  b = std::max(b, gemm_partials_bytes(H, qd, mt, GEPI_RESID));
  b = std::max(b, gemm_partials_bytes(F, H, mt, GEPI_SILU));
  b = std::max(b, gemm_partials_bytes(H, F, mt, GEPI_RESID));
  b = std::max(b, gemm_partials_bytes(m->vocab, H, mt, GEPI_STORE));
  if (mt <= 16) {  // a tree level's draft rows on 4-bit weights
    const int64_t shapes[4][2] = {{qkv, H}, {H, qd}, {2 * F, H}, {H, F}};
    for (const auto& sh : shapes)
      b = std::max(b, (size_t)gemm_w4_splits(sh[0], sh[1]) * mt * sh[0] * 4);
  }
  return b;
}

size_t carve_fwd(const subspec_model* m, int mt, int cap, void* ws, FwdWs* o) {
  Carver c{(char*)ws, 0};
  FwdWs w{};
  char* base = (char*)ws;
  w.sample_counter = base ? (uint32_t*)(base + kSampleCounterOff) : nullptr;
  w.attn_counters = base ? (uint32_t*)(base + kAttnCounterOff) : nullptr;
  w.qkv_ready = base ? (uint32_t*)(base + kQkvReadyOff) : nullptr;
  c.off = kCounterBytes;
  const int64_t H = m->hidden, F = m->ffn, qd = (int64_t)m->n_q_heads * m->head_dim;
  const int64_t qkv = (int64_t)(m->n_q_heads + 2 * m->n_kv_heads) * m->head_dim;
  w.h = (uint16_t*)c.take((size_t)mt * H * 2);
  w.xn = (uint16_t*)c.take((size_t)mt * H * 2);
  w.qkv = (uint16_t*)c.take((size_t)mt * qkv * 2);
  w.qrot = (uint16_t*)c.take((size_t)mt * qd * 2);
  w.attn = (uint16_t*)c.take((size_t)mt * qd * 2);
  w.act = (uint16_t*)c.take((size_t)mt * F * 2);
  w.gu = (uint16_t*)c.take((size_t)std::min(mt, 16) * 2 * F * 2);
  // attention split partials: verify [Hkv][ceil(cap/128)][mt][G][d + 4],
  // draft step [Hkv][ceil(cap/64)][G][d + 4]
  const size_t vsplits = (cap + decode_attn_keys_per_split() - 1) / decode_attn_keys_per_split();
  const size_t dsplits = (cap + draft_attn_keys_per_split() - 1) / draft_attn_keys_per_split();
  const size_t part_floats = (size_t)m->n_q_heads * std::max(vsplits * mt, dsplits) * (m->head_dim + 4);
  w.attn_part = (float*)c.take(part_floats * 4);
  w.part_recs = (int)std::max(vsplits * mt, dsplits);
  w.attn_ml = (float*)c.take((size_t)mt * m->n_q_heads * 2 * 4);
  w.rope_cs = (float*)c.take((size_t)mt * m->head_dim * 4);
  w.gemm_part = (float*)c.take(max_gemm_partials(m, mt));
  const int lm_blocks = gemv_max_blocks(false, m->vocab, EPI_LOGITS);
  w.logit_max = (float*)c.take((size_t)lm_blocks * 4);
  w.logit_arg = (int32_t*)c.take((size_t)lm_blocks * 4);
  w.sample_sums = (unsigned long long*)c.take(64 * 8);
  w.valid = (int32_t*)c.take(4);
  if (o) *o = w;
  return c.off;
}

struct RejWsL {
  RejectWs r;
};
size_t carve_reject(int gamma, int vocab, void* ws, RejectWs* o, int batch = 1) {
  Carver c{(char*)ws, kCounterBytes};
  const size_t C = (size_t)reject_chunks(vocab), rows = (size_t)(2 * gamma + 1), B = (size_t)batch;
  RejectWs r{};
  r.counter = ws ? (uint32_t*)((char*)ws + (batch > 1 ? kRejectBatchCounterOff : kRejectCounterOff)) : nullptr;
  r.row_max = (float*)c.take(B * rows * C * 4);
  r.row_arg = (int32_t*)c.take(B * rows * C * 4);
  r.row_bad = (int32_t*)c.take(B * rows * C * 4);
  r.row_sum = (unsigned long long*)c.take(B * rows * C * 8);
  r.res_sum = (unsigned long long*)c.take(B * C * 8);
  if (o) *o = r;
  return c.off;
}

// Static tree rejection: every chain's own round (batched, gamma = D - 1),
// their results, and the root's residual weights.
struct TreeRejWs {
  RejectWs r;
  int32_t* chain_n;
  int32_t* chain_out;
  int32_t* chain_status;
  unsigned long long* resid;
};
size_t carve_tree_reject(int k, int D, int vocab, void* ws, TreeRejWs* o) {
  TreeRejWs t{};
  size_t off = carve_reject(D - 1, vocab, ws, &t.r, k);
  Carver c{(char*)ws, off};
  t.chain_n = (int32_t*)c.take((size_t)k * 4);
  t.chain_out = (int32_t*)c.take((size_t)k * D * 4);
  t.chain_status = (int32_t*)c.take((size_t)k * 4);
  t.resid = (unsigned long long*)c.take((size_t)vocab * 8);
  if (o) *o = t;
  return c.off;
}

int need_ws(void* ws, size_t have, size_t need) {
  if (!ws) return fail(SUBSPEC_EWORKSPACE, "workspace is NULL");
  if (have < need)
    return fail(SUBSPEC_EWORKSPACE, "workspace of %zu bytes, %zu needed", have, need);
  return SUBSPEC_OK;
}

void set_linear(GemvArgs& a, const subspec_linear& l) {
  a.w = l.w;
  a.codes = l.codes;
  a.meta = l.meta;
  a.tiled = l.layout;
}

// Algorithmic bytes of one launch: weights, input, output (and residual)
// each counted once.
double gemv_bytes(const subspec_linear& l, int64_t n_out, bool resid) {
  const double n = (double)l.n, k = (double)l.k;
  const double wb = lin_is_w4(l) ? n * code_row_bytes(lin_bits(l), k) + n * (k / 64) * 4 : 2 * n * k;
  return wb + 2 * k + 2 * (double)n_out * (resid ? 2 : 1);
}
double gemm_bytes(int64_t n_phys, int64_t k, int m, int64_t n_out, bool resid) {
  return 2.0 * n_phys * k + 2.0 * m * k + 2.0 * m * n_out * (resid ? 2 : 1);
}
double gemm_w4_bytes(int64_t n_phys, int64_t k, int m, int64_t n_out, bool resid) {
  return (double)n_phys * k * (0.5 + 4.0 / 64) + 2.0 * m * k + 2.0 * m * n_out * (resid ? 2 : 1);
}
// site: 0 qkv, 1 o, 2 gate_up, 3 down
int gemv_class(const subspec_linear& l, int site) {
  return (lin_is_w4(l) ? SUBSPEC_K_W4_QKV : SUBSPEC_K_BF16_QKV) + site;
}

// Rows of one forward pass over the shared cache: the verify pass (gamma + 1
// or a prefill chunk of consecutive positions), a static tree's verify pass
// (all its nodes) and a tree's draft level (one node per chain, on the draft
// weights).  Row j takes the token tokens[j * tok_stride] and is node
// node0 + j * node_stride (AttnArgs: slot, position and visible keys).
struct RowsSpec {
  const int32_t* tokens;
  int tok_stride;
  int m;  // rows of each sequence
  int node0, node_stride, tree_d;
  // seqs > 1: a batch of sequences (subspec_batch_state), m rows each; the
  // token of row j of sequence z is tokens[z tok_seq_stride + j tok_stride]
  int seqs;
  int64_t tok_seq_stride;
  bool draft;        // draft weights: bf16 shared layers, 4-bit substitutes on the matrix cores (m <= 16)
  uint16_t* logits;  // [m][ld] or NULL
  int64_t ld;
};

// The cache, lengths and scores a row forward works on (one sequence's
// subspec_state, or a subspec_batch_state's sequences).
struct RowsCache {
  uint16_t *k_cache, *v_cache;
  int capacity;
  int32_t* kv_len;
  float* kv_score;  // importance scores (one sequence only) or NULL
  int score_window;
};
RowsCache rows_cache(const subspec_state* st) {
  return RowsCache{st->k_cache, st->v_cache, st->capacity, st->kv_len, st->kv_score, st->score_window};
}

int rows_forward(const subspec_model* m, const RowsCache& st, const RowsSpec& rs, void* ws, hipStream_t s) {
  const int nseq = rs.seqs > 1 ? rs.seqs : 1;
  const int mt = rs.m * nseq;  // rows of the whole launch
  FwdWs w;
  carve_fwd(m, mt, st.capacity, ws, &w);
  const int64_t H = m->hidden, F = m->ffn, d = m->head_dim;
  const int64_t qd = (int64_t)m->n_q_heads * d;
  const int64_t qkv = (int64_t)(m->n_q_heads + 2 * m->n_kv_heads) * d;
  const int rps = nseq > 1 ? rs.m : 0;
  {
    prof::Scope ps(SUBSPEC_K_MISC, 0.0, s);
    HIPCHK(launch_embed_rows(m->embed, rs.tokens, mt, (int)H, m->vocab, w.h, s, rs.tok_stride, rps,
                             rs.tok_seq_stride));
    HIPCHK(launch_rope_table(st.kv_len, rs.node0, rs.node_stride, rs.tree_d, mt, (int)d, m->rope_theta, w.rope_cs,
                             s, rps));
  }
  // Narrow GEMMs (QKV, O, down) split k over blocks and leave fp32 partial
  // sums; their consumers add them: RoPE for QKV, the residual + RMSNorm
  // kernel for O and down (h = bf16(h + sum), then the next norm).  The
  // 4-bit GEMM always leaves partials (also for one split).
  const float* pend = nullptr;  // partial sums still to be added to h
  int pend_splits = 0;
  auto norm_into_xn = [&](const uint16_t* g) -> hipError_t {
    const hipError_t e = launch_resid_rmsnorm_rows(w.h, pend, pend_splits, g, m->rms_eps, mt, (int)H, w.xn, s);
    pend = nullptr;
    pend_splits = 0;
    return e;
  };
  for (int l = 0; l < m->n_layers; ++l) {
    const subspec_layer& L = m->layers[l];
    const subspec_linear& lq = rs.draft ? L.qkv_d : L.qkv;
    const subspec_linear& lo = rs.draft ? L.o_d : L.o;
    const subspec_linear& lg = rs.draft ? L.gate_up_d : L.gate_up;
    const subspec_linear& ldn = rs.draft ? L.down_d : L.down;
    {
      prof::Scope ps(SUBSPEC_K_MISC, 0.0, s);
      HIPCHK(norm_into_xn(L.attn_norm));
    }
    int q_splits = 1;
    bool q_part = false;
    if (lin_is_w4(lq)) {
      prof::Scope ps(SUBSPEC_K_W4_QKV, gemm_w4_bytes(qkv, H, mt, qkv, false), s);
      HIPCHK(launch_gemm_w4(lq.codes, lq.meta, qkv, H, w.xn, mt, w.qkv, w.gemm_part, s, &q_splits, lq.layout));
      q_part = true;
    } else {
      GemmArgs q{lq.w, qkv, H, w.xn, mt, w.qkv, qkv, nullptr, w.gemm_part};
      prof::Scope ps(SUBSPEC_K_GEMM_QKV, gemm_bytes(qkv, H, mt, qkv, false), s);
      HIPCHK(launch_gemm(GEPI_STORE, q, s, &q_splits));
      q_part = q_splits > 1;
    }
    AttnArgs at{};
    at.qkv = w.qkv;
    if (q_part) {
      at.qkv_part = w.gemm_part;
      at.qkv_splits = q_splits;
    }
    at.q_rot = w.qrot;
    // layer l of the cache: [sequences][n_kv][capacity][d]
    at.k_cache = st.k_cache + (int64_t)l * nseq * m->n_kv_heads * st.capacity * d;
    at.v_cache = st.v_cache + (int64_t)l * nseq * m->n_kv_heads * st.capacity * d;
    at.kv_len = st.kv_len;
    at.pos_offset = rs.node0;
    at.row_stride = rs.node_stride;
    at.tree_d = rs.tree_d;
    at.m = rs.m;
    at.seqs = nseq;
    at.n_q = m->n_q_heads;
    at.n_kv = m->n_kv_heads;
    at.d = (int)d;
    at.cap = st.capacity;
    at.theta = m->rope_theta;
    at.rope_cs = w.rope_cs;
    at.part = w.attn_part;
    at.out = w.attn;
    at.split_keys = verify_attn_split_keys(st.capacity, m->n_kv_heads * nseq, rs.m * (m->n_q_heads / m->n_kv_heads));
    at.splits = (st.capacity + at.split_keys - 1) / at.split_keys;
    const bool scores = st.kv_score && !rs.draft && rs.tree_d == 0 && nseq == 1;
    if (scores) at.ml = w.attn_ml;
    {
      prof::Scope ps(SUBSPEC_K_ATTN_VERIFY, 0.0, s);
      HIPCHK(launch_rope_append(at, s));
      HIPCHK(launch_rows_attention(at, s));
    }
    if (scores) {
      prof::Scope ps(SUBSPEC_K_SCORES, 0.0, s);
      HIPCHK(launch_attn_scores(at, st.kv_score + (int64_t)l * m->n_kv_heads * st.capacity, st.score_window, s));
    }
    if (lin_is_w4(lo)) {
      prof::Scope ps(SUBSPEC_K_W4_O, gemm_w4_bytes(H, qd, mt, H, true), s);
      HIPCHK(launch_gemm_w4(lo.codes, lo.meta, H, qd, w.attn, mt, w.h, w.gemm_part, s, &pend_splits, lo.layout));
      pend = w.gemm_part;
    } else {
      GemmArgs o{lo.w, H, qd, w.attn, mt, w.h, H, w.h, w.gemm_part};
      prof::Scope ps(SUBSPEC_K_GEMM_O, gemm_bytes(H, qd, mt, H, true), s);
      HIPCHK(launch_gemm(GEPI_RESID, o, s, &pend_splits));
      if (pend_splits > 1) pend = w.gemm_part;
    }
    {
      prof::Scope ps(SUBSPEC_K_MISC, 0.0, s);
      HIPCHK(norm_into_xn(L.ffn_norm));
    }
    if (lin_is_w4(lg)) {
      prof::Scope ps(SUBSPEC_K_W4_GATE_UP, gemm_w4_bytes(2 * F, H, mt, F, false), s);
      if (gemm_w4_splits(2 * F, H) == 1) {  // SiLU * up in the GEMM's epilogue
        HIPCHK(launch_gemm_w4_silu(lg.codes, lg.meta, F, H, w.xn, mt, w.act, s, lg.layout));
      } else {
        HIPCHK(launch_gemm_w4(lg.codes, lg.meta, 2 * F, H, w.xn, mt, w.gu, w.gemm_part, s, nullptr, lg.layout));
        HIPCHK(launch_silu_rows(w.gu, F, mt, w.act, s));
      }
    } else {
      GemmArgs g{lg.w, F, H, w.xn, mt, w.act, F, nullptr, w.gemm_part};
      prof::Scope ps(SUBSPEC_K_GEMM_GATE_UP, gemm_bytes(2 * F, H, mt, F, false), s);
      HIPCHK(launch_gemm(GEPI_SILU, g, s, nullptr));
    }
    if (lin_is_w4(ldn)) {
      prof::Scope ps(SUBSPEC_K_W4_DOWN, gemm_w4_bytes(H, F, mt, H, true), s);
      HIPCHK(launch_gemm_w4(ldn.codes, ldn.meta, H, F, w.act, mt, w.h, w.gemm_part, s, &pend_splits, ldn.layout));
      pend = w.gemm_part;
    } else {
      GemmArgs dn{ldn.w, H, F, w.act, mt, w.h, H, w.h, w.gemm_part};
      prof::Scope ps(SUBSPEC_K_GEMM_DOWN, gemm_bytes(H, F, mt, H, true), s);
      HIPCHK(launch_gemm(GEPI_RESID, dn, s, &pend_splits));
      if (pend_splits > 1) pend = w.gemm_part;
    }
  }
  if (rs.logits) {
    {
      prof::Scope ps(SUBSPEC_K_MISC, 0.0, s);
      HIPCHK(norm_into_xn(m->final_norm));
    }
    GemmArgs lm{m->lm_head, m->vocab, H, w.xn, mt, rs.logits, rs.ld, nullptr, w.gemm_part};
    int lm_splits = 1;
    prof::Scope ps(SUBSPEC_K_GEMM_LM_HEAD, gemm_bytes(m->vocab, H, mt, m->vocab, false), s);
    HIPCHK(launch_gemm(GEPI_STORE, lm, s, &lm_splits));
    if (lm_splits > 1) HIPCHK(launch_gemm_reduce(w.gemm_part, lm_splits, mt, m->vocab, rs.logits, rs.ld, s));
  }
  return ok();
}

// 4-bit substitutes only (the draft rows' GEMM on the matrix cores)
int check_tree_draft_weights(const subspec_model* m) {
  for (int l = 0; l < m->n_layers; ++l) {
    const subspec_layer& L = m->layers[l];
    for (const subspec_linear* x : {&L.qkv_d, &L.o_d, &L.gate_up_d, &L.down_d})
      if (lin_is_w4(*x) && lin_bits(*x) != 4)
        return fail(SUBSPEC_EUNSUPPORTED, "layer %d: tree drafting takes bf16 or 4-bit draft weights", l);
  }
  return SUBSPEC_OK;
}

}  // namespace

// Error reporting for the entry points of other translation units.
int noalloc_fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}
int noalloc_ok() { return ok(); }

extern "C" {

int subspec_abi_version(void) { return SUBSPEC_ABI_VERSION; }

int64_t subspec_index_count(int64_t L, int32_t n_sink, int32_t n_recent, int32_t budget_permille) {
  if (L < 0 || n_sink < 0 || n_recent < 0 || budget_permille < 0 || budget_permille > 1000) {
    fail(SUBSPEC_EINVAL, "index_count: L, n_sink, n_recent must be >= 0 and budget_permille in [0, 1000]");
    return -1;
  }
  ok();
  return index_count_of(L, n_sink, n_recent, budget_permille);
}

const char* subspec_last_error(void) { return g_err.c_str(); }

size_t subspec_workspace_bytes(const subspec_model* m, int32_t max_tokens, int32_t capacity) {
  if (check_model(m)) return 0;
  if (max_tokens < 1 || max_tokens > kMaxTokens) {
    fail(SUBSPEC_EINVAL, "max_tokens must be in [1, %d]", kMaxTokens);
    return 0;
  }
  if (capacity < 1) {
    fail(SUBSPEC_ECAPACITY, "capacity must be >= 1");
    return 0;
  }
  size_t b = carve_fwd(m, max_tokens, capacity, nullptr, nullptr);
  b = std::max(b, carve_reject(kMaxGamma, m->vocab, nullptr, nullptr));
  b = std::max(b, kCounterBytes + (size_t)control_chunks(m->vocab) * 3 * sizeof(double));
  ok();
  return b;
}

int subspec_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws) return fail(SUBSPEC_EWORKSPACE, "workspace is NULL");
  if (ws_bytes < kCounterBytes) return fail(SUBSPEC_EWORKSPACE, "workspace below %zu bytes", kCounterBytes);
  HIPCHK(launch_zero(ws, ws_bytes & ~(size_t)15, hs(stream)));
  return ok();
}

int subspec_quantize(const uint16_t* w, int64_t n, int64_t k, int32_t group, int32_t bits,
                     uint8_t* codes, uint16_t* meta, void* stream) {
  if (!w || !codes || !meta) return fail(SUBSPEC_EINVAL, "w, codes and meta must be set");
  if (bits != 4 && bits != 3 && bits != 2) return fail(SUBSPEC_EUNSUPPORTED, "bits must be 4, 3 or 2");
  if (group != 64) return fail(SUBSPEC_EUNSUPPORTED, "only group = 64 is built");
  if (n < 1 || k < 1) return fail(SUBSPEC_EINVAL, "n and k must be positive");
  if (k % 64 != 0) return fail(SUBSPEC_ESHAPE, "k must be a multiple of 64");
  if (bits == 3 && k % 128 != 0) return fail(SUBSPEC_ESHAPE, "3-bit codes need k %% 128 == 0");
  HIPCHK(launch_quantize(w, n, k, bits, codes, meta, hs(stream)));
  return ok();
}

int subspec_tile_codes(const uint8_t* codes, const uint16_t* meta, int64_t n, int64_t k, int32_t bits,
                       uint8_t* tcodes, uint16_t* tmeta, void* stream) {
  if (!codes || !meta || !tcodes || !tmeta) return fail(SUBSPEC_EINVAL, "codes, meta, tcodes and tmeta must be set");
  if (n < 1 || k < 1) return fail(SUBSPEC_EINVAL, "n and k must be positive");
  const int kch = tile_chunk_k(bits);
  if (kch == 0) return fail(SUBSPEC_EUNSUPPORTED, "bits must be 4 or 2");
  if (n % 16 != 0 || k % kch != 0) return fail(SUBSPEC_ESHAPE, "n %% 16 == 0 and k %% %d == 0 needed", kch);
  HIPCHK(launch_tile_codes(codes, meta, n, k, bits, tcodes, tmeta, hs(stream)));
  return ok();
}

int subspec_draft_step(const subspec_model* m, const subspec_state* st, int32_t step,
                       float draft_temp, const uint32_t* u_codes, void* ws, size_t ws_bytes,
                       void* stream) {
  int r;
  if ((r = check_model(m)) || (r = check_state(m, st))) return r;
  if (!st->draft_logits) return fail(SUBSPEC_EINVAL, "state.draft_logits must be set");
  if (step < 0 || step >= st->gamma_max)
    return fail(SUBSPEC_EINVAL, "step %d outside [0, gamma_max = %d)", step, st->gamma_max);
  if (!(draft_temp >= 0.0f)) return fail(SUBSPEC_EINVAL, "draft_temp must be >= 0");
  if (draft_temp > 0.0f && !u_codes) return fail(SUBSPEC_EINVAL, "u_codes needed when draft_temp > 0");
  if ((r = need_ws(ws, ws_bytes, carve_fwd(m, 1, st->capacity, nullptr, nullptr)))) return r;
  FwdWs w;
  carve_fwd(m, 1, st->capacity, ws, &w);
  hipStream_t s = hs(stream);
  const int64_t H = m->hidden, F = m->ffn, d = m->head_dim;
  const int64_t qd = (int64_t)m->n_q_heads * d;
  const int64_t qkv = (int64_t)(m->n_q_heads + 2 * m->n_kv_heads) * d;
  int32_t* tok_out = st->tokens + step + 1;
  const bool sparse = st->use_index != 0;
  {
    prof::Scope ps(SUBSPEC_K_MISC, 0.0, s);
    HIPCHK(launch_pos_guard(st->kv_len, st->tokens + step, step, st->capacity, m->vocab, w.valid, tok_out,
                            (int)d, m->rope_theta, w.rope_cs, st->draft_len, s));
  }
  for (int l = 0; l < m->n_layers; ++l) {
    const subspec_layer& L = m->layers[l];
    GemvArgs a{};
    set_linear(a, L.qkv_d);
    a.n = qkv;
    a.k = H;
    a.h = w.h;
    a.norm_w = L.attn_norm;
    a.eps = m->rms_eps;
    a.embed = m->embed;
    a.token = st->tokens + step;
    a.vocab = m->vocab;
    a.h_out = w.h;
    a.y = w.qkv;
    a.valid = w.valid;
    const int qkv_pro = l == 0 ? PRO_EMBED_NORM : PRO_NORM;

    AttnArgs at{};
    at.qkv = w.qkv;
    at.q_rot = w.qrot;
    at.k_cache = st->k_cache + (int64_t)l * m->n_kv_heads * st->capacity * d;
    at.v_cache = st->v_cache + (int64_t)l * m->n_kv_heads * st->capacity * d;
    at.kv_len = st->kv_len;
    at.pos_offset = step;
    at.m = 1;
    at.n_q = m->n_q_heads;
    at.n_kv = m->n_kv_heads;
    at.d = (int)d;
    at.cap = st->capacity;
    at.theta = m->rope_theta;
    at.rope_cs = w.rope_cs;
    at.part = w.attn_part;
    at.out = w.attn;
    const int kpb = draft_attn_keys_per_split();
    at.splits = (st->capacity + kpb - 1) / kpb;
    if (sparse) {
      at.index = st->kv_index + (int64_t)l * m->n_kv_heads * st->index_cap;
      at.n_index = st->kv_index_len;
      at.index_cap = st->index_cap;
      // slots: n_index + step + 1 <= min(index_cap + gamma_max, capacity)
      at.splits = std::min(at.splits, (st->index_cap + st->gamma_max + kpb - 1) / kpb);
    }
    // keys of this launch: at most the capacity (dense), or the index plus the
    // speculative positions (sparse)
    at.max_keys = sparse ? std::min(st->capacity, st->index_cap + st->gamma_max) : st->capacity;
    // and no more blocks than compute units: a compute unit holding two of
    // them doubles the launch's critical path (at the 32B shape, 40 heads:
    // 8 splits 17.0 us a layer, 6 splits 12.8)
    at.head_splits = std::min(std::min(draft_head_splits(at.max_keys), w.part_recs),
                              std::max(1, compute_units() / std::max(1, m->n_q_heads)));
    at.counters = w.attn_counters;

    // the attention inside the QKV launch: low-bit tiled QKV weights, dense
    // keys, at most two 16-key chunks a wave
    const int ring = draft_head_ring(at);
    const bool fused = !st->attn_own_launch && !sparse && a.tiled && (ring == 1 || ring == 2) &&
                       m->n_q_heads + 2 * m->n_kv_heads < kReadyLines &&
                       qkv_attn_supported(lin_bits(L.qkv_d), qkv_pro, qkv, H);
    if (fused) {
      prof::Scope ps(SUBSPEC_K_QKV_ATTN, gemv_bytes(L.qkv_d, qkv, false), s);
      HIPCHK(launch_qkv_attn(lin_bits(L.qkv_d), qkv_pro, a, at, ring, w.qkv_ready, s));
    } else {
      {
        prof::Scope ps(gemv_class(L.qkv_d, 0), gemv_bytes(L.qkv_d, qkv, false), s);
        HIPCHK(launch_gemv(lin_bits(L.qkv_d), qkv_pro, EPI_STORE, a, s, nullptr));
      }
      {
        prof::Scope ps(SUBSPEC_K_ATTN_DRAFT, 0.0, s);
        HIPCHK(launch_decode_attention(at, w.valid, s));
      }
    }

    GemvArgs o{};
    set_linear(o, L.o_d);
    o.n = H;
    o.k = qd;
    o.y = w.h;
    o.resid = w.h;
    o.valid = w.valid;
    o.x = w.attn;
    {
      prof::Scope ps(gemv_class(L.o_d, 1), gemv_bytes(L.o_d, H, true), s);
      HIPCHK(launch_gemv(lin_bits(L.o_d), PRO_X, EPI_RESID, o, s, nullptr));
    }

    GemvArgs g{};
    set_linear(g, L.gate_up_d);
    g.n = F;
    g.k = H;
    g.h = w.h;
    g.norm_w = L.ffn_norm;
    g.eps = m->rms_eps;
    g.y = w.act;
    g.valid = w.valid;
    {
      prof::Scope ps(gemv_class(L.gate_up_d, 2), gemv_bytes(L.gate_up_d, F, false), s);
      HIPCHK(launch_gemv(lin_bits(L.gate_up_d), PRO_NORM, EPI_SILU, g, s, nullptr));
    }

    GemvArgs dn{};
    set_linear(dn, L.down_d);
    dn.n = H;
    dn.k = F;
    dn.x = w.act;
    dn.y = w.h;
    dn.resid = w.h;
    dn.valid = w.valid;
    {
      prof::Scope ps(gemv_class(L.down_d, 3), gemv_bytes(L.down_d, H, true), s);
      HIPCHK(launch_gemv(lin_bits(L.down_d), PRO_X, EPI_RESID, dn, s, nullptr));
    }
  }
  uint16_t* logits = st->draft_logits + (int64_t)step * m->vocab;
  GemvArgs lm{};
  lm.w = m->lm_head;
  lm.n = m->vocab;
  lm.k = H;
  lm.h = w.h;
  lm.norm_w = m->final_norm;
  lm.eps = m->rms_eps;
  lm.y = logits;
  lm.part_max = w.logit_max;
  lm.part_arg = w.logit_arg;
  lm.valid = w.valid;
  int lm_blocks = 0;
  {
    const subspec_linear lml{m->lm_head, nullptr, nullptr, m->vocab, H};
    prof::Scope ps(SUBSPEC_K_LM_HEAD, gemv_bytes(lml, m->vocab, false), s);
    HIPCHK(launch_gemv(16, PRO_NORM, EPI_LOGITS, lm, s, &lm_blocks));
  }
  SampleWs sw{w.logit_max, w.logit_arg, w.sample_sums, w.sample_counter};
  {
    prof::Scope ps(SUBSPEC_K_SAMPLE, 2.0 * m->vocab, s);
    HIPCHK(launch_sample(logits, m->vocab, draft_temp, u_codes ? u_codes + step : nullptr, w.logit_max,
                         w.logit_arg, lm_blocks, tok_out, w.valid, sw, s));
  }
  return ok();
}

int subspec_verify(const subspec_model* m, const subspec_state* st, int32_t n_tokens,
                   const int32_t* tokens, uint16_t* logits, void* ws, size_t ws_bytes, void* stream) {
  int r;
  if ((r = check_model(m)) || (r = check_state(m, st))) return r;
  if (!tokens) return fail(SUBSPEC_EINVAL, "tokens is NULL");
  if (n_tokens < 1 || n_tokens > kMaxTokens)
    return fail(SUBSPEC_EINVAL, "n_tokens %d outside [1, %d]", n_tokens, kMaxTokens);
  if (n_tokens > st->capacity) return fail(SUBSPEC_ECAPACITY, "n_tokens above the KV capacity");
  if ((r = need_ws(ws, ws_bytes, carve_fwd(m, n_tokens, st->capacity, nullptr, nullptr)))) return r;
  RowsSpec rs{};
  rs.tokens = tokens;
  rs.tok_stride = 1;
  rs.m = n_tokens;
  rs.node0 = 0;
  rs.node_stride = 1;
  rs.tree_d = 0;
  rs.draft = false;
  rs.logits = logits;
  rs.ld = m->vocab;
  return rows_forward(m, rows_cache(st), rs, ws, hs(stream));
}

int subspec_draft_verify(const subspec_model* m, const subspec_state* st, int32_t pos_offset, int32_t n_tokens,
                         const int32_t* tokens, uint16_t* logits, void* ws, size_t ws_bytes, void* stream) {
  int r;
  if ((r = check_model(m)) || (r = check_state(m, st)) || (r = check_tree_draft_weights(m))) return r;
  if (!tokens) return fail(SUBSPEC_EINVAL, "tokens is NULL");
  if (n_tokens < 1 || n_tokens > 16) return fail(SUBSPEC_EINVAL, "n_tokens %d outside [1, 16]", n_tokens);
  if (pos_offset < 0 || pos_offset + n_tokens > st->capacity)
    return fail(SUBSPEC_ECAPACITY, "positions past the KV capacity");
  if ((r = need_ws(ws, ws_bytes, carve_fwd(m, n_tokens, st->capacity, nullptr, nullptr)))) return r;
  RowsSpec rs{};
  rs.tokens = tokens;
  rs.tok_stride = 1;
  rs.m = n_tokens;
  rs.node0 = pos_offset;
  rs.node_stride = 1;
  rs.tree_d = 0;
  rs.draft = true;
  rs.logits = logits;
  rs.ld = m->vocab;
  return rows_forward(m, rows_cache(st), rs, ws, hs(stream));
}

int subspec_draft_append(const subspec_state* st, int32_t at, int32_t max_n, const int32_t* n_accepted,
                         const int32_t* out_tokens, void* stream) {
  if (!st || !st->tokens || !n_accepted || !out_tokens) return fail(SUBSPEC_EINVAL, "NULL buffer");
  if (at < 0 || max_n < 0 || at + max_n > st->gamma_max)
    return fail(SUBSPEC_EINVAL, "at %d + max_n %d outside the tokens buffer (gamma_max %d)", at, max_n, st->gamma_max);
  HIPCHK(launch_token_append(st->tokens + at, max_n, n_accepted, out_tokens, hs(stream)));
  return ok();
}

constexpr int kMaxBatch = 16;
constexpr int kMaxRowsVocab = 524288;  // vocabulary of the one-block-per-row samplers (64 chunks of 8192)

static int check_batch(const subspec_model* m, const subspec_batch_state* st) {
  if (!st) return fail(SUBSPEC_EINVAL, "batch state is NULL");
  if (!st->k_cache || !st->v_cache || !st->kv_len || !st->tokens)
    return fail(SUBSPEC_EINVAL, "batch state buffers k_cache, v_cache, kv_len, tokens must be set");
  if (st->batch < 1 || st->batch > kMaxBatch) return fail(SUBSPEC_EINVAL, "batch %d outside [1, %d]", st->batch, kMaxBatch);
  if (st->capacity < 1) return fail(SUBSPEC_ECAPACITY, "capacity must be >= 1");
  if (st->gamma_max < 0 || st->gamma_max > kMaxGamma)
    return fail(SUBSPEC_EINVAL, "gamma_max %d outside [0, %d]", st->gamma_max, kMaxGamma);
  (void)m;
  return SUBSPEC_OK;
}

static RowsCache batch_cache(const subspec_batch_state* st) {
  return RowsCache{st->k_cache, st->v_cache, st->capacity, st->kv_len, nullptr, 0};
}

size_t subspec_batch_workspace_bytes(const subspec_model* m, int32_t batch, int32_t max_tokens, int32_t capacity) {
  if (check_model(m)) return 0;
  if (batch < 1 || batch > kMaxBatch || max_tokens < 1 || max_tokens > kMaxTokens ||
      batch * max_tokens > kMaxTreeRows) {
    fail(SUBSPEC_EINVAL, "batch in [1, %d], max_tokens in [1, %d], batch x max_tokens <= %d", kMaxBatch, kMaxTokens,
         kMaxTreeRows);
    return 0;
  }
  if (capacity < 1) {
    fail(SUBSPEC_ECAPACITY, "capacity must be >= 1");
    return 0;
  }
  size_t b = carve_fwd(m, batch * max_tokens, capacity, nullptr, nullptr);
  b = std::max(b, carve_fwd(m, batch, capacity, nullptr, nullptr));
  b = std::max(b, carve_reject(max_tokens - 1, m->vocab, nullptr, nullptr, batch));
  ok();
  return b;
}

int subspec_batch_draft_step(const subspec_model* m, const subspec_batch_state* st, int32_t step, float draft_temp,
                             const uint32_t* u_codes, void* ws, size_t ws_bytes, void* stream) {
  int r;
  if ((r = check_model(m)) || (r = check_batch(m, st)) || (r = check_tree_draft_weights(m))) return r;
  if (m->vocab > kMaxRowsVocab) return fail(SUBSPEC_EUNSUPPORTED, "vocab above %d", kMaxRowsVocab);
  if (!st->draft_logits) return fail(SUBSPEC_EINVAL, "batch state draft_logits must be set");
  if (step < 0 || step >= st->gamma_max)
    return fail(SUBSPEC_EINVAL, "step %d outside [0, gamma_max = %d)", step, st->gamma_max);
  if (!(draft_temp >= 0.0f)) return fail(SUBSPEC_EINVAL, "draft_temp must be >= 0");
  if (draft_temp > 0.0f && !u_codes) return fail(SUBSPEC_EINVAL, "u_codes needed when draft_temp > 0");
  if ((r = need_ws(ws, ws_bytes, carve_fwd(m, st->batch, st->capacity, nullptr, nullptr)))) return r;
  if (st->batch == 1) {
    // one sequence: its buffers are a single-sequence state's, and the
    // single-sequence draft step (fused GEMVs, per-head split attention)
    // computes the same row
    subspec_state one{};
    one.k_cache = st->k_cache;
    one.v_cache = st->v_cache;
    one.capacity = st->capacity;
    one.kv_len = st->kv_len;
    one.tokens = st->tokens;
    one.draft_logits = st->draft_logits;
    one.gamma_max = st->gamma_max;
    return subspec_draft_step(m, &one, step, draft_temp, u_codes, ws, ws_bytes, stream);
  }
  hipStream_t s = hs(stream);
  const int64_t ldt = st->gamma_max + 1;
  RowsSpec rs{};
  rs.tokens = st->tokens + step;  // row b: tokens[b][step]
  rs.tok_stride = 1;
  rs.m = 1;
  rs.seqs = st->batch;
  rs.tok_seq_stride = ldt;
  rs.node0 = step;
  rs.node_stride = 1;
  rs.draft = true;
  rs.logits = st->draft_logits + (int64_t)step * m->vocab;  // row b: draft_logits[b][step]
  rs.ld = (int64_t)st->gamma_max * m->vocab;
  if ((r = rows_forward(m, batch_cache(st), rs, ws, s))) return r;
  RowsSampleArgs sa{};
  sa.logits = rs.logits;
  sa.ld = rs.ld;
  sa.V = m->vocab;
  sa.T = draft_temp;
  sa.u = u_codes ? u_codes + step : nullptr;
  sa.u_row = st->gamma_max;
  sa.tokens = st->tokens + step + 1;
  sa.t_row = ldt;
  sa.nout = 1;
  sa.kv_len = st->kv_len;
  sa.kv_row = 1;
  sa.need = step + 1;  // position kv_len + step inside the cache
  sa.cap = st->capacity;
  prof::Scope ps(SUBSPEC_K_SAMPLE, 2.0 * st->batch * m->vocab, s);
  HIPCHK(launch_rows_sample(sa, st->batch, s));
  return ok();
}

int subspec_batch_verify(const subspec_model* m, const subspec_batch_state* st, int32_t n_tokens,
                         const int32_t* tokens, int64_t ld_tokens, uint16_t* logits, void* ws, size_t ws_bytes,
                         void* stream) {
  int r;
  if ((r = check_model(m)) || (r = check_batch(m, st))) return r;
  if (!tokens) return fail(SUBSPEC_EINVAL, "tokens is NULL");
  if (n_tokens < 1 || n_tokens > kMaxTokens || st->batch * n_tokens > kMaxTreeRows)
    return fail(SUBSPEC_EINVAL, "n_tokens %d outside [1, %d] or batch x n_tokens above %d", n_tokens, kMaxTokens,
                kMaxTreeRows);
  if (ld_tokens < n_tokens) return fail(SUBSPEC_EINVAL, "ld_tokens below n_tokens");
  if (n_tokens > st->capacity) return fail(SUBSPEC_ECAPACITY, "n_tokens above the KV capacity");
  if ((r = need_ws(ws, ws_bytes, carve_fwd(m, st->batch * n_tokens, st->capacity, nullptr, nullptr)))) return r;
  RowsSpec rs{};
  rs.tokens = tokens;
  rs.tok_stride = 1;
  rs.m = n_tokens;
  rs.seqs = st->batch;
  rs.tok_seq_stride = ld_tokens;
  rs.node0 = 0;
  rs.node_stride = 1;
  rs.draft = false;
  rs.logits = logits;
  rs.ld = m->vocab;
  return rows_forward(m, batch_cache(st), rs, ws, hs(stream));
}

int subspec_batch_reject(const subspec_model* m, const subspec_batch_state* st, float temp, float draft_temp,
                         const uint16_t* target_logits, const uint32_t* r_codes, const uint32_t* u_codes,
                         int32_t* n_accepted, int32_t* out_tokens, int32_t* status, void* ws, size_t ws_bytes,
                         void* stream) {
  int r;
  if ((r = check_model(m)) || (r = check_batch(m, st))) return r;
  if (!target_logits || !st->draft_logits || !n_accepted || !out_tokens || !status)
    return fail(SUBSPEC_EINVAL, "NULL buffer");
  if (!(temp >= 0.0f) || !(draft_temp >= 0.0f)) return fail(SUBSPEC_EINVAL, "temperatures must be >= 0");
  if (temp > 0.0f && (!r_codes || !u_codes)) return fail(SUBSPEC_EINVAL, "r_codes and u_codes needed when temp > 0");
  const int gamma = st->gamma_max;
  RejectWs w;
  if ((r = need_ws(ws, ws_bytes, carve_reject(gamma, m->vocab, nullptr, nullptr, st->batch)))) return r;
  carve_reject(gamma, m->vocab, ws, &w, st->batch);
  hipStream_t s = hs(stream);
  prof::Scope ps(SUBSPEC_K_REJECT, 0.0, s);
  HIPCHK(launch_reject(gamma, m->vocab, temp, draft_temp, target_logits, st->draft_logits, st->tokens + 1, r_codes,
                       u_codes, n_accepted, out_tokens, status, nullptr, w, s, nullptr, st->batch, gamma + 1, gamma,
                       1));
  return ok();
}

int subspec_batch_rollback(const subspec_batch_state* st, const int32_t* n_accepted, const int32_t* out_tokens,
                           int32_t delta, void* stream) {
  int r;
  if ((r = check_batch(nullptr, st))) return r;
  if (n_accepted && !out_tokens) return fail(SUBSPEC_EINVAL, "out_tokens is NULL");
  HIPCHK(launch_batch_rollback(st->kv_len, st->tokens, st->gamma_max + 1, n_accepted, out_tokens,
                               st->gamma_max + 1, st->batch, delta, hs(stream)));
  return ok();
}

static int check_tree(int32_t k, int32_t D) {
  if (k < 1 || k > kMaxTreeK) return fail(SUBSPEC_EINVAL, "tree width k = %d outside [1, %d]", k, kMaxTreeK);
  if (D < 1 || D > kMaxTreeD) return fail(SUBSPEC_EINVAL, "tree depth %d outside [1, %d]", D, kMaxTreeD);
  if (1 + k * D > kMaxTreeRows)
    return fail(SUBSPEC_EINVAL, "tree of %d nodes above %d", 1 + k * D, kMaxTreeRows);
  return SUBSPEC_OK;
}

size_t subspec_tree_workspace_bytes(const subspec_model* m, int32_t k, int32_t depth, int32_t capacity) {
  if (check_model(m) || check_tree(k, depth)) return 0;
  if (capacity < 1) {
    fail(SUBSPEC_ECAPACITY, "capacity must be >= 1");
    return 0;
  }
  size_t b = carve_fwd(m, 1 + k * depth, capacity, nullptr, nullptr);
  b = std::max(b, carve_fwd(m, k, capacity, nullptr, nullptr));
  b = std::max(b, carve_tree_reject(k, depth, m->vocab, nullptr, nullptr));
  ok();
  return b;
}

int subspec_tree_draft(const subspec_model* m, const subspec_state* st, int32_t k, int32_t depth, int32_t level,
                       float draft_temp, const uint32_t* u_codes, void* ws, size_t ws_bytes, void* stream) {
  int r;
  if ((r = check_model(m)) || (r = check_state(m, st)) || (r = check_tree(k, depth)) ||
      (r = check_tree_draft_weights(m)))
    return r;
  if (m->vocab > kMaxRowsVocab) return fail(SUBSPEC_EUNSUPPORTED, "vocab above %d", kMaxRowsVocab);
  if (!st->draft_logits) return fail(SUBSPEC_EINVAL, "state.draft_logits must be set");
  if (level < 0 || level >= depth) return fail(SUBSPEC_EINVAL, "level %d outside [0, depth = %d)", level, depth);
  if (!(draft_temp >= 0.0f)) return fail(SUBSPEC_EINVAL, "draft_temp must be >= 0");
  if (draft_temp > 0.0f && !u_codes) return fail(SUBSPEC_EINVAL, "u_codes needed when draft_temp > 0");
  if (1 + k * depth > st->capacity) return fail(SUBSPEC_ECAPACITY, "a tree of %d nodes above the KV capacity", 1 + k * depth);
  const int rows = level == 0 ? 1 : k;
  if ((r = need_ws(ws, ws_bytes, carve_fwd(m, rows, st->capacity, nullptr, nullptr)))) return r;
  hipStream_t s = hs(stream);
  RowsSpec rs{};
  rs.m = rows;
  rs.draft = true;
  rs.tree_d = depth;
  if (level == 0) {  // the root
    rs.tokens = st->tokens;
    rs.tok_stride = 1;
    rs.node0 = 0;
    rs.node_stride = 1;
    rs.logits = st->draft_logits;
    rs.ld = m->vocab;
  } else {  // depth `level` of every chain: nodes level + c D, draft rows level + c (D - 1)
    rs.tokens = st->tokens + level;
    rs.tok_stride = depth;
    rs.node0 = level;
    rs.node_stride = depth;
    rs.logits = st->draft_logits + (int64_t)level * m->vocab;
    rs.ld = (int64_t)(depth - 1) * m->vocab;
  }
  if (level == 0 && !st->use_index && !st->draft_len) {
    // the root is one row: the single-sequence draft step (fused GEMVs)
    // writes its K/V at slot kv_len and its logits in draft_logits row 0;
    // its own argmax in tokens[1] is replaced by the root's children below
    if ((r = subspec_draft_step(m, st, 0, 0.0f, nullptr, ws, ws_bytes, stream))) return r;
  } else if ((r = rows_forward(m, rows_cache(st), rs, ws, s))) {
    return r;
  }
  {
    prof::Scope ps(SUBSPEC_K_SAMPLE, 2.0 * rows * m->vocab, s);
    RowsSampleArgs sa{};
    sa.logits = rs.logits;
    sa.ld = rs.ld;
    sa.V = m->vocab;
    sa.T = draft_temp;
    sa.kv_len = st->kv_len;
    sa.kv_row = 0;
    sa.need = 1 + k * depth;  // the whole tree must fit
    sa.cap = st->capacity;
    if (level == 0) {  // the root's k children: tokens[1 + c D], draws u[c]
      sa.nout = k;
      sa.tokens = st->tokens + 1;
      sa.t_out = depth;
      sa.u = u_codes;
      sa.u_out = 1;
    } else {  // chain c's next token tokens[1 + c D + level], draw u[k + c (D - 1) + level - 1]
      sa.nout = 1;
      sa.tokens = st->tokens + 1 + level;
      sa.t_row = depth;
      sa.u = u_codes ? u_codes + k + level - 1 : nullptr;
      sa.u_row = depth - 1;
    }
    HIPCHK(launch_rows_sample(sa, rows, s));
  }
  return ok();
}

int subspec_tree_verify(const subspec_model* m, const subspec_state* st, int32_t k, int32_t depth, uint16_t* logits,
                        void* ws, size_t ws_bytes, void* stream) {
  int r;
  if ((r = check_model(m)) || (r = check_state(m, st)) || (r = check_tree(k, depth))) return r;
  if (!logits) return fail(SUBSPEC_EINVAL, "logits is NULL");
  const int n = 1 + k * depth;
  if (n > st->capacity) return fail(SUBSPEC_ECAPACITY, "a tree of %d nodes above the KV capacity", n);
  if ((r = need_ws(ws, ws_bytes, carve_fwd(m, n, st->capacity, nullptr, nullptr)))) return r;
  RowsSpec rs{};
  rs.tokens = st->tokens;
  rs.tok_stride = 1;
  rs.m = n;
  rs.node0 = 0;
  rs.node_stride = 1;
  rs.tree_d = depth;
  rs.draft = false;
  rs.logits = logits;
  rs.ld = m->vocab;
  return rows_forward(m, rows_cache(st), rs, ws, hs(stream));
}

int subspec_tree_reject(int32_t k, int32_t depth, int32_t vocab, float temp, float draft_temp,
                        const uint16_t* target_logits, const uint16_t* draft_logits, const int32_t* tokens,
                        const uint32_t* r_codes, const uint32_t* u_code, int32_t* n_accepted, int32_t* chain,
                        int32_t* out_tokens, int32_t* status, void* ws, size_t ws_bytes, void* stream) {
  int r;
  if ((r = check_tree(k, depth))) return r;
  if (vocab < 1 || vocab > kMaxRowsVocab) return fail(SUBSPEC_EINVAL, "vocab outside [1, %d]", kMaxRowsVocab);
  if (!(temp >= 0.0f) || !(draft_temp >= 0.0f)) return fail(SUBSPEC_EINVAL, "temperatures must be >= 0");
  if (!target_logits || !draft_logits || !tokens || !n_accepted || !chain || !out_tokens || !status)
    return fail(SUBSPEC_EINVAL, "NULL buffer");
  if (temp > 0.0f && (!r_codes || !u_code)) return fail(SUBSPEC_EINVAL, "r_codes and u_code needed when temp > 0");
  TreeRejWs t;
  if ((r = need_ws(ws, ws_bytes, carve_tree_reject(k, depth, vocab, nullptr, nullptr)))) return r;
  carve_tree_reject(k, depth, vocab, ws, &t);
  hipStream_t s = hs(stream);
  prof::Scope ps(SUBSPEC_K_REJECT, 0.0, s);
  // every chain's own round over its depth-1..D target rows and depth-1..D-1
  // draft rows (the draft tokens of depths 2..D), sharing r_codes[k..] and u
  HIPCHK(launch_reject(depth - 1, vocab, temp, draft_temp, target_logits + vocab, draft_logits + vocab, tokens + 2,
                       r_codes ? r_codes + k : nullptr, u_code, t.chain_n, t.chain_out, t.chain_status, nullptr, t.r,
                       s, nullptr, k, depth, 0, 0));
  HIPCHK(launch_tree_root(target_logits, draft_logits, vocab, temp, draft_temp, tokens, k, depth, r_codes, u_code,
                          t.chain_n, t.chain_out, t.chain_status, t.resid, n_accepted, chain, out_tokens, status, s));
  return ok();
}

int subspec_tree_commit(const subspec_model* m, const subspec_state* st, int32_t k, int32_t depth,
                        const int32_t* n_accepted, const int32_t* chain, const int32_t* out_tokens, void* stream) {
  int r;
  if ((r = check_model(m)) || (r = check_state(m, st)) || (r = check_tree(k, depth))) return r;
  if (!n_accepted || !chain || !out_tokens) return fail(SUBSPEC_EINVAL, "NULL buffer");
  hipStream_t s = hs(stream);
  prof::Scope ps(SUBSPEC_K_MISC, 0.0, s);
  HIPCHK(launch_tree_commit(st->k_cache, st->v_cache, m->n_layers * m->n_kv_heads, st->capacity, m->head_dim,
                            st->kv_len, n_accepted, chain, depth, s));
  HIPCHK(launch_kv_rollback(st->kv_len, st->tokens, n_accepted, out_tokens, s));
  return ok();
}

int subspec_reject_len(int32_t gamma, int32_t vocab, float temp, float draft_temp,
                       const uint16_t* target_logits, const uint16_t* draft_logits,
                       const int32_t* draft_tokens, const uint32_t* r_codes, const uint32_t* u_code,
                       const int32_t* gamma_len, int32_t* n_accepted, int32_t* out_tokens, int32_t* status,
                       float* probs, void* ws, size_t ws_bytes, void* stream) {
  if (gamma < 0 || gamma > kMaxGamma) return fail(SUBSPEC_EINVAL, "gamma outside [0, %d]", kMaxGamma);
  if (vocab < 1 || vocab > (1 << 24)) return fail(SUBSPEC_EINVAL, "vocab outside [1, 2^24]");
  if (!(temp >= 0.0f) || !(draft_temp >= 0.0f)) return fail(SUBSPEC_EINVAL, "temperatures must be >= 0");
  if (!target_logits || !n_accepted || !out_tokens || !status)
    return fail(SUBSPEC_EINVAL, "target_logits, n_accepted, out_tokens and status must be set");
  if (gamma > 0 && (!draft_logits || !draft_tokens))
    return fail(SUBSPEC_EINVAL, "draft_logits and draft_tokens must be set when gamma > 0");
  if (temp > 0.0f && (!u_code || (gamma > 0 && !r_codes)))
    return fail(SUBSPEC_EINVAL, "r_codes and u_code must be set when temp > 0");
  int r;
  if ((r = need_ws(ws, ws_bytes, carve_reject(gamma, vocab, nullptr, nullptr)))) return r;
  RejectWs rw;
  carve_reject(gamma, vocab, ws, &rw);
  prof::Scope ps(SUBSPEC_K_REJECT, 2.0 * (2 * gamma + 1) * vocab, hs(stream));
  HIPCHK(launch_reject(gamma, vocab, temp, draft_temp, target_logits, draft_logits, draft_tokens,
                       r_codes, u_code, n_accepted, out_tokens, status, probs, rw, hs(stream), gamma_len));
  return ok();
}

int subspec_reject(int32_t gamma, int32_t vocab, float temp, float draft_temp,
                   const uint16_t* target_logits, const uint16_t* draft_logits,
                   const int32_t* draft_tokens, const uint32_t* r_codes, const uint32_t* u_code,
                   int32_t* n_accepted, int32_t* out_tokens, int32_t* status, float* probs,
                   void* ws, size_t ws_bytes, void* stream) {
  return subspec_reject_len(gamma, vocab, temp, draft_temp, target_logits, draft_logits, draft_tokens, r_codes,
                            u_code, nullptr, n_accepted, out_tokens, status, probs, ws, ws_bytes, stream);
}

size_t subspec_reject_workspace_bytes(int32_t batch, int32_t gamma, int32_t vocab) {
  if (batch < 1 || batch > kMaxRejectBatch || gamma < 0 || gamma > kMaxGamma || vocab < 1 || vocab > (1 << 24)) {
    fail(SUBSPEC_EINVAL, "batch in [1, %d], gamma in [0, %d], vocab in [1, 2^24]", kMaxRejectBatch, kMaxGamma);
    return 0;
  }
  ok();
  return carve_reject(gamma, vocab, nullptr, nullptr, batch);
}

int subspec_reject_batch(int32_t batch, int32_t gamma, int32_t vocab, float temp, float draft_temp,
                         const uint16_t* target_logits, const uint16_t* draft_logits, const int32_t* draft_tokens,
                         const uint32_t* r_codes, const uint32_t* u_codes, const int32_t* gamma_len,
                         int32_t* n_accepted, int32_t* out_tokens, int32_t* status, float* probs, void* ws,
                         size_t ws_bytes, void* stream) {
  if (batch < 1 || batch > kMaxRejectBatch) return fail(SUBSPEC_EINVAL, "batch outside [1, %d]", kMaxRejectBatch);
  if (gamma < 0 || gamma > kMaxGamma) return fail(SUBSPEC_EINVAL, "gamma outside [0, %d]", kMaxGamma);
  if (vocab < 1 || vocab > (1 << 24)) return fail(SUBSPEC_EINVAL, "vocab outside [1, 2^24]");
  if (!(temp >= 0.0f) || !(draft_temp >= 0.0f)) return fail(SUBSPEC_EINVAL, "temperatures must be >= 0");
  if (!target_logits || !n_accepted || !out_tokens || !status)
    return fail(SUBSPEC_EINVAL, "target_logits, n_accepted, out_tokens and status must be set");
  if (gamma > 0 && (!draft_logits || !draft_tokens))
    return fail(SUBSPEC_EINVAL, "draft_logits and draft_tokens must be set when gamma > 0");
  if (temp > 0.0f && (!u_codes || (gamma > 0 && !r_codes)))
    return fail(SUBSPEC_EINVAL, "r_codes and u_codes must be set when temp > 0");
  int r;
  if ((r = need_ws(ws, ws_bytes, carve_reject(gamma, vocab, nullptr, nullptr, batch)))) return r;
  RejectWs rw;
  carve_reject(gamma, vocab, ws, &rw, batch);
  prof::Scope ps(SUBSPEC_K_REJECT, 2.0 * batch * (2 * gamma + 1) * vocab, hs(stream));
  HIPCHK(launch_reject(gamma, vocab, temp, draft_temp, target_logits, draft_logits, draft_tokens, r_codes, u_codes,
                       n_accepted, out_tokens, status, probs, rw, hs(stream), gamma_len, batch));
  return ok();
}

int subspec_kv_rollback(const subspec_state* st, const int32_t* n_accepted,
                        const int32_t* out_tokens, void* stream) {
  if (!st || !st->kv_len || !st->tokens) return fail(SUBSPEC_EINVAL, "state kv_len/tokens NULL");
  if (!n_accepted || !out_tokens) return fail(SUBSPEC_EINVAL, "n_accepted and out_tokens must be set");
  prof::Scope ps(SUBSPEC_K_MISC, 0.0, hs(stream));
  HIPCHK(launch_kv_rollback(st->kv_len, st->tokens, n_accepted, out_tokens, hs(stream)));
  return ok();
}

int subspec_kv_select(const subspec_model* m, const subspec_state* st, void* stream) {
  int r;
  if ((r = check_model(m)) || (r = check_state(m, st))) return r;
  if (!st->kv_score || !st->kv_index || !st->kv_index_len)
    return fail(SUBSPEC_EINVAL, "kv_score, kv_index and kv_index_len must be set");
  prof::Scope ps(SUBSPEC_K_SELECT, 0.0, hs(stream));
  HIPCHK(launch_kv_select(st->kv_score, st->capacity, st->kv_len, m->n_layers * m->n_kv_heads, st->n_sink,
                          st->n_recent, st->budget_permille, st->kv_index, st->index_cap, st->kv_index_len,
                          hs(stream)));
  return ok();
}

static int control_args(const subspec_control* ctl, ControlArgs* o) {
  if (!ctl || !ctl->draft_len || !ctl->state || !ctl->entropy)
    return fail(SUBSPEC_EINVAL, "control: draft_len, state and entropy must be set");
  if (ctl->gamma_max < 1 || ctl->gamma_max > kMaxGamma)
    return fail(SUBSPEC_EINVAL, "control: gamma_max outside [1, %d]", kMaxGamma);
  if (!(ctl->c > 0.0) || !(ctl->beta > 0.0 && ctl->beta <= 1.0))
    return fail(SUBSPEC_EINVAL, "control: c must be > 0 and beta in (0, 1]");
  *o = ControlArgs{ctl->draft_len, ctl->state, ctl->entropy, ctl->c, ctl->beta, ctl->gamma_max};
  return SUBSPEC_OK;
}

int subspec_control_init(const subspec_control* ctl, void* stream) {
  ControlArgs c;
  int r;
  if ((r = control_args(ctl, &c))) return r;
  HIPCHK(launch_control_init(c, hs(stream)));
  return ok();
}

int subspec_draft_control(const subspec_model* m, const subspec_state* st, int32_t step,
                          const subspec_control* ctl, void* ws, size_t ws_bytes, void* stream) {
  ControlArgs c;
  int r;
  if ((r = check_model(m)) || (r = check_state(m, st)) || (r = control_args(ctl, &c))) return r;
  if (!st->draft_logits) return fail(SUBSPEC_EINVAL, "state.draft_logits must be set");
  if (st->draft_len != ctl->draft_len)
    return fail(SUBSPEC_EINVAL, "state.draft_len must be the controller's draft_len");
  if (ctl->gamma_max > st->gamma_max) return fail(SUBSPEC_EINVAL, "control gamma_max above the state's");
  if (step < 0 || step >= ctl->gamma_max)
    return fail(SUBSPEC_EINVAL, "step %d outside [0, gamma_max = %d)", step, ctl->gamma_max);
  const size_t part_bytes = (size_t)control_chunks(m->vocab) * 3 * sizeof(double);
  if ((r = need_ws(ws, ws_bytes, kCounterBytes + part_bytes))) return r;
  char* base = (char*)ws;
  prof::Scope ps(SUBSPEC_K_SAMPLE, 2.0 * m->vocab, hs(stream));
  HIPCHK(launch_draft_control(c, step, st->draft_logits + (int64_t)step * m->vocab, m->vocab,
                              (double*)(base + kCounterBytes), (uint32_t*)(base + kControlCounterOff),
                              hs(stream)));
  return ok();
}

int subspec_control_update(const subspec_control* ctl, const int32_t* n_accepted, void* stream) {
  ControlArgs c;
  int r;
  if ((r = control_args(ctl, &c))) return r;
  if (!n_accepted) return fail(SUBSPEC_EINVAL, "n_accepted must be set");
  prof::Scope ps(SUBSPEC_K_MISC, 0.0, hs(stream));
  HIPCHK(launch_control_update(c, n_accepted, hs(stream)));
  return ok();
}

int subspec_kv_advance(const subspec_state* st, int32_t delta, void* stream) {
  if (!st || !st->kv_len) return fail(SUBSPEC_EINVAL, "state kv_len NULL");
  HIPCHK(launch_kv_advance(st->kv_len, delta, hs(stream)));
  return ok();
}

int subspec_w4_gemv(const uint8_t* codes, const uint16_t* meta, int64_t n, int64_t k,
                    const uint16_t* x, uint16_t* y, void* stream) {
  if (!codes || !meta || !x || !y) return fail(SUBSPEC_EINVAL, "codes, meta, x and y must be set");
  if (n < 1 || k < 1) return fail(SUBSPEC_EINVAL, "n and k must be positive");
  if (k % 64 != 0) return fail(SUBSPEC_ESHAPE, "k must be a multiple of 64");
  if (k > kMaxGemvK) return fail(SUBSPEC_EUNSUPPORTED, "k above %d", kMaxGemvK);
  GemvArgs a{};
  a.codes = codes;
  a.meta = meta;
  a.n = n;
  a.k = k;
  a.x = x;
  a.y = y;
  HIPCHK(launch_gemv(4, PRO_X, EPI_STORE, a, hs(stream), nullptr));
  return ok();
}

int subspec_gemv(const subspec_linear* w, const uint16_t* x, const uint16_t* norm_w, float eps,
                 int32_t epilogue, const uint16_t* resid, uint16_t* y, void* stream) {
  if (!w || !x || !y) return fail(SUBSPEC_EINVAL, "w, x and y must be set");
  if (!lin_is_bf16(*w) && !lin_is_w4(*w))
    return fail(SUBSPEC_EINVAL, "set exactly one of w (bf16) or codes+meta with bits 4, 3 or 2");
  if (w->n < 1 || w->k < 1) return fail(SUBSPEC_EINVAL, "n and k must be positive");
  if (w->k % 64 != 0) return fail(SUBSPEC_ESHAPE, "k must be a multiple of 64");
  if (lin_bits(*w) == 3 && w->k % 128 != 0) return fail(SUBSPEC_ESHAPE, "3-bit codes need k %% 128 == 0");
  if (w->k > kMaxGemvK) return fail(SUBSPEC_EUNSUPPORTED, "k above %d", kMaxGemvK);
  if (norm_w && w->k > kMaxNormK) return fail(SUBSPEC_EUNSUPPORTED, "k above %d with norm_w", kMaxNormK);
  if (epilogue < 0 || epilogue > 2) return fail(SUBSPEC_EINVAL, "epilogue must be 0, 1 or 2");
  if (epilogue == 1 && !resid) return fail(SUBSPEC_EINVAL, "resid must be set for epilogue 1");
  if (epilogue == 2 && w->n % 2 != 0) return fail(SUBSPEC_ESHAPE, "epilogue 2 needs an even row count");
  if (norm_w && !(eps >= 0.0f)) return fail(SUBSPEC_EINVAL, "eps must be >= 0");
  int r;
  if ((r = check_layout(*w, "w", -1))) return r;
  if (lin_is_w4(*w) && w->layout == 1 && epilogue == 2 && (w->n / 2) % 16 != 0)
    return fail(SUBSPEC_ESHAPE, "layout 1 with epilogue 2 needs n %% 32 == 0");
  GemvArgs a{};
  set_linear(a, *w);
  a.n = epilogue == 2 ? w->n / 2 : w->n;
  a.k = w->k;
  a.x = x;
  a.h = x;
  a.norm_w = norm_w;
  a.eps = eps;
  a.resid = resid;
  a.y = y;
  const int epi = epilogue == 0 ? EPI_STORE : epilogue == 1 ? EPI_RESID : EPI_SILU;
  const int pro = norm_w ? PRO_NORM : PRO_X;
  if (pro == PRO_X && epi == EPI_SILU)
    return fail(SUBSPEC_EUNSUPPORTED, "epilogue 2 is fused with the norm prologue only");
  if (pro == PRO_NORM && epi == EPI_RESID)
    return fail(SUBSPEC_EUNSUPPORTED, "epilogue 1 is fused with the plain prologue only");
  HIPCHK(launch_gemv(lin_bits(*w), pro, epi, a, hs(stream), nullptr));
  return ok();
}

size_t subspec_w4_gemm_workspace_bytes(int64_t n, int64_t k, int32_t m) {
  if (n < 1 || k < 128 || k % 128 != 0 || m < 1 || m > 16) {
    fail(SUBSPEC_EINVAL, "n >= 1, k a positive multiple of 128, 1 <= m <= 16");
    return 0;
  }
  ok();
  return kCounterBytes + (size_t)gemm_w4_splits(n, k) * m * n * 4;
}

int subspec_w4_gemm(const subspec_linear* w, const uint16_t* x, int32_t m, uint16_t* y, void* ws, size_t ws_bytes,
                    void* stream) {
  if (!w || !x || !y) return fail(SUBSPEC_EINVAL, "w, x and y must be set");
  if (!lin_is_w4(*w) || lin_bits(*w) != 4) return fail(SUBSPEC_EINVAL, "w must be 4-bit codes + meta");
  if (w->n < 1 || w->k < 1) return fail(SUBSPEC_EINVAL, "n and k must be positive");
  if (w->k % 128 != 0) return fail(SUBSPEC_ESHAPE, "k must be a multiple of 128");
  if (m < 1 || m > 16) return fail(SUBSPEC_EINVAL, "m outside [1, 16]");
  int r;
  if ((r = check_layout(*w, "w", -1))) return r;
  if ((r = need_ws(ws, ws_bytes, kCounterBytes + (size_t)gemm_w4_splits(w->n, w->k) * m * w->n * 4))) return r;
  prof::Scope ps(SUBSPEC_K_W4_GATE_UP, w->n * code_row_bytes(4, (double)w->k) + w->n * (w->k / 64) * 4.0 +
                 2.0 * m * (w->k + w->n), hs(stream));
  HIPCHK(launch_gemm_w4(w->codes, w->meta, w->n, w->k, x, m, y, (float*)((char*)ws + kCounterBytes), hs(stream),
                        nullptr, w->layout));
  return ok();
}

int subspec_bf16_gemv(const uint16_t* w, int64_t n, int64_t k, const uint16_t* x, uint16_t* y,
                      void* stream) {
  if (!w || !x || !y) return fail(SUBSPEC_EINVAL, "w, x and y must be set");
  if (n < 1 || k < 1) return fail(SUBSPEC_EINVAL, "n and k must be positive");
  if (k % 8 != 0) return fail(SUBSPEC_ESHAPE, "k must be a multiple of 8");
  if (k > kMaxGemvK) return fail(SUBSPEC_EUNSUPPORTED, "k above %d", kMaxGemvK);
  GemvArgs a{};
  a.w = w;
  a.n = n;
  a.k = k;
  a.x = x;
  a.y = y;
  HIPCHK(launch_gemv(16, PRO_X, EPI_STORE, a, hs(stream), nullptr));
  return ok();
}

int subspec_bf16_gemm(const uint16_t* w, int64_t n, int64_t k, const uint16_t* x, int32_t m,
                      uint16_t* y, void* ws, size_t ws_bytes, void* stream) {
  if (!w || !x || !y) return fail(SUBSPEC_EINVAL, "w, x and y must be set");
  if (n < 1 || k < 1) return fail(SUBSPEC_EINVAL, "n and k must be positive");
  if (m < 1 || m > kMaxTreeRows) return fail(SUBSPEC_EINVAL, "m outside [1, %d]", kMaxTreeRows);
  if (k % 128 != 0) return fail(SUBSPEC_ESHAPE, "k must be a multiple of 128");
  const size_t need = kCounterBytes + align256(gemm_partials_bytes(n, k, m, GEPI_STORE));
  int r;
  if ((r = need_ws(ws, ws_bytes, need))) return r;
  float* part = (float*)((char*)ws + kCounterBytes);
  GemmArgs a{w, n, k, x, m, y, n, nullptr, part};
  int splits = 1;
  HIPCHK(launch_gemm(GEPI_STORE, a, hs(stream), &splits));
  if (splits > 1) HIPCHK(launch_gemm_reduce(part, splits, m, n, y, n, hs(stream)));
  return ok();
}

int subspec_sample(const uint16_t* logits, int32_t vocab, float temp, const uint32_t* u_code,
                   int32_t* token, void* ws, size_t ws_bytes, void* stream) {
  if (!logits || !token) return fail(SUBSPEC_EINVAL, "logits and token must be set");
  if (vocab < 1 || vocab > (1 << 24)) return fail(SUBSPEC_EINVAL, "vocab outside [1, 2^24]");
  if (!(temp >= 0.0f)) return fail(SUBSPEC_EINVAL, "temp must be >= 0");
  if (temp > 0.0f && !u_code) return fail(SUBSPEC_EINVAL, "u_code needed when temp > 0");
  const int nc = sample_chunks(vocab);
  Carver c{(char*)ws, kCounterBytes};
  float* pm = (float*)c.take(nc * 4);
  int32_t* pa = (int32_t*)c.take(nc * 4);
  unsigned long long* sums = (unsigned long long*)c.take(64 * 8);
  int r;
  if ((r = need_ws(ws, ws_bytes, c.off))) return r;
  hipStream_t s = hs(stream);
  HIPCHK(launch_rowmax(logits, vocab, pm, pa, nc, s));
  SampleWs sw{pm, pa, sums, (uint32_t*)((char*)ws + kSampleCounterOff)};
  HIPCHK(launch_sample(logits, vocab, temp, u_code, pm, pa, nc, token, nullptr, sw, s));
  return ok();
}

int subspec_hbm_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink) return fail(SUBSPEC_EINVAL, "buf and sink must be set");
  if (bytes < 16 || bytes % 16 != 0) return fail(SUBSPEC_ESHAPE, "bytes must be a positive multiple of 16");
  if (reinterpret_cast<uintptr_t>(buf) % 16 != 0) return fail(SUBSPEC_EINVAL, "buf must be 16-byte aligned");
  HIPCHK(launch_hbm_read(buf, bytes, sink, hs(stream)));
  return ok();
}

}  // extern "C"
