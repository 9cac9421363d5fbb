// subspec_reject_noalloc: the rejection round with its scratch (per-row
// partial maxima, argmaxima, flags and fixed-point sums, the residual chunk
// sums and the arrival counter) in a file-scope device array instead of a
// caller workspace, for callers that cannot allocate device memory (code
// under graph capture, tight serving loops).  The kernels are the ones
// subspec_reject launches; only where their scratch lives differs.
//
// The array is one per GPU and lives until the process ends.  Host code never
// passes its name to a kernel: the name is a host-side stand-in, not a device
// address.  The device address comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that address is used.
#include <mutex>

#include "../../include/subspec.h"
#include "internal.h"
#include "profile.h"

namespace {

constexpr size_t kScratchBytes = size_t(1) << 20;  // 1 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

// Layout of one call: the 256-byte counter block first, then the row arrays.
size_t layout(int gamma, int vocab, char* base, RejectWs* o) {
  const size_t C = (size_t)reject_chunks(vocab), rows = (size_t)(2 * gamma + 1);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off = up256(off + bytes);
    return p;
  };
  RejectWs r{};
  r.counter = (uint32_t*)take(256);
  r.row_max = (float*)take(rows * C * 4);
  r.row_arg = (int32_t*)take(rows * C * 4);
  r.row_bad = (int32_t*)take(rows * C * 4);
  r.row_sum = (unsigned long long*)take(rows * C * 8);
  r.res_sum = (unsigned long long*)take(C * 8);
  if (o) *o = r;
  return off;
}

// Device address of this GPU's array (looked up once per device).
hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

int noalloc_fail(int code, const char* fmt, ...);  // api.hip: sets subspec_last_error
int noalloc_ok();

extern "C" int subspec_reject_noalloc(int32_t gamma, int32_t vocab, float temp, float draft_temp,
                                      const uint16_t* target_logits, const uint16_t* draft_logits,
                                      const int32_t* draft_tokens, const uint32_t* r_codes,
                                      const uint32_t* u_code, int32_t* n_accepted, int32_t* out_tokens,
                                      int32_t* status, float* probs, void* stream) {
  if (gamma < 0 || gamma > 64) return noalloc_fail(SUBSPEC_EINVAL, "gamma outside [0, 64]");
  if (vocab < 1 || vocab > (1 << 24)) return noalloc_fail(SUBSPEC_EINVAL, "vocab outside [1, 2^24]");
  if (!(temp >= 0.0f) || !(draft_temp >= 0.0f))
    return noalloc_fail(SUBSPEC_EINVAL, "temperatures must be >= 0");
  if (!target_logits || !n_accepted || !out_tokens || !status)
    return noalloc_fail(SUBSPEC_EINVAL, "target_logits, n_accepted, out_tokens and status must be set");
  if (gamma > 0 && (!draft_logits || !draft_tokens))
    return noalloc_fail(SUBSPEC_EINVAL, "draft_logits and draft_tokens must be set when gamma > 0");
  if (temp > 0.0f && (!u_code || (gamma > 0 && !r_codes)))
    return noalloc_fail(SUBSPEC_EINVAL, "r_codes and u_code must be set when temp > 0");
  const size_t need = layout(gamma, vocab, nullptr, nullptr);
  if (need > kScratchBytes)
    return noalloc_fail(SUBSPEC_ECAPACITY,
                        "gamma %d x vocab %d needs %zu bytes of scratch; the static scratch holds %zu "
                        "((2 gamma + 1) x ceil(vocab / 4096) x 20 bytes plus 1 KiB must fit)",
                        gamma, vocab, need, kScratchBytes);
  void* base = nullptr;
  hipError_t e = scratch_ptr(&base);
  if (e != hipSuccess)
    return noalloc_fail(SUBSPEC_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
  RejectWs rw;
  layout(gamma, vocab, (char*)base, &rw);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  prof::Scope ps(SUBSPEC_K_REJECT, 2.0 * (2 * gamma + 1) * vocab, s);
  // the arrival counter must start at zero: cleared by a fill kernel (no
  // memset node), whatever an earlier call left there
  e = launch_zero(rw.counter, 256, s);
  if (e == hipSuccess)
    e = launch_reject(gamma, vocab, temp, draft_temp, target_logits, draft_logits, draft_tokens, r_codes,
                      u_code, n_accepted, out_tokens, status, probs, rw, s);
  if (e != hipSuccess) return noalloc_fail(SUBSPEC_EHIP, "launch_reject: %s", hipGetErrorString(e));
  return noalloc_ok();
}
