// HBM read ceiling: the rate at which a plain streaming read of a large
// buffer runs on this GPU.  The draft GEMVs and the verify GEMMs are bound by
// streaming weights from HBM ("How speculative decoding makes LLMs go brrr",
// Module 2), so their rates are also reported against this measured ceiling,
// not only against the 8 TB/s datasheet figure.
//
// Each block reads one contiguous region, 32 KiB at a time (a wave load is a
// contiguous 1 KiB), through a buffer resource that covers exactly the region
// (reads past its end return zeros, so every load is unconditional).  Two
// register slots of eight 16-byte loads per lane alternate: one slot's loads
// are in flight while the other is folded.  The fold is a XOR of every 32-bit
// word; a wave adds its word into *sink with one atomic XOR, so *sink ends
// XORed with every word of the buffer, whatever the order (zeros are
// neutral), which a test can check.
#include "common.h"

namespace {

typedef __amdgpu_buffer_rsrc_t Res;
constexpr int kBufferWord3 = 0x00020000;  // buffer resource word 3 (CDNA): raw 32-bit data
constexpr int kNonTemporal = 2;           // buffer load cache policy: nt (streamed once)
constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;                                       // loads per lane and slot
constexpr int64_t kSlotBytes = (int64_t)kReadThreads * 16 * kReadUnroll;  // 32 KiB

struct Slot {
  u32x4 v[kReadUnroll];
};

__device__ __forceinline__ void load_slot(Slot& s, Res r, int64_t slot, int tid) {
#pragma unroll
  for (int j = 0; j < kReadUnroll; ++j)
    s.v[j] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(slot * kSlotBytes) + 16 * (j * kReadThreads + tid), 0,
                                                   kNonTemporal);
}

__device__ __forceinline__ uint32_t fold_slot(const Slot& s, uint32_t acc) {
#pragma unroll
  for (int j = 0; j < kReadUnroll; ++j) acc ^= s.v[j].x ^ s.v[j].y ^ s.v[j].z ^ s.v[j].w;
  return acc;
}

__global__ __launch_bounds__(kReadThreads) void hbm_read_kernel(const uint8_t* p, int64_t bytes, int64_t per_block,
                                                                 uint32_t* sink) {
  const int tid = threadIdx.x;
  const int64_t start = (int64_t)blockIdx.x * per_block;
  const int64_t len = bytes - start < per_block ? bytes - start : per_block;  // > 0: the grid covers bytes
  const Res r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p) + start, 0, (int)len, kBufferWord3);
  const int64_t n_slots = (len + kSlotBytes - 1) / kSlotBytes;
  uint32_t acc = 0;
  Slot a, b;
  load_slot(a, r, 0, tid);
  int64_t s = 0;
  for (; s + 2 < n_slots; s += 2) {
    load_slot(b, r, s + 1, tid);
    acc = fold_slot(a, acc);
    load_slot(a, r, s + 2, tid);
    acc = fold_slot(b, acc);
  }
  if (s + 2 == n_slots) {
    load_slot(b, r, s + 1, tid);
    acc = fold_slot(a, acc);
    acc = fold_slot(b, acc);
  } else {
    acc = fold_slot(a, acc);
  }
#pragma unroll
  for (int o = SS_WAVE / 2; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, SS_WAVE);
  if ((tid & (SS_WAVE - 1)) == 0) atomicXor(sink, acc);
}

}  // namespace

hipError_t launch_hbm_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t s) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  // one block per compute unit, each a region of whole 32 KiB slots (below
  // 2 GiB, the reach of a buffer offset); fewer blocks for small buffers.  Over
  // 4 GiB this read 6.8 TB/s; 2, 3, 4 and 8 blocks per compute unit read 6.7,
  // 6.5, 6.3 and 6.0 TB/s (more requests in flight, lower DRAM efficiency),
  // and 16 loads per lane and slot instead of 8 changed nothing.
  const int64_t slots = (bytes + kSlotBytes - 1) / kSlotBytes;
  int64_t blocks = (int64_t)cus;
  int64_t per_slots = (slots + blocks - 1) / blocks;
  const int64_t max_slots = ((int64_t)1 << 31) / kSlotBytes - 1;
  if (per_slots > max_slots) per_slots = max_slots;
  blocks = (slots + per_slots - 1) / per_slots;
  hipLaunchKernelGGL(hbm_read_kernel, dim3((unsigned)blocks), dim3(kReadThreads), 0, s,
                     reinterpret_cast<const uint8_t*>(buf), bytes, per_slots * kSlotBytes, sink);
  return hipGetLastError();
}
