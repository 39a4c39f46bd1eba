// mla_decode_noalloc: mla_decode with its split partials in a static device
// array, for callers that cannot allocate (graph capture, serving loops,
// harnesses that forbid hipMalloc).  The array is a file-scope __device__
// object: in host code its name is only a stand-in, so its device address is
// taken once per device with hipGetSymbolAddress (with that device current) and
// that address is what the kernels receive.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/mla.h"

namespace {

constexpr size_t kScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// uninitialised (no bytes in the library file); each device holds its own copy
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's copy of the array, taken on the first
// call on that device.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_EHIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MLA_EHIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MLA_OK;
}

}  // namespace

extern "C" int mla_decode_noalloc(const mla_dims* dims, const void* q_lat, const void* q_pe, const void* cache,
                                  const int64_t* seq_start, const int32_t* seq_len, int32_t batch,
                                  int32_t max_len, const void* w_uv, void* out, void* stream) {
  // host-side checks first: nothing reaches the device for a call that is refused
  const int st = mla_check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 0) return MLA_EINVAL;
  if (batch == 0) return MLA_OK;
  if (max_len <= 0) return MLA_EINVAL;
  for (const void* ptr : {q_lat, q_pe, cache, static_cast<const void*>(seq_start), static_cast<const void*>(seq_len),
                          w_uv, static_cast<const void*>(out)})
    if (ptr == nullptr || (reinterpret_cast<uintptr_t>(ptr) & 15u) != 0) return MLA_EINVAL;
  const size_t need = mla_workspace_size(dims, MLA_OP_DECODE, batch, 0, max_len);
  if (need > kScratchBytes) return MLA_ESCRATCH;
  void* ws = nullptr;
  const int sa = scratch_address(&ws);
  if (sa != MLA_OK) return sa;
  // every partial the decode reads is written by its attention kernel first
  // (an empty split writes m = -inf, l = 0, o = 0), so nothing is cleared
  return mla_decode(dims, q_lat, q_pe, cache, seq_start, seq_len, batch, max_len, w_uv, out, ws,
                    kScratchBytes, stream);
}
