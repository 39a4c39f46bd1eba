// Host-side range checks of the device index arrays (lengths, segment offsets,
// cache slots), on host copies.  The release calls never read device contents;
// a library built with MLA_DEBUG_CHECKS copies the arrays to the host before
// every decode, prefill and cache-write call and refuses bad ones here.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "../../include/mla.h"
#include "mla_internal.h"

extern "C" int mla_check_decode_rows(const int64_t* seq_start, const int32_t* seq_len, int32_t batch,
                                     int32_t max_len, int64_t cache_rows) {
  if (batch < 0 || (batch > 0 && (seq_start == nullptr || seq_len == nullptr)) || cache_rows < 0) return MLA_EINVAL;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t n = seq_len[b], s0 = seq_start[b];
    if (n < 1 || n > max_len || s0 < 0 || s0 > cache_rows - n) return MLA_EINVAL;
  }
  return MLA_OK;
}

extern "C" int mla_check_prefill_rows(const int64_t* cu_seqlens, int32_t batch, int64_t n_tokens,
                                      int32_t max_len, int64_t cache_rows) {
  if (batch < 0 || n_tokens < 0 || cache_rows < 0 || cu_seqlens == nullptr) return MLA_EINVAL;
  if (cu_seqlens[0] != 0 || cu_seqlens[batch] != n_tokens || n_tokens > cache_rows) return MLA_EINVAL;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t len = cu_seqlens[b + 1] - cu_seqlens[b];
    if (len < 0 || len > max_len) return MLA_EINVAL;
  }
  return MLA_OK;
}

extern "C" int mla_check_write_rows(const int64_t* slots, int64_t n_tokens, int64_t cache_rows) {
  if (n_tokens < 0 || cache_rows < 0 || (n_tokens > 0 && slots == nullptr)) return MLA_EINVAL;
  std::vector<int64_t> s(slots, slots + n_tokens);
  for (const int64_t v : s)
    if (v < 0 || v >= cache_rows) return MLA_EINVAL;
  std::sort(s.begin(), s.end());
  return std::adjacent_find(s.begin(), s.end()) == s.end() ? MLA_OK : MLA_EINVAL;
}

namespace mla {

// Debug builds: copy a device array to the host (synchronising) for the checks.
template <typename T>
static int to_host(const T* dev, int64_t n, std::vector<T>* out) {
  out->resize(static_cast<size_t>(n));
  if (n == 0) return MLA_OK;
  return hipMemcpy(out->data(), dev, sizeof(T) * static_cast<size_t>(n), hipMemcpyDeviceToHost) == hipSuccess
             ? MLA_OK
             : MLA_EHIP;
}

int debug_check_decode(const int64_t* seq_start, const int32_t* seq_len, int32_t batch, int32_t max_len) {
  if (!kDebugChecks) return MLA_OK;
  std::vector<int64_t> s;
  std::vector<int32_t> l;
  int st = to_host(seq_start, batch, &s);
  if (st == MLA_OK) st = to_host(seq_len, batch, &l);
  return st == MLA_OK ? mla_check_decode_rows(s.data(), l.data(), batch, max_len, INT64_MAX) : st;
}

int debug_check_prefill(const int64_t* cu_seqlens, int32_t batch, int64_t n_tokens, int32_t max_len) {
  if (!kDebugChecks) return MLA_OK;
  std::vector<int64_t> cu;
  const int st = to_host(cu_seqlens, static_cast<int64_t>(batch) + 1, &cu);
  return st == MLA_OK ? mla_check_prefill_rows(cu.data(), batch, n_tokens, max_len, INT64_MAX) : st;
}

int debug_check_write(const int64_t* slots, int64_t n_tokens, int64_t cache_rows) {
  if (!kDebugChecks) return MLA_OK;
  std::vector<int64_t> s;
  const int st = to_host(slots, n_tokens, &s);
  return st == MLA_OK ? mla_check_write_rows(s.data(), n_tokens, cache_rows) : st;
}

}  // namespace mla
