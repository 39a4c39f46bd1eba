// Row epilogues of the projection GEMMs:
//  - cache rows: optional unit-gain RMSNorm over the latent, rotate-half RoPE of
//    each rotary-key group at the token's position, cast, store to its slot;
//  - query rotary part: RoPE of q_pe per head;
//  - normalised rows: sum of K-split slices, RMSNorm with a gain, cast (the
//    low-rank query's q_a_layernorm);
//  - per-head casts of fp32 projection columns.
// RoPE pairs dims (j, j + d/2), angle p·θ^(-2j/d) formed and reduced in double.
#include <algorithm>
#include <cmath>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kMaxHalf = 256;  // rotary pairs per group supported by the shared cos/sin table

template <typename T, int kSlices>
__global__ __launch_bounds__(256) void cache_rows_kernel(const float* __restrict__ proj, int64_t ld,
                                                         int splits, int64_t sps,
                                                         T* __restrict__ cache,
                                                         const int64_t* __restrict__ slots,
                                                         const int32_t* __restrict__ positions,
                                                         int r, int n_groups, int d_rope,
                                                         int latent_rmsnorm, float eps,
                                                         double rope_base,
                                                         const double* __restrict__ freqs) {
  __shared__ float row[1024];  // summed projection row (r + G*d_rope <= 1024)
  __shared__ float cs[kMaxHalf], sn[kMaxHalf];
  __shared__ float red[4];
  const int64_t t = blockIdx.x;
  const int row_w = r + n_groups * d_rope;
  const int half = d_rope / 2;
  // every slice load of this thread's (up to four) elements goes out first,
  // from clamped addresses so no branch splits them (splits <= kSlices)
  constexpr int kIt = 1024 / 256;
  float part[kIt][kSlices];
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    const int i = min(static_cast<int>(threadIdx.x) + 256 * it, row_w - 1);
#pragma unroll
    for (int p = 0; p < kSlices; ++p) part[it][p] = proj[min(p, splits - 1) * sps + t * ld + i];
  }
  const int32_t pos = positions[t];
  for (int j = threadIdx.x; j < half; j += blockDim.x) rope_cos_sin(pos, j, rope_base, freqs, &cs[j], &sn[j]);
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    const int i = static_cast<int>(threadIdx.x) + 256 * it;
    float v = 0.f;
#pragma unroll
    for (int p = 0; p < kSlices; ++p) v += p < splits ? part[it][p] : 0.f;
    if (i < row_w) row[i] = v;
  }
  __syncthreads();
  T* dst = cache + slots[t] * static_cast<int64_t>(row_w);

  float inv = 1.f;
  if (latent_rmsnorm) {
    float ss = 0.f;
    for (int i = threadIdx.x; i < r; i += blockDim.x) ss = fmaf(row[i], row[i], ss);
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int w = 0; w < static_cast<int>(blockDim.x) / 64; ++w) tot += red[w];
    inv = 1.0f / sqrtf(tot / static_cast<float>(r) + eps);
  }
  for (int i = threadIdx.x; i < r; i += blockDim.x) Elem<T>::store(dst, i, row[i] * inv);
  for (int i = threadIdx.x; i < n_groups * half; i += blockDim.x) {
    const int g = i / half, j = i % half;
    const float* src = row + r + g * d_rope;
    const float a = src[j], b = src[j + half];
    Elem<T>::store(dst, r + g * d_rope + j, a * cs[j] - b * sn[j]);
    Elem<T>::store(dst, r + g * d_rope + j + half, b * cs[j] + a * sn[j]);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void query_rope_kernel(const float* __restrict__ proj, int64_t ld,
                                                         int hstride, T* __restrict__ q_pe,
                                                         const int32_t* __restrict__ positions,
                                                         int n_heads, int d_rope, double rope_base,
                                                         const double* __restrict__ freqs) {
  const int64_t t = blockIdx.x;
  const int half = d_rope / 2;
  const int32_t pos = positions[t];
  const float* src = proj + t * ld;
  T* dst = q_pe + t * static_cast<int64_t>(n_heads) * d_rope;
  // blockIdx.y picks a slice of the (head, pair) items so one token's heads
  // spread over several workgroups
  const int items = n_heads * half;
  const int per = (items + gridDim.y - 1) / gridDim.y;
  const int lo = blockIdx.y * per, hi = min(items, lo + per);
  for (int i = lo + threadIdx.x; i < hi; i += blockDim.x) {
    // the pair's loads go out before its angle is formed
    const int h = i / half, j = i % half;
    const float a = src[h * hstride + j], b = src[h * hstride + j + half];
    float c, sn;
    rope_cos_sin(pos, j, rope_base, freqs, &c, &sn);
    Elem<T>::store(dst, h * d_rope + j, a * c - b * sn);
    Elem<T>::store(dst, h * d_rope + j + half, b * c + a * sn);
  }
}

// The query projection's K slices summed and its rotary part rotated in one
// launch: workgroups y < y_sum sum every other column into slice 0 (in place,
// in sum_slices_kernel's order), the rest sum and rotate the rotary pairs of head
// h (columns rope_off + h*hstride + j and + j + d_rope/2) into q_pe, as
// query_rope_kernel does from summed columns.
template <typename T>
__global__ __launch_bounds__(256) void query_sum_rope_kernel(float* __restrict__ q, int64_t ld, int splits,
                                                             int64_t sps, int n_cols, int rope_off, int hstride,
                                                             T* __restrict__ q_pe,
                                                             const int32_t* __restrict__ positions, int n_heads,
                                                             int d_rope, double rope_base,
                                                             const double* __restrict__ freqs, int y_sum) {
  const int64_t t = blockIdx.x;
  float* row = q + t * ld;
  const int half = d_rope / 2;
  if (static_cast<int>(blockIdx.y) < y_sum) {
    const int per = (n_cols + y_sum - 1) / y_sum;
    const int lo = blockIdx.y * per, hi = min(n_cols, lo + per);
    for (int c = lo + threadIdx.x; c < hi; c += blockDim.x) {
      const int rc = c - rope_off;
      if (rc >= 0 && rc % hstride < d_rope) continue;  // a rotary column: the other workgroups
      float part[16];
#pragma unroll
      for (int p = 0; p < 16; ++p) part[p] = p < splits ? row[p * sps + c] : 0.f;
      float v = 0.f;
#pragma unroll
      for (int p = 0; p < 16; ++p) v += part[p];
      row[c] = v;
    }
    return;
  }
  const int32_t pos = positions[t];
  T* dst = q_pe + t * static_cast<int64_t>(n_heads) * d_rope;
  const int items = n_heads * half;
  const int y_rope = gridDim.y - y_sum;
  const int per = (items + y_rope - 1) / y_rope;
  const int lo = (blockIdx.y - y_sum) * per, hi = min(items, lo + per);
  for (int i = lo + threadIdx.x; i < hi; i += blockDim.x) {
    const int h = i / half, j = i % half;
    const int ca = rope_off + h * hstride + j, cb = ca + half;
    float pa[16], pb[16];
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      pa[p] = p < splits ? row[p * sps + ca] : 0.f;
      pb[p] = p < splits ? row[p * sps + cb] : 0.f;
    }
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      a += pa[p];
      b += pb[p];
    }
    float c, sn;
    rope_cos_sin(pos, j, rope_base, freqs, &c, &sn);
    Elem<T>::store(dst, h * d_rope + j, a * c - b * sn);
    Elem<T>::store(dst, h * d_rope + j + half, b * c + a * sn);
  }
}

// dst[t, h*n + c] = src[t*ld + h*hstride + c] for c < n, cast to T (per-head
// columns of an fp32 projection, e.g. q_nope out of [q_nope ; q_pe] head rows).
template <typename T>
__global__ __launch_bounds__(256) void cast_heads_kernel(const float* __restrict__ src, int64_t ld,
                                                         int hstride, int n_heads, int n,
                                                         T* __restrict__ dst, int64_t n_rows) {
  const int i = blockIdx.x * 256 + threadIdx.x;  // column of the output row
  if (i >= n_heads * n) return;
  const int h = i / n, c = i - h * n;
  for (int64_t t = blockIdx.y; t < n_rows; t += gridDim.y)
    Elem<T>::store(dst, t * n_heads * n + i, src[t * ld + static_cast<int64_t>(h) * hstride + c]);
}

// out[t, i] = v[i] / sqrt(mean(v^2) + eps) * gain[i], v = the sum of `splits`
// fp32 slices of row t (n <= kNormMax, splits <= kNormSlices); gain == nullptr:
// unit gain.  1024 threads per row; each thread's slice loads go out before any
// sum (clamped addresses, no branch between them).
constexpr int kNormThreads = 1024;
constexpr int kNormPer = 4;  // elements per thread
constexpr int kNormMax = kNormThreads * kNormPer;
constexpr int kNormSlices = 16;
template <typename T>
__global__ __launch_bounds__(kNormThreads) void norm_rows_kernel(const float* __restrict__ proj, int64_t ld,
                                                                 int splits, int64_t sps, int n,
                                                                 const T* __restrict__ gain, float eps,
                                                                 T* __restrict__ out, int64_t ld_out) {
  __shared__ float red[kNormThreads / 64];
  const int64_t t = blockIdx.x;
  float part[kNormPer][kNormSlices];
#pragma unroll
  for (int e = 0; e < kNormPer; ++e) {
    const int i = min(static_cast<int>(threadIdx.x) + kNormThreads * e, n - 1);
#pragma unroll
    for (int p = 0; p < kNormSlices; ++p) part[e][p] = proj[min(p, splits - 1) * sps + t * ld + i];
  }
  float v[kNormPer];
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < kNormPer; ++e) {
    float a = 0.f;
#pragma unroll
    for (int p = 0; p < kNormSlices; ++p) a += p < splits ? part[e][p] : 0.f;
    v[e] = a;
    if (static_cast<int>(threadIdx.x) + kNormThreads * e < n) ss = fmaf(a, a, ss);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kNormThreads / 64; ++w) tot += red[w];
  const float inv = 1.0f / sqrtf(tot / static_cast<float>(n) + eps);
#pragma unroll
  for (int e = 0; e < kNormPer; ++e) {
    const int i = static_cast<int>(threadIdx.x) + kNormThreads * e;
    if (i < n) {
      const float g = gain != nullptr ? Elem<T>::load(gain, i) : 1.f;
      Elem<T>::store(out, t * ld_out + i, v[e] * inv * g);
    }
  }
}

}  // namespace

void cast_heads(int dtype, const float* src, int64_t ld, int hstride, int n_heads, int n, void* dst,
                int64_t n_rows, hipStream_t s) {
  if (n_rows <= 0 || n <= 0 || n_heads <= 0) return;
  dim3 grid(static_cast<unsigned>((n_heads * n + 255) / 256),
            static_cast<unsigned>(std::min<int64_t>(n_rows, 65535)));
  if (dtype == kF32)
    hipLaunchKernelGGL(cast_heads_kernel<float>, grid, dim3(256), 0, s, src, ld, hstride, n_heads, n,
                       static_cast<float*>(dst), n_rows);
  else
    hipLaunchKernelGGL(cast_heads_kernel<bf16_t>, grid, dim3(256), 0, s, src, ld, hstride, n_heads, n,
                       static_cast<bf16_t*>(dst), n_rows);
}

bool norm_rows_supported(int n) { return n > 0 && n <= kNormMax; }

void norm_rows(int dtype, const float* proj, int64_t ld, int splits, int64_t sps, int n, const void* gain,
               float eps, void* out, int64_t ld_out, int64_t n_rows, hipStream_t s) {
  if (n_rows <= 0) return;
  dim3 grid(static_cast<unsigned>(n_rows));
  if (dtype == kF32)
    hipLaunchKernelGGL(norm_rows_kernel<float>, grid, dim3(kNormThreads), 0, s, proj, ld, splits, sps, n,
                       static_cast<const float*>(gain), eps, static_cast<float*>(out), ld_out);
  else
    hipLaunchKernelGGL(norm_rows_kernel<bf16_t>, grid, dim3(kNormThreads), 0, s, proj, ld, splits, sps, n,
                       static_cast<const bf16_t*>(gain), eps, static_cast<bf16_t*>(out), ld_out);
}

void finalize_cache_rows(int dtype, const float* proj, int64_t ld, int splits, int64_t sps,
                         void* cache, const int64_t* slots, const int32_t* positions,
                         int64_t n_tokens, int r, int n_groups, int d_rope, int latent_rmsnorm,
                         float eps, double theta, const double* freqs, hipStream_t s) {
  if (n_tokens <= 0) return;
  const double base = std::pow(theta, -2.0 / d_rope);
  dim3 grid(static_cast<unsigned>(n_tokens));
  auto launch = [&](auto kernel, auto* out) {
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, s, proj, ld, splits, sps, out, slots, positions, r,
                       n_groups, d_rope, latent_rmsnorm, eps, base, freqs);
  };
  if (dtype == kF32) {
    float* out = static_cast<float*>(cache);
    if (splits <= 1) launch(cache_rows_kernel<float, 1>, out);
    else launch(cache_rows_kernel<float, 16>, out);
  } else {
    bf16_t* out = static_cast<bf16_t*>(cache);
    if (splits <= 1) launch(cache_rows_kernel<bf16_t, 1>, out);
    else launch(cache_rows_kernel<bf16_t, 16>, out);
  }
}

void finalize_query(int dtype, float* q, int64_t ld, int splits, int64_t sps, int n_cols, int rope_off,
                    int hstride, void* q_pe, const int32_t* positions, int64_t n_tokens, int n_heads,
                    int d_rope, double theta, const double* freqs, hipStream_t s) {
  if (n_tokens <= 0) return;
  if (splits <= 1) {
    finalize_query_rope(dtype, q + rope_off, ld, hstride, q_pe, positions, n_tokens, n_heads, d_rope, theta,
                        freqs, s);
    return;
  }
  const double base = std::pow(theta, -2.0 / d_rope);
  const int y_sum = std::max(1, std::min(16, n_cols / 256));
  const int y_rope = std::max(1, std::min(16, n_heads * (d_rope / 2) / 256));
  dim3 grid(static_cast<unsigned>(n_tokens), static_cast<unsigned>(y_sum + y_rope));
  if (dtype == kF32)
    hipLaunchKernelGGL(query_sum_rope_kernel<float>, grid, dim3(256), 0, s, q, ld, splits, sps, n_cols, rope_off,
                       hstride, static_cast<float*>(q_pe), positions, n_heads, d_rope, base, freqs, y_sum);
  else
    hipLaunchKernelGGL(query_sum_rope_kernel<bf16_t>, grid, dim3(256), 0, s, q, ld, splits, sps, n_cols, rope_off,
                       hstride, static_cast<bf16_t*>(q_pe), positions, n_heads, d_rope, base, freqs, y_sum);
}

void finalize_query_rope(int dtype, const float* proj, int64_t ld, int hstride, void* q_pe,
                         const int32_t* positions, int64_t n_tokens, int n_heads, int d_rope,
                         double theta, const double* freqs, hipStream_t s) {
  if (n_tokens <= 0) return;
  const double base = std::pow(theta, -2.0 / d_rope);
  const int items = n_heads * (d_rope / 2);
  dim3 grid(static_cast<unsigned>(n_tokens), static_cast<unsigned>(std::max(1, std::min(16, items / 256))));
  if (dtype == kF32)
    hipLaunchKernelGGL(query_rope_kernel<float>, grid, dim3(256), 0, s, proj, ld, hstride,
                       static_cast<float*>(q_pe), positions, n_heads, d_rope, base, freqs);
  else
    hipLaunchKernelGGL(query_rope_kernel<bf16_t>, grid, dim3(256), 0, s, proj, ld, hstride,
                       static_cast<bf16_t*>(q_pe), positions, n_heads, d_rope, base, freqs);
}

}  // namespace mla
