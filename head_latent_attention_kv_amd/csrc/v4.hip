// Kernels of the DeepSeek-V4 / nanowhale MLA variant (nanowhale MLA page): one
// KV head of D values, normalised by kv_norm and rotated on its last d_rope dims,
// is both the key and the value of every query head.
//  - v4_rows_kernel: row epilogue of the KV / query projections: sum of K-split
//    slices, optional RMSNorm with gain (kv_norm; a null gain is unit gain), the page's complex-form RoPE
//    (apply_rotary_emb: pairs (2i, 2i+1) turned by p·f_i) of the last d_rope
//    dims, cast, store (to the token's cache slot, or dense per head);
//  - v4_merge_kernel: the split softmax merge with the attention sink in the
//    normalisation, then the inverse rotation of the output's last d_rope dims
//    by the query's own position (the page's rotation after attention).
// The attention itself runs in decode_mfma_kernel / attend_generic_kernel with
// the row as both the score and the PV operand.
#include <math.h>

#include <algorithm>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kRowMax = 1024;

template <typename T>
__global__ __launch_bounds__(256) void v4_rows_kernel(const float* __restrict__ proj, int64_t ld, int splits,
                                                      int64_t sps, int heads, int D, int d_rope, int norm,
                                                      const T* __restrict__ gain, float eps,
                                                      const int32_t* __restrict__ positions,
                                                      const int64_t* __restrict__ slots, double base,
                                                      const double* __restrict__ freqs, T* __restrict__ out) {
  __shared__ float row[kRowMax];
  __shared__ float red[4];
  const int64_t r = blockIdx.x;
  const int64_t t = r / heads;
  const int h = static_cast<int>(r - t * heads);
  const float* src = proj + t * ld + static_cast<int64_t>(h) * D;
  float ss = 0.f;
  for (int i = threadIdx.x; i < D; i += 256) {
    float v = 0.f;
    for (int p = 0; p < splits; ++p) v += src[p * sps + i];
    row[i] = v;
    ss = fmaf(v, v, ss);
  }
  float inv = 1.f;
  if (norm) {
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    inv = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / static_cast<float>(D) + eps);
  }
  __syncthreads();
  T* dst = out + (slots != nullptr ? slots[t] : r) * static_cast<int64_t>(D);
  const int n_plain = D - d_rope;
  for (int i = threadIdx.x; i < n_plain; i += 256) {
    const float g = gain != nullptr ? Elem<T>::load(gain, i) : 1.f;
    Elem<T>::store(dst, i, row[i] * inv * g);
  }
  const int32_t pos = positions[t];
  for (int k = threadIdx.x; k < d_rope / 2; k += 256) {
    const int i = n_plain + 2 * k;
    const float ga = gain != nullptr ? Elem<T>::load(gain, i) : 1.f;
    const float gb = gain != nullptr ? Elem<T>::load(gain, i + 1) : 1.f;
    const float a = row[i] * inv * ga, b = row[i + 1] * inv * gb;
    float c, sn;
    angle_cos_sin(static_cast<double>(pos) * rope_freq(k, base, freqs), &c, &sn);
    Elem<T>::store(dst, i, a * c - b * sn);
    Elem<T>::store(dst, i + 1, b * c + a * sn);
  }
}

// Eight consecutive values (16-byte aligned for bf16) as float, and back.
__device__ __forceinline__ void load8(const bf16_t* p, float (&v)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = p[i];
}
__device__ __forceinline__ void store8(bf16_t* p, const float (&v)[8]) {
  *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                            pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
}
__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = v[i];
}

// Workgroups (query, y): each thread merges 8 consecutive values of the
// query's [H, D] output (16-byte loads of every split's part), so the pass
// streams at memory speed for one split (prefill) as for several (decode).
template <typename T>
__global__ __launch_bounds__(256) void v4_merge_kernel(const T* __restrict__ part_o, const float* __restrict__ part_ml,
                                                       int n_split, int H, int D, int d_rope,
                                                       const float* __restrict__ sink,
                                                       const int32_t* __restrict__ seq_len,
                                                       const int64_t* __restrict__ cu, int batch, double base,
                                                       const double* __restrict__ freqs, T* __restrict__ out) {
  const int64_t q = blockIdx.x;
  // the query's own position: the last row of its sequence (decode), or its
  // offset in its sequence (prefill)
  int32_t pos;
  if (cu == nullptr) {
    pos = seq_len[q] - 1;
  } else {
    int lo = 0, hi = batch;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (cu[mid] <= q) lo = mid;
      else hi = mid;
    }
    pos = static_cast<int32_t>(q - cu[lo]);
  }
  const int n_plain = D - d_rope;
  const int per_q = H * D;
  for (int e0 = (blockIdx.y * 256 + threadIdx.x) * 8; e0 < per_q; e0 += gridDim.y * 256 * 8) {
    const int h = e0 / D, c0 = e0 - h * D;
    // softmax states are base 2 (u = s·log2 e): the sink joins as 2^(sink·log2 e - M)
    const float su = sink[h] * kLog2e;
    float mx = su;
    for (int j = 0; j < n_split; ++j) mx = fmaxf(mx, part_ml[((q * n_split + j) * H + h) * 2]);
    float den = exp2f(su - mx);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < n_split; ++j) {
      const int64_t pidx = (q * n_split + j) * H + h;
      const float l = part_ml[pidx * 2 + 1];
      const float w = l > 0.f ? exp2f(part_ml[pidx * 2] - mx) * l : 0.f;
      den += w;
      float v[8];
      load8(part_o + pidx * D + c0, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(w, v[i], acc[i]);
    }
    const float inv = 1.f / den;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float a = acc[2 * k] * inv, b = acc[2 * k + 1] * inv;
      const int col = c0 + 2 * k;
      if (col >= n_plain) {
        float c, sn;
        angle_cos_sin(-static_cast<double>(pos) * rope_freq((col - n_plain) / 2, base, freqs), &c, &sn);
        const float a2 = a * c - b * sn, b2 = b * c + a * sn;
        a = a2;
        b = b2;
      }
      acc[2 * k] = a;
      acc[2 * k + 1] = b;
    }
    store8(out + q * static_cast<int64_t>(per_q) + e0, acc);
  }
}

}  // namespace

bool v4_rows_supported(int D, int d_rope) {
  return D > 0 && D <= kRowMax && d_rope >= 0 && d_rope % 2 == 0 && d_rope <= D && D % 2 == 0;
}

void v4_rows(int dtype, const float* proj, int64_t ld, int splits, int64_t sps, int heads, int D, int d_rope,
             int norm, const void* gain, float eps, const int32_t* positions, const int64_t* slots, double theta,
             const double* freqs, void* out, int64_t n_tokens, hipStream_t s) {
  if (n_tokens <= 0) return;
  const double base = d_rope > 0 ? std::pow(theta, -2.0 / d_rope) : 1.0;
  dim3 grid(static_cast<unsigned>(n_tokens * heads));
  if (dtype == kF32)
    hipLaunchKernelGGL(v4_rows_kernel<float>, grid, dim3(256), 0, s, proj, ld, splits, sps, heads, D, d_rope,
                       norm, static_cast<const float*>(gain), eps, positions, slots, base, freqs,
                       static_cast<float*>(out));
  else
    hipLaunchKernelGGL(v4_rows_kernel<bf16_t>, grid, dim3(256), 0, s, proj, ld, splits, sps, heads, D, d_rope,
                       norm, static_cast<const bf16_t*>(gain), eps, positions, slots, base, freqs,
                       static_cast<bf16_t*>(out));
}

void v4_merge(int dtype, const void* part_o, const float* part_ml, int64_t n_q, int n_split, int H, int D,
              int d_rope, const float* sink, const int32_t* seq_len, const int64_t* cu, int batch, double theta,
              const double* freqs, void* out, hipStream_t s) {
  if (n_q <= 0) return;
  const double base = d_rope > 0 ? std::pow(theta, -2.0 / d_rope) : 1.0;
  // 2048 values per workgroup, or fewer pieces when the queries alone fill the chip
  const int pieces = (H * D + 2047) / 2048;
  dim3 grid(static_cast<unsigned>(n_q), static_cast<unsigned>(n_q >= 4096 ? 1 : pieces));
  if (dtype == kF32)
    hipLaunchKernelGGL(v4_merge_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(part_o), part_ml,
                       n_split, H, D, d_rope, sink, seq_len, cu, batch, base, freqs, static_cast<float*>(out));
  else
    hipLaunchKernelGGL(v4_merge_kernel<bf16_t>, grid, dim3(256), 0, s, static_cast<const bf16_t*>(part_o),
                       part_ml, n_split, H, D, d_rope, sink, seq_len, cu, batch, base, freqs,
                       static_cast<bf16_t*>(out));
}

}  // namespace mla
