// Weight-streaming GEMM for few tokens (M <= 64):
//   C[z][m][n] = Σ_k A[z][m][k] · W[z][n][k]
// where output columns [0, N0) come from weight B0 and [N0, N) from B1 (row
// n - N0), so the two projections of one input (W_QC | W_QR, W_DKV | W_KR) run
// as one launch.
//
// The projection steps of a decode step multiply a handful of token rows by
// large [out, in] weights, so the time is the weight read.  A workgroup owns 64
// output columns and a K range; each of its four waves streams a contiguous
// quarter of that range in 32-wide k-steps, each lane loading its MFMA
// fragments straight from global memory (8 consecutive k of one weight row or
// token row = 16 bytes), with two k-steps of loads in flight ahead of the
// v_mfma_f32_16x16x32_bf16 that consume them.  The four waves' partial tiles are
// summed through LDS.  With splits > 1 the K range is cut into pieces whose fp32
// tiles go to C + s*sPs; the consumer of the output sums them.
#include <algorithm>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kBN = 64;     // output columns per workgroup
constexpr int kKS = 32;     // k per MFMA step
constexpr int kDepth = 2;   // k-steps of loads in flight per wave

template <bool A_F32>
__device__ __forceinline__ void load_a(const void* A, int64_t off, bool ok, bf16x8& hi, bf16x8& lo) {
  if (!ok) {
    hi = lo = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
    return;
  }
  if constexpr (A_F32) {
    // fp32 operand as hi = bf16(a) and lo = bf16(a - hi): hi·w + lo·w keeps ~16 bits of a
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(A) + off);
    const float4 a = p[0], b = p[1];
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
      const float h0 = bf16_to_f32(static_cast<bf16_t>(h[i] & 0xFFFF));
      const float h1 = bf16_to_f32(static_cast<bf16_t>(h[i] >> 16));
      l[i] = pack_bf16x2(v[2 * i] - h0, v[2 * i + 1] - h1);
    }
    hi = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
    lo = __builtin_bit_cast(bf16x8, make_uint4(l[0], l[1], l[2], l[3]));
  } else {
    hi = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(A) + off));
  }
}

template <int MB, bool A_F32, typename OutT>
__global__ __launch_bounds__(256) void skinny_kernel(SkinnyArgs sa) {
  __shared__ float red[3][MB * 4][4][64];  // partial tiles of waves 1..3
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * kBN;
  const int z = blockIdx.y;
  const int split = blockIdx.z;
  const int k_lo = split * sa.k_per_split;
  const int k_hi = min(sa.K, k_lo + sa.k_per_split);
  const int64_t a_base = static_cast<int64_t>(z) * sa.sAz;
  const int64_t b_base = static_cast<int64_t>(z) * sa.sBz;

  f32x4 acc[MB][4];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // contiguous k-steps of this wave
  const int n_steps = max(0, (k_hi - k_lo + kKS - 1) / kKS);  // 0 for an empty trailing piece
  const int per = n_steps / 4, extra = n_steps % 4;
  const int s_lo = wave * per + min(wave, extra);
  const int my_steps = per + (wave < extra ? 1 : 0);

  // weight row pointer of each n-block this lane feeds
  const bf16_t* wrow[4];
  bool nok[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + 16 * j + l16;
    nok[j] = n < sa.N;
    const bf16_t* base = n < sa.N0 ? sa.B0 + static_cast<int64_t>(n) * sa.sBo
                                   : sa.B1 + static_cast<int64_t>(n - sa.N0) * sa.sBo;
    wrow[j] = base + b_base;
  }

  bf16x8 ah[kDepth][MB], al[kDepth][MB], bw[kDepth][4];
  auto fetch = [&](int s, int slot) {
    const int k = k_lo + kKS * (s_lo + s) + 8 * lg;
    const bool kok = k < k_hi;  // K is a multiple of 8
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int m = 16 * i + l16;
      load_a<A_F32>(sa.A, a_base + static_cast<int64_t>(m) * sa.sAm + k, kok && m < sa.M, ah[slot][i],
                    al[slot][i]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      bw[slot][j] = (kok && nok[j]) ? __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(wrow[j] + k))
                                    : __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
  };

#pragma unroll
  for (int d = 0; d < kDepth; ++d)
    if (d < my_steps) fetch(d, d);
  for (int s = 0; s < my_steps; s += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      if (s + d < my_steps) {
        bf16x8 a_h[MB], a_l[MB], b_w[4];
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          a_h[i] = ah[d][i];
          a_l[i] = al[d][i];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) b_w[j] = bw[d][j];
        if (s + d + kDepth < my_steps) fetch(s + d + kDepth, d);
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_h[i], b_w[j], acc[i][j], 0, 0, 0);
            if constexpr (A_F32)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_l[i], b_w[j], acc[i][j], 0, 0, 0);
          }
      }
    }
  }

  // sum the four waves' tiles
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[wave - 1][i * 4 + j][e][lane] = acc[i][j][e];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc[i][j][e] += red[0][i * 4 + j][e][lane] + red[1][i * 4 + j][e][lane] + red[2][i * 4 + j][e][lane];

  // lane holds C[m = 16i + 4lg + e][n = n0 + 16j + l16]
  OutT* C = static_cast<OutT*>(sa.C) + static_cast<int64_t>(split) * sa.sPs + static_cast<int64_t>(z) * sa.sCz;
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + 16 * j + l16;
      if (n >= sa.N) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 16 * i + 4 * lg + e;
        if (m < sa.M) Elem<OutT>::store(C, static_cast<int64_t>(m) * sa.sCm + n, acc[i][j][e]);
      }
    }
}

template <int MB, bool A_F32>
void launch_mb(const SkinnyArgs& sa, dim3 grid, bool out_bf16, hipStream_t s) {
  if (out_bf16)
    hipLaunchKernelGGL((skinny_kernel<MB, A_F32, bf16_t>), grid, dim3(256), 0, s, sa);
  else
    hipLaunchKernelGGL((skinny_kernel<MB, A_F32, float>), grid, dim3(256), 0, s, sa);
}

template <bool A_F32>
void launch_a(const SkinnyArgs& sa, dim3 grid, int mb, bool out_bf16, hipStream_t s) {
  switch (mb) {
    case 1: launch_mb<1, A_F32>(sa, grid, out_bf16, s); break;
    case 2: launch_mb<2, A_F32>(sa, grid, out_bf16, s); break;
    case 3: launch_mb<3, A_F32>(sa, grid, out_bf16, s); break;
    default: launch_mb<4, A_F32>(sa, grid, out_bf16, s); break;
  }
}

}  // namespace

namespace {
int k_per_split(int K, int splits) {
  int kps = (K + splits - 1) / splits;
  return (kps + 4 * kKS - 1) / (4 * kKS) * (4 * kKS);
}

__global__ __launch_bounds__(256) void sum_slices_kernel(float* __restrict__ c, int splits, int64_t sps,
                                                         int M, int N, int64_t ldc) {
  const int64_t total = static_cast<int64_t>(M) * N;
  for (int64_t i = blockIdx.x * 256LL + threadIdx.x; i < total; i += gridDim.x * 256LL) {
    const int64_t off = (i / N) * ldc + i % N;
    float v = c[off];
    for (int p = 1; p < splits; ++p) v += c[p * sps + off];
    c[off] = v;
  }
}
}  // namespace

int skinny_splits(int N, int Z, int K) {
  // enough workgroups for 256 compute units, at least 512 k per split; the value
  // returned is the number of K pieces the kernel actually uses
  const int tiles = (N + kBN - 1) / kBN * Z;
  int splits = (256 + tiles - 1) / tiles;
  splits = std::max(1, std::min(splits, std::max(1, K / 512)));
  const int kps = k_per_split(K, splits);
  return (K + kps - 1) / kps;
}

void sum_split_slices(float* c, int splits, int64_t sps, int M, int N, int64_t ldc, hipStream_t s) {
  if (splits <= 1 || M <= 0 || N <= 0) return;
  const int64_t total = static_cast<int64_t>(M) * N;
  const int blocks = static_cast<int>(std::min<int64_t>(1024, (total + 255) / 256));
  hipLaunchKernelGGL(sum_slices_kernel, dim3(blocks), dim3(256), 0, s, c, splits, sps, M, N, ldc);
}

void gemm_skinny(SkinnyArgs sa, bool a_f32, bool out_bf16, hipStream_t s) {
  if (sa.M <= 0 || sa.N <= 0 || sa.Z <= 0) return;
  if (sa.splits < 1) sa.splits = 1;
  sa.k_per_split = k_per_split(sa.K, sa.splits);
  const int mb = (sa.M + 15) / 16;
  // every one of the `splits` slices is written (an empty K piece writes zeros)
  dim3 grid((sa.N + kBN - 1) / kBN, sa.Z, sa.splits);
  if (a_f32) launch_a<true>(sa, grid, mb, out_bf16, s);
  else launch_a<false>(sa, grid, mb, out_bf16, s);
}

}  // namespace mla
