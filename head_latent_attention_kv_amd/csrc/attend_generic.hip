// Generic absorbed attention over latent-cache rows (VALU; any dtype/shape up to r = 512).
//
// Per query q, head h and cache row l of its key range:
//   s = scale·(q_lat[q,h]·c[l] + q_pe[q,h]·kr[l, g(h)])
// computed as one dot product of the whole cache row [c ; kr_0 ; ... ; kr_{G-1}]
// with a query row that is zero outside [q_lat ; q_pe at group g(h)].
// Online softmax over l (base-2: scale·log2(e) folded into the query), then
// o_[q,h,:] = Σ_l P[h,l]·c[l,:] in latent space; W_UV is applied afterwards.
//
// Block = 256 threads, a block of kHB heads x one query x one split of the key
// range; tiles of kLT rows staged through LDS and shared by the kHB heads.
// This kernel serves the fp32 layer and any shape the MFMA kernels do not take.
#include <math.h>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kHB = 8;    // heads per block
constexpr int kLT = 32;   // cache rows per tile
constexpr int kRJ = 16;   // latent columns per thread (r <= 32 * kRJ = 512)

// LDS row pitch (elements) of a staged cache tile: an odd number of 32-bit words,
// so the per-row and per-column reads of the score and PV loops hit distinct banks.
__host__ __device__ inline int lds_pitch(int row_w, int elem_bytes) {
  if (elem_bytes == 4) return row_w | 1;
  int p = (row_w + 1) & ~1;
  return ((p / 2) & 1) ? p : p + 2;
}

template <typename T>
__global__ __launch_bounds__(256) void attend_generic_kernel(
    const T* __restrict__ q_lat, const T* __restrict__ q_pe, const T* __restrict__ cache,
    const int64_t* __restrict__ seq_start, const int32_t* __restrict__ seq_len,
    const int64_t* __restrict__ cu, int batch, AttnShape sh, int n_split, int split_len,
    T* __restrict__ part_o, float* __restrict__ part_ml, float* __restrict__ o_out) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int row_w = sh.row_w;
  const int pitch = lds_pitch(row_w, sizeof(T));
  float* sq = reinterpret_cast<float*>(smem);                        // [kHB][row_w]
  float* sp = sq + kHB * row_w;                                      // [kHB][kLT]
  T* sc = reinterpret_cast<T*>(sp + kHB * kLT);                      // [kLT][pitch]

  const int64_t q = blockIdx.x;
  const int h0 = blockIdx.y * kHB;
  const int split = blockIdx.z;
  const int tid = threadIdx.x;
  const int hl = tid >> 5;        // local head of this thread (score and PV)
  const int lane32 = tid & 31;
  const int head = h0 + hl;
  const int per_group = sh.H / sh.G;

  int64_t start;
  int len;
  if (cu == nullptr) {
    start = seq_start[q];
    len = seq_len[q];
  } else {
    int lo = 0, hi = batch - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (cu[mid] <= q) lo = mid; else hi = mid - 1;
    }
    start = cu[lo];
    len = static_cast<int>(q - cu[lo] + 1);
  }
  const int l_begin = split * split_len;
  const int l_end = min(len, l_begin + split_len);

  // extended query rows, pre-scaled by scale*log2(e)
  const float qscale = sh.scale * 1.4426950408889634f;
  for (int i = tid; i < kHB * row_w; i += 256) {
    int hh = i / row_w, k = i % row_w, hd = h0 + hh;
    float v = 0.f;
    if (hd < sh.H) {
      if (k < sh.r) {
        v = Elem<T>::load(q_lat, (q * sh.H + hd) * sh.r + k);
      } else {
        int g = (k - sh.r) / sh.d_rope, j = (k - sh.r) % sh.d_rope;
        if (g == hd / per_group) v = Elem<T>::load(q_pe, (q * sh.H + hd) * sh.d_rope + j);
      }
    }
    sq[i] = v * qscale;
  }

  float m_run = -INFINITY, l_run = 0.f;
  float acc[kRJ];
#pragma unroll
  for (int j = 0; j < kRJ; ++j) acc[j] = 0.f;

  for (int l0 = l_begin; l0 < l_end; l0 += kLT) {
    __syncthreads();
    const int rows = min(kLT, l_end - l0);
    for (int i = tid; i < rows * row_w; i += 256) {
      int l = i / row_w, k = i % row_w;
      sc[l * pitch + k] = cache[(start + l0 + l) * row_w + k];
    }
    __syncthreads();
    float s = -INFINITY;
    if (lane32 < rows) {
      const float* qr = sq + hl * row_w;
      const T* cr = sc + lane32 * pitch;
      float a = 0.f;
      for (int k = 0; k < row_w; ++k) a = fmaf(qr[k], Elem<T>::load(cr, k), a);
      s = a;
    }
    float tmax = s;
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, o, 64));
    const float m_new = fmaxf(m_run, tmax);
    const float p = exp2f(s - m_new);
    float psum = p;
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) psum += __shfl_xor(psum, o, 64);
    const float alpha = exp2f(m_run - m_new);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    sp[hl * kLT + lane32] = p;
    __syncthreads();
    const float* pr = sp + hl * kLT;
#pragma unroll
    for (int j = 0; j < kRJ; ++j) {
      int c = lane32 + 32 * j;
      if (c < sh.r) {
        float a = acc[j] * alpha;
        for (int l = 0; l < rows; ++l) a = fmaf(pr[l], Elem<T>::load(sc + l * pitch, c), a);
        acc[j] = a;
      }
    }
  }

  if (head >= sh.H) return;
  if (part_o == nullptr) {  // normalised o_ (one split)
    const float inv = 1.f / l_run;
#pragma unroll
    for (int j = 0; j < kRJ; ++j) {
      int c = lane32 + 32 * j;
      if (c < sh.r) o_out[(q * sh.H + head) * sh.r + c] = acc[j] * inv;
    }
  } else {
    // the split's normalised o_ in the layer's element type (an empty split: 0)
    const int64_t pidx = (q * n_split + split) * sh.H + head;
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
    for (int j = 0; j < kRJ; ++j) {
      int c = lane32 + 32 * j;
      if (c < sh.r) Elem<T>::store(part_o, pidx * sh.r + c, acc[j] * inv);
    }
    if (lane32 == 0) {
      part_ml[pidx * 2 + 0] = m_run;
      part_ml[pidx * 2 + 1] = l_run;
    }
  }
}

// o_ = Σ_j 2^(m_j - M) l_j o_j / Σ_j 2^(m_j - M) l_j over the splits j of (query, head).
// One workgroup per (query, head): the max and the denominator are block
// reductions over the splits; the weights w_j = 2^(m_j - M) l_j / den go to
// LDS 256 at a time, and each thread sums two adjacent columns over the splits
// with independent loads.  An empty split (m = -inf, l = 0) weighs 0.  The
// splits of query q are the partial-state items q·n_split .. q·n_split +
// n_split - 1, or, with ragged_items > 0, the items the device plan over
// seq_len gives q (each wave recomputes that plan, as the attention kernel did).
constexpr int kMergeThreads = 256;

__device__ __forceinline__ float block_reduce(float v, bool is_max, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float u = __shfl_xor(v, o, 64);
    v = is_max ? fmaxf(v, u) : v + u;
  }
  const int wave = threadIdx.x >> 6;
  __syncthreads();  // red is free
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  v = red[0];
#pragma unroll
  for (int w = 1; w < kMergeThreads / 64; ++w) v = is_max ? fmaxf(v, red[w]) : v + red[w];
  return v;
}

template <typename T>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(AttnShape sh, int n_split,
                                                              const T* __restrict__ part_o,
                                                              const float* __restrict__ part_ml,
                                                              float* __restrict__ o_out,
                                                              const int32_t* __restrict__ seq_len,
                                                              int ragged_items) {
  __shared__ float w_lds[kMergeThreads];
  __shared__ float red[kMergeThreads / 64];
  const int64_t q = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  int64_t first = q * n_split;  // first partial-state item of query q
  if (ragged_items > 0) {
    const RaggedLane rl = ragged_plan(seq_len, static_cast<int>(gridDim.x), ragged_items);
    first = __builtin_amdgcn_readfirstlane(__shfl(rl.first, static_cast<int>(q), kWave));
    n_split = __builtin_amdgcn_readfirstlane(__shfl(rl.count, static_cast<int>(q), kWave));
  }
  const float* ml0 = part_ml + (first * sh.H + h) * 2;  // split j at ml0 + 2 j H
  float mx = -INFINITY;
  for (int j = tid; j < n_split; j += kMergeThreads) mx = fmaxf(mx, ml0[2 * static_cast<int64_t>(j) * sh.H]);
  mx = block_reduce(mx, true, red);
  float den = 0.f;
  if (mx != -INFINITY)
    for (int j = tid; j < n_split; j += kMergeThreads) {
      const float* ml = ml0 + 2 * static_cast<int64_t>(j) * sh.H;
      den += exp2f(ml[0] - mx) * ml[1];
    }
  den = block_reduce(den, false, red);
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const T* po = part_o + (first * sh.H + h) * static_cast<int64_t>(sh.r);  // split j at po + j H r
  const int64_t js = static_cast<int64_t>(sh.H) * sh.r;
  // every thread runs every barrier: the column and split loops are uniform,
  // only the loads and stores are guarded (r is even)
  for (int c0 = 0; c0 < sh.r; c0 += 2 * kMergeThreads) {
    const int c = c0 + 2 * tid;
    const bool active = c < sh.r;
    float a0 = 0.f, a1 = 0.f;
    for (int j0 = 0; j0 < n_split; j0 += kMergeThreads) {
      const int jn = min(kMergeThreads, n_split - j0);
      __syncthreads();  // the previous chunk's weights are consumed
      if (tid < jn) {
        const float* ml = ml0 + 2 * static_cast<int64_t>(j0 + tid) * sh.H;
        w_lds[tid] = inv > 0.f ? exp2f(ml[0] - mx) * ml[1] * inv : 0.f;
      }
      __syncthreads();
      if (!active) continue;
      const T* p = po + j0 * js + c;
      int jj = 0;
      for (; jj + 4 <= jn; jj += 4) {
        float x[4][2];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          x[u][0] = Elem<T>::load(p, (jj + u) * js);
          x[u][1] = Elem<T>::load(p, (jj + u) * js + 1);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          a0 = fmaf(w_lds[jj + u], x[u][0], a0);
          a1 = fmaf(w_lds[jj + u], x[u][1], a1);
        }
      }
      for (; jj < jn; ++jj) {
        a0 = fmaf(w_lds[jj], Elem<T>::load(p, jj * js), a0);
        a1 = fmaf(w_lds[jj], Elem<T>::load(p, jj * js + 1), a1);
      }
    }
    if (active) {
      o_out[(q * sh.H + h) * sh.r + c] = a0;
      o_out[(q * sh.H + h) * sh.r + c + 1] = a1;
    }
  }
}

template <typename T>
size_t smem_bytes(const AttnShape& sh) {
  return sizeof(float) * (kHB * sh.row_w + kHB * kLT) +
         sizeof(T) * kLT * lds_pitch(sh.row_w, sizeof(T));
}

}  // namespace

int generic_head_block() { return kHB; }

bool attend_generic_fits(int dtype, const AttnShape& sh) {
  const size_t b = dtype == kF32 ? smem_bytes<float>(sh) : smem_bytes<bf16_t>(sh);
  return b <= 160 * 1024;
}

void attend_generic(int dtype, const AttnShape& sh, const void* q_lat, const void* q_pe,
                    const void* cache, const int64_t* seq_start, const int32_t* seq_len,
                    const int64_t* cu, int batch, int64_t n_q, int n_split, int split_len,
                    void* part_o, float* part_ml, float* o_out, hipStream_t s) {
  if (n_q <= 0) return;
  dim3 grid(static_cast<unsigned>(n_q), (sh.H + kHB - 1) / kHB, n_split);
  if (dtype == kF32) {
    size_t smem = smem_bytes<float>(sh);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(attend_generic_kernel<float>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
    hipLaunchKernelGGL(attend_generic_kernel<float>, grid, dim3(256), smem, s,
                       static_cast<const float*>(q_lat), static_cast<const float*>(q_pe),
                       static_cast<const float*>(cache), seq_start, seq_len, cu, batch, sh, n_split,
                       split_len, static_cast<float*>(part_o), part_ml, o_out);
  } else {
    size_t smem = smem_bytes<bf16_t>(sh);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(attend_generic_kernel<bf16_t>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
    hipLaunchKernelGGL(attend_generic_kernel<bf16_t>, grid, dim3(256), smem, s,
                       static_cast<const bf16_t*>(q_lat), static_cast<const bf16_t*>(q_pe),
                       static_cast<const bf16_t*>(cache), seq_start, seq_len, cu, batch, sh,
                       n_split, split_len, static_cast<bf16_t*>(part_o), part_ml, o_out);
  }
}

void merge_splits(int dtype, const AttnShape& sh, int64_t n_q, int n_split, const void* part_o,
                  const float* part_ml, float* o_out, hipStream_t s, const int32_t* seq_len, int ragged_items) {
  if (n_q <= 0) return;
  const dim3 grid(static_cast<unsigned>(n_q), sh.H);
  if (dtype == kF32)
    hipLaunchKernelGGL(merge_kernel<float>, grid, dim3(kMergeThreads), 0, s, sh, n_split,
                       static_cast<const float*>(part_o), part_ml, o_out, seq_len, ragged_items);
  else
    hipLaunchKernelGGL(merge_kernel<bf16_t>, grid, dim3(kMergeThreads), 0, s, sh, n_split,
                       static_cast<const bf16_t*>(part_o), part_ml, o_out, seq_len, ragged_items);
}

}  // namespace mla
