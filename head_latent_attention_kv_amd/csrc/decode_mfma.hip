// bf16 MFMA decode over the latent cache: one query token per sequence, all
// heads of that sequence in one workgroup, so every cache row is read from HBM
// once and used by all heads (the property that makes MLA decode cheap: the
// absorbed score q_lat·c + q_pe·kr and the latent-space P·c both read only the
// cached [c ; kr] rows).
//
// Workgroup = 8 wave64s, one (sequence, split of its rows).  Per 32-row tile:
//  1. the tile is copied HBM -> LDS with global_load_lds_dwordx4 (no register
//     staging), three tiles in flight;
//  2. score: wave w < H/16 computes Sᵀ[32 rows x 16 heads] = C·Qᵀ with
//     v_mfma_f32_16x16x32_bf16; C (the cache tile) is the A operand read from
//     LDS, Qᵀ the B operand held in registers (q_lat and the group's q_pe,
//     zero elsewhere, so one K loop covers the whole cache row);
//  3. online softmax per head in registers (base 2, max/sum across the four
//     lane groups that hold a head), P written to LDS as bf16, the rescale
//     factor of each head to LDS;
//  4. PV: wave w owns latent columns [w·R/8, (w+1)·R/8) for every head;
//     O += P·C with P (A operand) from LDS and C (B operand) read transposed
//     from the same tile with ds_read_b64_tr_b16.
// Output: normalised o_ (one split) or (m, l, unnormalised o_) partials.
#include <math.h>

#include <algorithm>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kTL = 32;      // cache rows per tile
constexpr int kStages = 3;   // tiles in flight
constexpr int kPP = 80;      // LDS bytes per head row of P (32 bf16 + pad: conflict-free reads)
constexpr float kLog2e = 1.4426950408889634f;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

template <int R, int RW, int NHB>
struct Shape {
  static_assert(R % (16 * kWaves) == 0, "latent width must split into 16-column blocks per wave");
  static_assert(RW % 32 == 0, "row width must be a multiple of 32");
  static constexpr int kSteps = RW / 32;                         // score k-steps
  static constexpr int kPitch = (((RW * 2 + 31) / 32) | 1) * 32;  // LDS row bytes: odd multiple of 32
  static constexpr int kTileBytes = kTL * kPitch;
  static constexpr int kChunks = (kTileBytes + 1023) / 1024;     // 1 KB direct-load chunks per tile
  static constexpr int kCPW = (kChunks + kWaves - 1) / kWaves;   // chunks per wave (padded)
  static constexpr int kNC = R / kWaves;                         // PV columns per wave
  static constexpr int kNB = kNC / 16;
  static constexpr int kLdsBytes = kStages * ((kTileBytes + 1023) / 1024) * 1024 + NHB * 16 * kPP +
                                   NHB * 16 * 4 + NHB * 16 * 8;
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
};

// s_waitcnt with vmcnt = N (expcnt, lgkmcnt left at their maximum), gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0xF70 | N);
}

// 16 bytes per lane, global -> LDS (global_load_lds_dwordx4): lane i's bytes land
// at LDS address lds_base + 16*i.  Issued from asm so the compiler does not treat
// every later LDS read as aliasing the in-flight copy (which makes it wait for
// all outstanding loads, prefetches included); the kernel waits with explicit
// vmcnt counts instead.  No register is written, so nothing is live in flight.
__device__ __forceinline__ void global_to_lds16(const void* gptr, uint32_t lds_base) {
  __asm__ __volatile__(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(gptr), "s"(lds_base)
      : "memory", "m0");
}

// Workgroup barrier for LDS traffic only: wait for this wave's LDS operations,
// then s_barrier.  Unlike __syncthreads() it does not wait for outstanding
// global loads, so the tiles prefetched into other LDS buffers stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt at maximum
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
}

template <int R, int RW, int NHB>
__global__ __launch_bounds__(kThreads) void decode_mfma_kernel(
    const bf16_t* __restrict__ q_lat, const bf16_t* __restrict__ q_pe,
    const bf16_t* __restrict__ cache, const int64_t* __restrict__ seq_start,
    const int32_t* __restrict__ seq_len, int H, int G, int d_rope, float scale, int n_split,
    int split_len, float* __restrict__ part_o, float* __restrict__ part_ml,
    float* __restrict__ o_out) {
  using S = Shape<R, RW, NHB>;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  constexpr int kBufBytes = S::kChunks * 1024;
  unsigned char* pbuf = smem + kStages * kBufBytes;               // P: [NHB*16 heads][kPP bytes]
  float* alpha_lds = reinterpret_cast<float*>(pbuf + NHB * 16 * kPP);  // [NHB*16]
  float* ml_lds = alpha_lds + NHB * 16;                             // [NHB*16][2]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;

  const int split = blockIdx.x % n_split;
  const int b = blockIdx.x / n_split;
  const int64_t row0 = seq_start[b];
  const int len = seq_len[b];
  const int l_begin = split * split_len;
  const int l_end = min(len, l_begin + split_len);
  const int n_tiles = l_end > l_begin ? (l_end - l_begin + kTL - 1) / kTL : 0;

  const char* cache_b = reinterpret_cast<const char*>(cache + row0 * RW);

  // ---- tile loader: chunk j of the padded tile image -> LDS [j*1 KB + lane*16]
  auto issue_tile = [&](int t) {
    const int tile_row = l_begin + t * kTL;
    const uint32_t dst_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u8*)smem)) +
                              (t % kStages) * kBufBytes;
#pragma unroll
    for (int i = 0; i < S::kCPW; ++i) {
      int j = wave + kWaves * i;
      if (j >= S::kChunks) j = S::kChunks - 1;  // duplicate of the last chunk: same bytes, benign
      const int off = j * 1024 + lane * 16;
      const int r = off / S::kPitch;
      int cb = off - r * S::kPitch;
      int row = tile_row + r;
      if (row >= l_end || r >= kTL) row = l_end - 1;   // masked rows / tail: read a valid row
      if (cb >= RW * 2) cb = 0;                        // pad bytes: any valid 16 B
      const char* src = cache_b + static_cast<uint32_t>(row * (RW * 2) + cb);
      global_to_lds16(src, __builtin_amdgcn_readfirstlane(dst_base + j * 1024));
    }
  };

  // ---- query fragments (score waves): Qᵀ B operand, lane: head = 16w + l16, k = 32ks + 8lg + e
  const bool score_wave = wave < NHB;
  const int head_s = wave * 16 + l16;
  bf16x8 qf[S::kSteps];
  if (score_wave) {
    const int per_group = H / G;
#pragma unroll
    for (int ks = 0; ks < S::kSteps; ++ks) {
      const int k0 = ks * 32 + lg * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (head_s < H) {
        if (k0 < R) {
          v = *reinterpret_cast<const uint4*>(q_lat + (static_cast<int64_t>(b) * H + head_s) * R + k0);
        } else {
          const int g = (k0 - R) / d_rope, j0 = (k0 - R) - g * d_rope;
          if (g == head_s / per_group)
            v = *reinterpret_cast<const uint4*>(q_pe + (static_cast<int64_t>(b) * H + head_s) * d_rope + j0);
        }
      }
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }
  const float qk_scale = scale * kLog2e;
  // Q fragments must have landed before any tile copy is issued: otherwise the
  // compiler's wait for them (at their first use, inside the tile loop) would
  // also drain the tile copies in flight.
  wait_vmcnt<0>();

  float m_run = -INFINITY, l_run = 0.f;  // per head (score waves), replicated over lane groups
  f32x4 o[NHB][S::kNB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int nb = 0; nb < S::kNB; ++nb) o[hb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int c0 = wave * S::kNC;  // PV column slice of this wave

  if (n_tiles > 0) issue_tile(0);
  if (n_tiles > 1) issue_tile(1);

  for (int t = 0; t < n_tiles; ++t) {
    if (t + 1 < n_tiles) wait_vmcnt<S::kCPW>();
    else wait_vmcnt<0>();
    lds_barrier();
    if (t + 2 < n_tiles) issue_tile(t + 2);
    const unsigned char* tile = smem + (t % kStages) * kBufBytes;
    const int valid = min(kTL, l_end - (l_begin + t * kTL));

    if (score_wave) {
      f32x4 sacc[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const unsigned char* arow = tile + (mb * 16 + l16) * S::kPitch + lg * 16;
#pragma unroll
        for (int ks = 0; ks < S::kSteps; ++ks) {
          bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(arow + ks * 64));
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[ks], acc, 0, 0, 0);
        }
        sacc[mb] = acc;
      }
      // rows of this lane: 16mb + 4lg + i ; head: l16
      float tmax = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = mb * 16 + lg * 4 + i;
          float s = sacc[mb][i] * qk_scale;
          s = row < valid ? s : -INFINITY;
          sacc[mb][i] = s;
          tmax = fmaxf(tmax, s);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = exp2f(m_run - m_new);
      float psum = 0.f;
      unsigned char* prow = pbuf + head_s * kPP;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        float p0 = exp2f(sacc[mb][0] - m_new), p1 = exp2f(sacc[mb][1] - m_new);
        float p2 = exp2f(sacc[mb][2] - m_new), p3 = exp2f(sacc[mb][3] - m_new);
        psum += (p0 + p1) + (p2 + p3);
        uint2 pk = make_uint2(pack_bf16x2(p0, p1), pack_bf16x2(p2, p3));
        *reinterpret_cast<uint2*>(prow + (mb * 16 + lg * 4) * 2) = pk;
      }
      psum += __shfl_xor(psum, 16, 64);
      psum += __shfl_xor(psum, 32, 64);
      l_run = l_run * alpha + psum;
      m_run = m_new;
      if (lg == 0) alpha_lds[head_s] = alpha;
    }
    lds_barrier();

    // ---- PV: O[heads][c0 : c0+kNC] += P[heads][rows] · C[rows][cols]
    bf16x8 bfrag[S::kNB];
#pragma unroll
    for (int nb = 0; nb < S::kNB; ++nb) {
      const int col = c0 + nb * 16 + 4 * (l16 & 3);
      const unsigned char* base = tile + (lg * 8 + (l16 >> 2)) * S::kPitch + col * 2;
      s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base));
      s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + 4 * S::kPitch));
      typedef short s16x8 __attribute__((ext_vector_type(8)));
      s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      bfrag[nb] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      const float4 al = *reinterpret_cast<const float4*>(alpha_lds + hb * 16 + lg * 4);
      const bf16x8 pa = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4*>(pbuf + (hb * 16 + l16) * kPP + lg * 16));
#pragma unroll
      for (int nb = 0; nb < S::kNB; ++nb) {
        f32x4 acc = o[hb][nb];
        acc[0] *= al.x;
        acc[1] *= al.y;
        acc[2] *= al.z;
        acc[3] *= al.w;
        o[hb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, bfrag[nb], acc, 0, 0, 0);
      }
    }
  }

  // ---- epilogue
  if (score_wave && lg == 0) {
    ml_lds[head_s * 2 + 0] = m_run;
    ml_lds[head_s * 2 + 1] = l_run;
    if (n_split > 1 && head_s < H) {
      const int64_t pidx = (static_cast<int64_t>(b) * n_split + split) * H + head_s;
      part_ml[pidx * 2 + 0] = m_run;
      part_ml[pidx * 2 + 1] = l_run;
    }
  }
  __syncthreads();
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = hb * 16 + lg * 4 + i;
      if (h >= H) continue;
      if (n_split == 1) {
        const float inv = 1.f / ml_lds[h * 2 + 1];
        float* dst = o_out + (static_cast<int64_t>(b) * H + h) * R + c0 + l16;
#pragma unroll
        for (int nb = 0; nb < S::kNB; ++nb) dst[nb * 16] = o[hb][nb][i] * inv;
      } else {
        float* dst = part_o + ((static_cast<int64_t>(b) * n_split + split) * H + h) * R + c0 + l16;
#pragma unroll
        for (int nb = 0; nb < S::kNB; ++nb) dst[nb * 16] = o[hb][nb][i];
      }
    }
}

template <int R, int RW, int NHB>
void launch(const AttnShape& sh, const void* q_lat, const void* q_pe, const void* cache,
            const int64_t* seq_start, const int32_t* seq_len, int batch, int n_split, int split_len,
            float* part_o, float* part_ml, float* o_out, hipStream_t s) {
  using S = Shape<R, RW, NHB>;
  auto kern = decode_mfma_kernel<R, RW, NHB>;
  hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                      S::kLdsBytes);
  hipLaunchKernelGGL(kern, dim3(batch * n_split), dim3(kThreads), S::kLdsBytes, s,
                     static_cast<const bf16_t*>(q_lat), static_cast<const bf16_t*>(q_pe),
                     static_cast<const bf16_t*>(cache), seq_start, seq_len, sh.H, sh.G, sh.d_rope,
                     sh.scale, n_split, split_len, part_o, part_ml, o_out);
}

}  // namespace

bool decode_mfma_supported(const AttnShape& sh) {
  const int nhb = (sh.H + 15) / 16;
  if (sh.d_rope % 8 != 0) return false;
  if (sh.r == 512 && sh.row_w == 576 && nhb == 8) return true;   // DeepSeek-V2 shape
  if (sh.r == 512 && sh.row_w == 544 && nhb == 2) return true;   // Qwen3-30B-A3B shape
  if (sh.r == 128 && sh.row_w == 160 && nhb == 2) return true;   // Qwen2.5-7B shape
  return false;
}

int decode_mfma_blocks_per_cu(const AttnShape& sh) {
  const int nhb = (sh.H + 15) / 16;
  int lds = 0;
  if (sh.r == 512 && sh.row_w == 576 && nhb == 8) lds = Shape<512, 576, 8>::kLdsBytes;
  else if (sh.r == 512 && sh.row_w == 544 && nhb == 2) lds = Shape<512, 544, 2>::kLdsBytes;
  else if (sh.r == 128 && sh.row_w == 160 && nhb == 2) lds = Shape<128, 160, 2>::kLdsBytes;
  if (lds == 0) return 1;
  return std::max(1, std::min(4, (160 * 1024) / lds));
}

void decode_mfma(const AttnShape& sh, const void* q_lat, const void* q_pe, const void* cache,
                 const int64_t* seq_start, const int32_t* seq_len, int batch, int n_split,
                 int split_len, float* part_o, float* part_ml, float* o_out, hipStream_t s) {
  if (batch <= 0) return;
  const int nhb = (sh.H + 15) / 16;
  if (sh.r == 512 && sh.row_w == 576 && nhb == 8)
    launch<512, 576, 8>(sh, q_lat, q_pe, cache, seq_start, seq_len, batch, n_split, split_len,
                        part_o, part_ml, o_out, s);
  else if (sh.r == 512 && sh.row_w == 544 && nhb == 2)
    launch<512, 544, 2>(sh, q_lat, q_pe, cache, seq_start, seq_len, batch, n_split, split_len,
                        part_o, part_ml, o_out, s);
  else if (sh.r == 128 && sh.row_w == 160 && nhb == 2)
    launch<128, 160, 2>(sh, q_lat, q_pe, cache, seq_start, seq_len, batch, n_split, split_len,
                        part_o, part_ml, o_out, s);
}

}  // namespace mla
