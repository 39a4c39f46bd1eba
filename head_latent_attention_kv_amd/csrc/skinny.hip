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

#include "lds_dma.h"
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kWideNB = 6;  // 16-column blocks per workgroup of the wide bf16 variant
constexpr int kKS = 32;     // k per MFMA step
constexpr int kMaxMerge = 8;

// A operand kinds
constexpr int kABf16 = 0;   // bf16 rows
constexpr int kAF32 = 1;    // fp32 rows, split hi/lo into two bf16 MFMA operands
constexpr int kAMerge = 2;  // rows formed as Σ_s w[m][s]·A_s from bf16 split partials (softmax merge)

// Raw A data of one lane for one k-step and one 16-row block: 8 consecutive k.
template <int AK, int NS>
struct ARaw;
template <int NS>
struct ARaw<kABf16, NS> {
  uint4 v;
};
template <int NS>
struct ARaw<kAF32, NS> {
  float4 v[2];
};
template <int NS>
struct ARaw<kAMerge, NS> {
  uint4 v[NS];  // 8 bf16 of each split
};

__device__ __forceinline__ void split_hi_lo(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
  // hi = bf16(x), lo = bf16(x - hi): hi·w + lo·w carries ~16 bits of x
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    const float h0 = __uint_as_float(h[i] << 16);
    const float h1 = __uint_as_float(h[i] & 0xFFFF0000u);
    l[i] = pack_bf16x2(x[2 * i] - h0, x[2 * i + 1] - h1);
  }
  hi = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(bf16x8, make_uint4(l[0], l[1], l[2], l[3]));
}

template <int MB, int NB, int AK, int NS, int DEPTH, int MINB, typename OutT>
__global__ __launch_bounds__(256, MINB) void skinny_kernel(SkinnyArgs sa) {
  __shared__ float red[3][MB * NB][4][64];  // partial tiles of waves 1..3
  __shared__ float wmerge[AK == kAMerge ? 64 * NS : 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  // blockIdx.x = column tile x token group; this workgroup's token rows are
  // [m0, m0 + 16 MB) of the M rows
  const int m_groups = max(1, sa.m_groups);
  const int n0 = (blockIdx.x / m_groups) * 16 * NB;
  const int m0 = (blockIdx.x % m_groups) * 16 * MB;
  const int m_last = sa.M - 1 - m0;  // last local row
  const int z = blockIdx.y;
  const int split = blockIdx.z;
  const int k_lo = split * sa.k_per_split;
  const int k_hi = min(sa.K, k_lo + sa.k_per_split);
  const int64_t a_base = static_cast<int64_t>(z) * sa.sAz + static_cast<int64_t>(m0) * sa.sAm;
  const int64_t b_base = static_cast<int64_t>(z) * sa.sBz;

  if constexpr (AK == kAMerge) {
    // w[m][s] = 2^(m_s - M) l_s / Σ_s 2^(m_s - M) l_s, M = max_s m_s, for this
    // workgroup's head z (each split's partial is its normalised o_)
    if (tid < 16 * MB && tid <= m_last) {
      const int ns = min(sa.n_merge, NS);
      const float* ml = sa.ml + (static_cast<int64_t>(m0 + tid) * ns * sa.ml_heads + z) * 2;
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < NS; ++j)
        if (j < ns) mx = fmaxf(mx, ml[j * sa.ml_heads * 2]);
      float den = 0.f, e[NS];
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        e[j] = j < ns ? exp2f(ml[j * sa.ml_heads * 2] - mx) * ml[j * sa.ml_heads * 2 + 1] : 0.f;
        den += e[j];
      }
      const float inv = 1.f / den;
#pragma unroll
      for (int j = 0; j < NS; ++j) wmerge[tid * NS + j] = e[j] * inv;
    }
    __syncthreads();
  }

  f32x4 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // contiguous k-steps of this wave
  const int n_steps = max(0, (k_hi - k_lo + kKS - 1) / kKS);  // 0 for an empty trailing piece
  const int per = n_steps / 4, extra = n_steps % 4;
  const int s_lo = wave * per + min(wave, extra);
  const int my_steps = per + (wave < extra ? 1 : 0);

  // Loads are unconditional: rows m >= M and columns n >= N read a clamped
  // (valid) row and only feed outputs that are never stored; k-groups past the
  // end of the K piece (only in a wave's last step) are zeroed at use.
  const bf16_t* wrow[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int n = min(n0 + 16 * j + l16, sa.N - 1);
    const uint16_t* base = n < sa.N0 ? sa.B0 + static_cast<int64_t>(n) * sa.sBo
                                     : sa.B1 + static_cast<int64_t>(n - sa.N0) * sa.sBo;
    wrow[j] = base + b_base;
  }
  int64_t arow[MB];
  float wm[MB][AK == kAMerge ? NS : 1];
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int m = min(16 * i + l16, m_last);  // local row
    arow[i] = a_base + static_cast<int64_t>(m) * sa.sAm;
    if constexpr (AK == kAMerge) {
#pragma unroll
      for (int j = 0; j < NS; ++j) wm[i][j] = wmerge[m * NS + j];
    }
  }

  // loads in flight: DEPTH k-steps of raw A and B fragments
  ARaw<AK, NS> ar[DEPTH][MB];
  uint4 bw[DEPTH][NB];
  bool kin[DEPTH];
  // step s of this wave; steps past its range re-read its last step's
  // addresses (cache hits) and are zeroed at use, so the loop has no branches
  auto fetch = [&](int s, int slot) {
    const int s_eff = max(0, min(s, my_steps - 1));
    const int k_raw = k_lo + kKS * (s_lo + s_eff) + 8 * lg;
    kin[slot] = s < my_steps && k_raw < k_hi;  // K is a multiple of 8
    const int k = min(kin[slot] ? k_raw : k_lo + kKS * (s_lo + s_eff), sa.K - 8);
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int64_t off = arow[i] + k;
      if constexpr (AK == kABf16) {
        ar[slot][i].v = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(sa.A) + off);
      } else if constexpr (AK == kAF32) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(sa.A) + off);
        ar[slot][i].v[0] = p[0];
        ar[slot][i].v[1] = p[1];
      } else {
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          const int jj = j < sa.n_merge ? j : 0;
          ar[slot][i].v[j] = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(sa.A) + off + jj * sa.sAs);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) bw[slot][j] = *reinterpret_cast<const uint4*>(wrow[j] + k);
  };

  auto consume = [&](int slot) {
    bf16x8 ah[MB], al[MB], bf[NB];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      if constexpr (AK == kABf16) {
        const uint4 v = ar[slot][i].v;
        ah[i] = __builtin_bit_cast(bf16x8, kin[slot] ? v : make_uint4(0, 0, 0, 0));
      } else {
        float x[8];
        if constexpr (AK == kAF32) {
          const float4 a = ar[slot][i].v[0], b = ar[slot][i].v[1];
          x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = 0.f;
#pragma unroll
          for (int j = 0; j < NS; ++j) {
            const uint4 a = ar[slot][i].v[j];
            const float w = wm[i][j];
            const uint32_t u[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              x[2 * q] = fmaf(w, __uint_as_float(u[q] << 16), x[2 * q]);
              x[2 * q + 1] = fmaf(w, __uint_as_float(u[q] & 0xFFFF0000u), x[2 * q + 1]);
            }
          }
        }
        if (!kin[slot]) {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = 0.f;
        }
        split_hi_lo(x, ah[i], al[i]);
      }
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) bf[j] = __builtin_bit_cast(bf16x8, bw[slot][j]);
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[i], bf[j], acc[i][j], 0, 0, 0);
        if constexpr (AK != kABf16)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[i], bf[j], acc[i][j], 0, 0, 0);
      }
  };

#pragma unroll
  for (int d = 0; d < DEPTH; ++d) fetch(d, d);
  for (int s = 0; s < my_steps; s += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      consume(d);
      fetch(s + d + DEPTH, d);
    }
  }

  // sum the four waves' tiles
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[wave - 1][i * NB + j][e][lane] = acc[i][j][e];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc[i][j][e] += red[0][i * NB + j][e][lane] + red[1][i * NB + j][e][lane] + red[2][i * NB + j][e][lane];

  // lane holds C[m = 16i + 4lg + e][n = n0 + 16j + l16]
  OutT* C = static_cast<OutT*>(sa.C) + static_cast<int64_t>(split) * sa.sPs + static_cast<int64_t>(z) * sa.sCz +
            static_cast<int64_t>(m0) * sa.sCm;
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int n = n0 + 16 * j + l16;
      if (n >= sa.N) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 16 * i + 4 * lg + e;
        if (m <= m_last) Elem<OutT>::store(C, static_cast<int64_t>(m) * sa.sCm + n, acc[i][j][e]);
      }
    }
}

// ---- DMA-staged variant for many column tiles, bf16 A (M <= 64) ----
// Per-lane fragment loads read 64 bytes of each of 16 weight rows per
// instruction, which leaves DRAM pages mostly idle (measured: ~4.9 TB/s at
// best for that pattern against ~6.2 TB/s for runs of 512 bytes and more).
// Here a workgroup owns 96 output columns and copies, per stage of 128 k, the
// tile's 96 weight rows and its 16·MB token rows (256-byte runs of each row)
// HBM/L2 -> LDS with global_load_lds_dwordx4: four stages in flight at 64 token
// rows, five at 16 or 32 (160 KB; two stages of 256 k measured slower).  16-byte chunk p of LDS row r holds
// global chunk p ^ (r & 15), so the 16 rows of one MFMA fragment read fall on
// distinct banks.  Eight waves, two per SIMD: waves 4-7 issue every copy and
// compute nothing, so the stalls of a copy's issue (the CU's memory pipeline
// is full most of the time) never hold up the matrix work; inside a stage
// compute wave w < 4 takes k-step w (32 k) for all 64 x 96 outputs, and the four
// partial tiles are summed through LDS at the end.  k past the K piece is read
// from a clamped address and its A fragments are zeroed.
// With the weights in the tiled layout (sa.Bt) a stage's weight image is one
// contiguous 24 KB block, already swizzled, so each weight copy reads one
// contiguous kilobyte: HBM then serves whole DRAM pages instead of 256-byte runs
// of 96 rows 10 KB apart.
constexpr int kDmaCols = kTileRows;                  // 6 column blocks
constexpr int kDmaNB = kDmaCols / 16;
constexpr int kDmaWaves = 8;                         // 4 compute + 4 copy waves
constexpr int kDmaThreads = 64 * kDmaWaves;
constexpr int kDmaLdsMax = 160 * 1024;

// stage geometry for KC k per stage and AR staged token rows (16 per row block
// of the MFMA tile; KC = 128: four stages at 64 rows, five at 16 or 32)
template <int KC, int AR>
struct DmaStage {
  static constexpr int kRun = KC * 2;                    // bytes of a row per stage
  static constexpr int kRowsPerOp = 1024 / kRun;         // rows per 1 KB copy
  static constexpr int kWOps = kDmaCols * kRun / 1024;   // weight copies per stage
  static constexpr int kAOps = AR * kRun / 1024;         // token-row copies per stage
  static constexpr int kOps = kWOps + kAOps;
  static constexpr int kOpsPerWave = kOps / 4;
  static constexpr int kBytes = kOps * 1024;
  static constexpr int kStages = kDmaLdsMax / kBytes;
  static constexpr int kLds = kStages * kBytes;
  static constexpr int kStepsPerWave = KC / 4 / kKS;     // k-steps of one wave per stage
  static_assert(kWOps % 4 == 0 && kAOps % 4 == 0, "copies of each kind split evenly over the copy waves");
  static_assert(kOpsPerWave * (kStages - 1) < 64 && kStages <= 5, "vmcnt range");
  static_assert(kStepsPerWave >= 1 && kRun / 16 <= 16 * 2, "swizzle covers a row's chunks");
};

template <int MB, int KC, typename OutT, bool TILED>
__global__ __launch_bounds__(kDmaThreads, 1) void skinny_dma_kernel(SkinnyArgs sa) {
  using G = DmaStage<KC, 16 * MB>;
  static_assert(KC == kTileK && G::kWOps * 1024 == kTileRows * kTileK * 2, "a stage's weights are one tiled block");
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  const bool copy_wave = wave >= 4;  // waves w and w + 4 share a SIMD
  const int n0 = blockIdx.x * kDmaCols;
  const int z = blockIdx.y;
  const int split = blockIdx.z;
  const int k_lo = split * sa.k_per_split;
  const int k_hi = min(sa.K, k_lo + sa.k_per_split);
  const int n_st = k_hi > k_lo ? (k_hi - k_lo + KC - 1) / KC : 0;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) unsigned char*)smem));
  const bf16_t* a_mat = static_cast<const bf16_t*>(sa.A) + static_cast<int64_t>(z) * sa.sAz;
  const int64_t b_off = static_cast<int64_t>(z) * sa.sBz;

  // copy o of stage st (1 KB, R = 1024 / run rows): rows R·o' .. R·o'+R-1 of the
  // weight tile (o < kWOps, o' = o) or of the token rows (o' = o - kWOps); the
  // lanes of row R·o'+q fill its LDS chunks p in order.  The rows of a weight
  // copy come from one matrix (B0 rows [0, N0), B1 the rest; N0 is a multiple
  // of 4 and of R).  Copy wave 4 + c issues weight copies o = c + 4i, then
  // token-row copies o = kWOps + c + 4i, so which kind a copy is never depends
  // on the wave.  Tiled weights: block (column tile, k block) is the stage's
  // weight image, copied kilobyte by kilobyte.
  const char* w_tiled = nullptr;
  if constexpr (TILED)
    w_tiled = reinterpret_cast<const char*>(sa.Bt) +
              (static_cast<int64_t>(blockIdx.x) * ((sa.K + KC - 1) / KC) + k_lo / KC) * (G::kWOps * 1024LL);
  auto issue = [&](int st) {
    if (!copy_wave) return;
    const int c = wave - 4;
    const int kb = k_lo + st * KC;
    const uint32_t dst = lds0 + (st % G::kStages) * G::kBytes;
    int ln = lane;
    __asm__ volatile("" : "+v"(ln));
    constexpr int kLanesPerRow = G::kRun / 16;
    const int q = ln / kLanesPerRow, p = ln % kLanesPerRow;
    // k of this lane's chunk in a row whose swizzle key is key (clamped into the K piece)
    auto k_of = [&](int key) {
      const int kc = kb + 8 * (p ^ key);
      return kc < k_hi ? kc : k_hi - 8;
    };
    // weights are read once per launch (non-temporal copy); the token rows
    // are read by every workgroup and stay cached
#pragma unroll
    for (int i = 0; i < G::kWOps / 4; ++i) {
      const int o = c + 4 * i;
      const uint32_t to = __builtin_amdgcn_readfirstlane(dst + o * 1024);
      if constexpr (TILED) {
        global_to_lds16_stream(w_tiled + static_cast<int64_t>(st) * (G::kWOps * 1024) + o * 1024,
                               static_cast<uint32_t>(ln) * 16u, to);
      } else {
        // rows past N read row N - 1; the base row keeps every lane offset >= 0
        const int r_base = min(n0 + o * G::kRowsPerOp, sa.N - 1);
        const int r = min(n0 + o * G::kRowsPerOp + q, sa.N - 1);
        const uint16_t* mat = r_base < sa.N0 ? sa.B0 + static_cast<int64_t>(r_base) * sa.sBo
                                             : sa.B1 + static_cast<int64_t>(r_base - sa.N0) * sa.sBo;
        const int kc = k_of((o * G::kRowsPerOp + q) & 15);
        global_to_lds16_stream(reinterpret_cast<const char*>(mat + b_off),
                               static_cast<uint32_t>((r - r_base) * sa.sBo + kc) * 2u, to);
      }
    }
#pragma unroll
    for (int i = 0; i < G::kAOps / 4; ++i) {
      const int o2 = c + 4 * i;
      const int m_base = min(o2 * G::kRowsPerOp, sa.M - 1);
      const int m = min(o2 * G::kRowsPerOp + q, sa.M - 1);
      const int kc = k_of((o2 * G::kRowsPerOp + q) & 15);
      global_to_lds16(reinterpret_cast<const char*>(a_mat + static_cast<int64_t>(m_base) * sa.sAm),
                      static_cast<uint32_t>((m - m_base) * sa.sAm + kc) * 2u,
                      __builtin_amdgcn_readfirstlane(dst + (G::kWOps + o2) * 1024));
    }
  };

  f32x4 acc[MB][kDmaNB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < kDmaNB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragment reads: row t of a region, logical chunk c -> LDS chunk c ^ (t & 15);
  // wave w takes k-steps [w S, w S + S) of the stage, S = kStepsPerWave
#pragma unroll
  for (int st = 0; st < G::kStages - 1; ++st)
    if (st < n_st) issue(st);
  int issued = min(G::kStages - 1, n_st) - 1;

  for (int st = 0; st < n_st; ++st) {
    if (copy_wave) {
      switch (issued - st) {  // stages issued after st
        case 0: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<G::kOpsPerWave>(); break;
        case 2: wait_vmcnt<2 * G::kOpsPerWave>(); break;
        default: wait_vmcnt<3 * G::kOpsPerWave>(); break;
      }
    }
    lds_barrier();  // stage st visible; stage st-1 read everywhere: its buffer is free
    if (st + G::kStages - 1 < n_st) {
      issue(st + G::kStages - 1);
      issued = st + G::kStages - 1;
    }
    if (copy_wave) continue;
    const unsigned char* sb = smem + (st % G::kStages) * G::kBytes;
#pragma unroll
    for (int q = 0; q < G::kStepsPerWave; ++q) {
      const int c_log = (wave * G::kStepsPerWave + q) * 4 + lg;
      const int frag_off = l16 * G::kRun + ((c_log ^ l16) << 4);
      const bool k_in = k_lo + st * KC + 8 * c_log < k_hi;
      bf16x8 af[MB], bf[kDmaNB];
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const uint4 v = *reinterpret_cast<const uint4*>(sb + G::kWOps * 1024 + i * 16 * G::kRun + frag_off);
        af[i] = __builtin_bit_cast(bf16x8, k_in ? v : make_uint4(0, 0, 0, 0));
      }
#pragma unroll
      for (int j = 0; j < kDmaNB; ++j)
        bf[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(sb + j * 16 * G::kRun + frag_off));
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < kDmaNB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  }

  // sum the four compute waves' tiles: each writes its partial tile, then every
  // wave sums an eighth of the tile over the four copies and stores it
  lds_barrier();  // every stage read; no copy in flight
  float* red = reinterpret_cast<float*>(smem);  // [4 compute waves][MB * kDmaNB][4][64]
  constexpr int kTile = MB * kDmaNB * 4 * 64;
  static_assert(4 * kTile * 4 <= G::kLds, "reduction buffer inside the ring");
  if (!copy_wave)
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < kDmaNB; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[wave * kTile + ((i * kDmaNB + j) * 4 + e) * 64 + lane] = acc[i][j][e];
  lds_barrier();
  OutT* C = static_cast<OutT*>(sa.C) + static_cast<int64_t>(split) * sa.sPs + static_cast<int64_t>(z) * sa.sCz;
  // blocks (i, j) = b handled by wave b % 8; lane holds C[m = 16i + 4lg + e][n = n0 + 16j + l16]
#pragma unroll
  for (int b = 0; b < MB * kDmaNB; ++b) {
    if (b % kDmaWaves != wave) continue;
    const int i = b / kDmaNB, j = b % kDmaNB;
    const int n = n0 + 16 * j + l16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = (b * 4 + e) * 64 + lane;
      const float v = red[idx] + red[kTile + idx] + red[2 * kTile + idx] + red[3 * kTile + idx];
      const int m = 16 * i + 4 * lg + e;
      if (n < sa.N && m < sa.M) Elem<OutT>::store(C, static_cast<int64_t>(m) * sa.sCm + n, v);
    }
  }
}

// ---- split merge + W_UV, DMA-staged (32 token rows per workgroup, 128 columns) ----
// out[m][z][:] = W_UV[z] · Σ_j w[m][j] A_j[m][z][:], with A_j the bf16 split
// partials and w the softmax-merge weights from (m_j, l_j).  A workgroup takes
// one head z and 32 token rows; per stage of 128 k it copies the head's 128
// W_UV rows and the 32 x NS partial rows (256-byte runs) HBM -> LDS with
// global_load_lds_dwordx4, two stages in flight.  Chunk p of an LDS row holds
// global chunk p ^ key, key = (row & 15) for W_UV rows and (token & 15) for the
// partial rows (NS consecutive rows per token), so the 16 rows of one fragment
// read fall on distinct banks.  Wave w takes k-step w of every stage: it forms
// the merged A fragment from the NS partial fragments in fp32, splits it into
// hi + lo bf16, and runs both against the W_UV fragments; the four partial
// tiles are summed through LDS at the end.
constexpr int kMgCols = 128;                       // output columns (d_v) per workgroup
constexpr int kMgRows = 32;                        // token rows per workgroup
constexpr int kMgKC = 128;                         // k per stage
constexpr int kMgRun = kMgKC * 2;                  // 256 bytes of a row per stage
constexpr int kMgStages = 2;

template <int NS>
struct MergeStage {
  static constexpr int kWOps = kMgCols * kMgRun / 1024;       // 32 W_UV copies (4 rows each)
  static constexpr int kAOps = kMgRows * NS * kMgRun / 1024;  // partial copies (4 rows each)
  static constexpr int kOps = kWOps + kAOps;
  static constexpr int kOpsPerWave = kOps / 4;
  static constexpr int kBytes = kOps * 1024;
  static constexpr int kLds = kMgStages * kBytes;
  static_assert(NS == 4, "one token's partial rows per copy");
  static_assert(kWOps % 4 == 0 && kAOps % 4 == 0, "copies of each kind split evenly over the waves");
  static_assert(kLds <= 160 * 1024 - 1024, "LDS budget (merge weights after the ring)");
  static_assert(kOpsPerWave < 64, "vmcnt range");
};

template <int NS>
__global__ __launch_bounds__(256, 1) void merge_uv_kernel(SkinnyArgs sa) {
  using G = MergeStage<NS>;
  constexpr int MB = kMgRows / 16, NB = kMgCols / 16;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  float* wmerge = reinterpret_cast<float*>(smem + G::kLds);  // [kMgRows][NS]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  const int m_groups = max(1, sa.m_groups);
  // Workgroups are dealt to the 8 XCDs round-robin by linear id.  When the
  // grid divides evenly the ids are renumbered so that the token groups of one
  // head share an XCD: the head's W_UV rows then cross HBM into one L2.
  int wg = blockIdx.x + gridDim.x * blockIdx.y;
  const int n_wg = gridDim.x * gridDim.y;
  if (n_wg % (8 * gridDim.x) == 0) wg = (wg % 8) * (n_wg / 8) + wg / 8;
  const int m0 = (wg % gridDim.x % m_groups) * kMgRows;
  const int m_last = sa.M - 1 - m0;  // last local token row
  const int z = wg / gridDim.x;
  const int n_st = (sa.K + kMgKC - 1) / kMgKC;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) unsigned char*)smem));
  const bf16_t* a_head = static_cast<const bf16_t*>(sa.A) + static_cast<int64_t>(z) * sa.sAz;
  const uint16_t* w_head = sa.B0 + static_cast<int64_t>(z) * sa.sBz;

  // merge weights w[t][j] = 2^(m_j - M) l_j / Σ_j 2^(m_j - M) l_j of token m0 + t
  if (tid < kMgRows && tid <= m_last) {
    const float* ml = sa.ml + (static_cast<int64_t>(m0 + tid) * NS * sa.ml_heads + z) * 2;
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < NS; ++j) mx = fmaxf(mx, ml[j * sa.ml_heads * 2]);
    float e[NS], den = 0.f;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      e[j] = exp2f(ml[j * sa.ml_heads * 2] - mx) * ml[j * sa.ml_heads * 2 + 1];
      den += e[j];
    }
    const float inv = 1.f / den;
#pragma unroll
    for (int j = 0; j < NS; ++j) wmerge[tid * NS + j] = e[j] * inv;
  }

  // copy o of stage st: 4 rows R = 4o'..4o'+3 of the W_UV region (o < kWOps,
  // o' = o) or of the partial region (o' = o - kWOps: token o', splits 0..3);
  // lanes 16q..16q+15 take row 4o'+q, LDS chunks p = lane % 16 in order.  Wave
  // w issues the W_UV copies o = w + 4i, then the partial copies o = kWOps + w + 4i.
  auto issue = [&](int st) {
    const int kb = st * kMgKC;
    const uint32_t dst = lds0 + (st % kMgStages) * G::kBytes;
    int ln = lane;
    __asm__ volatile("" : "+v"(ln));
    const int q = ln >> 4, p = ln & 15;
    auto k_of = [&](int key) {
      const int kc = kb + 8 * (p ^ key);
      return kc < sa.K ? kc : sa.K - 8;
    };
#pragma unroll
    for (int i = 0; i < G::kWOps / 4; ++i) {
      const int o = wave + 4 * i;
      const int n_base = min(4 * o, sa.N - 1), n = min(4 * o + q, sa.N - 1);
      const int kc = k_of((4 * o + q) & 15);
      global_to_lds16(reinterpret_cast<const char*>(w_head + static_cast<int64_t>(n_base) * sa.sBo),
                      static_cast<uint32_t>((n - n_base) * sa.sBo + kc) * 2u,
                      __builtin_amdgcn_readfirstlane(dst + o * 1024));
    }
#pragma unroll
    for (int i = 0; i < G::kAOps / 4; ++i) {
      const int t = wave + 4 * i;  // token row of the copy, splits j = q
      const int m = min(t, m_last);
      const int kc = k_of(t & 15);
      global_to_lds16(reinterpret_cast<const char*>(a_head + static_cast<int64_t>(m0 + m) * sa.sAm),
                      static_cast<uint32_t>(q * sa.sAs + kc) * 2u,
                      __builtin_amdgcn_readfirstlane(dst + (G::kWOps + t) * 1024));
    }
  };

  f32x4 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  issue(0);
  __syncthreads();  // merge weights visible (the copy of stage 0 stays in flight)
  float wm[MB][NS];
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int t = min(16 * i + l16, max(m_last, 0));
#pragma unroll
    for (int j = 0; j < NS; ++j) wm[i][j] = wmerge[t * NS + j];
  }
  const int c_log = wave * 4 + lg;  // this wave's k-step within the stage, chunk of the lane
  const int frag_off = (c_log ^ l16) << 4;
  for (int st = 0; st < n_st; ++st) {
    if (st + 1 < n_st) {
      issue(st + 1);  // its buffer was last read in step st - 1, before the previous barrier
      wait_vmcnt<G::kOpsPerWave>();
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();  // stage st visible everywhere
    const unsigned char* sb = smem + (st % kMgStages) * G::kBytes;
    const bool k_in = st * kMgKC + 8 * c_log < sa.K;
    bf16x8 ah[MB], al[MB], bf[NB];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const uint4 v = *reinterpret_cast<const uint4*>(sb + G::kWOps * 1024 + ((16 * i + l16) * NS + j) * kMgRun + frag_off);
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          x[2 * qq] = fmaf(wm[i][j], __uint_as_float(u[qq] << 16), x[2 * qq]);
          x[2 * qq + 1] = fmaf(wm[i][j], __uint_as_float(u[qq] & 0xFFFF0000u), x[2 * qq + 1]);
        }
      }
      if (!k_in) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.f;
      }
      split_hi_lo(x, ah[i], al[i]);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j)
      bf[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(sb + (16 * j + l16) * kMgRun + frag_off));
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[i], bf[j], acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[i], bf[j], acc[i][j], 0, 0, 0);
      }
    lds_barrier();  // stage st read everywhere before its buffer is refilled
  }

  // sum the four waves' tiles; wave b % 4 stores block b
  float* red = reinterpret_cast<float*>(smem);  // [4 waves][MB * NB][4][64]
  constexpr int kTile = MB * NB * 4 * 64;
  static_assert(4 * kTile * 4 <= G::kLds, "reduction buffer inside the ring");
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[wave * kTile + ((i * NB + j) * 4 + e) * 64 + lane] = acc[i][j][e];
  lds_barrier();
  bf16_t* C = static_cast<bf16_t*>(sa.C) + static_cast<int64_t>(z) * sa.sCz + static_cast<int64_t>(m0) * sa.sCm;
#pragma unroll
  for (int bk = 0; bk < MB * NB; ++bk) {
    if (bk % 4 != wave) continue;
    const int i = bk / NB, j = bk % NB;
    const int n = 16 * j + l16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = (bk * 4 + e) * 64 + lane;
      const float v = red[idx] + red[kTile + idx] + red[2 * kTile + idx] + red[3 * kTile + idx];
      const int m = 16 * i + 4 * lg + e;
      if (n < sa.N && m <= m_last) C[static_cast<int64_t>(m) * sa.sCm + n] = f32_to_bf16(v);
    }
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
    float part[16];
#pragma unroll
    for (int p = 0; p < 16; ++p) part[p] = p < splits ? c[p * sps + off] : 0.f;
    float v = 0.f;
#pragma unroll
    for (int p = 0; p < 16; ++p) v += part[p];
    c[off] = v;
  }
}
}  // namespace

namespace {
// bf16 variant choice, shared by the split planner and the launcher:
//  wide   = 96 columns per workgroup, one workgroup per CU (many column tiles,
//           A re-read per tile 2/3 of the weight bytes);
//  narrow = 32 columns, two per CU, deeper prefetch (few column tiles, where
//           K splits supply the parallelism);
//  else   = 64 columns, two per CU (up to 32 token rows).
enum class Bf16Variant { kWide, kNarrow, kBase };
Bf16Variant bf16_variant(int M, int N, int Z, int K) {
  // wide (96-column) tiles when they, or they times the K splits a long K allows,
  // fill the chip: a 5120-column output of K = 16384 runs 54 tiles x 5 splits
  const int tiles = (N + 16 * kWideNB - 1) / (16 * kWideNB) * Z;
  const int max_splits = std::max(1, std::min(16, K / 256));
  if (tiles >= 128 || tiles * max_splits >= 256) return Bf16Variant::kWide;
  return M <= 32 ? Bf16Variant::kBase : Bf16Variant::kNarrow;
}
}  // namespace

int skinny_splits(int M, int N, int Z, int K) {
  // workgroups to fill the slots (one or two per compute unit, as the bf16
  // launch picks), at least 256 k per split and at most 16 slices; the value
  // returned is the number of K pieces the kernel uses
  const Bf16Variant v = bf16_variant(M, N, Z, K);
  const int cols = v == Bf16Variant::kWide ? 16 * kWideNB : v == Bf16Variant::kNarrow ? 32 : 64;
  const int slots = v == Bf16Variant::kWide ? 256 : 512;
  const int tiles = (N + cols - 1) / cols * Z;
  // as many K pieces as keep the grid within one wave of workgroup slots (a
  // second, partly filled wave would take as long as the first)
  int splits = std::max(1, slots / tiles);
  splits = std::max(1, std::min({splits, std::max(1, K / 256), 16}));
  const int kps = k_per_split(K, splits);
  return (K + kps - 1) / kps;
}

template <typename T>
__global__ __launch_bounds__(256) void sum_cast_kernel(const float* __restrict__ c, int splits, int64_t sps,
                                                       int M, int N, int64_t ldc, T* __restrict__ out) {
  const int64_t total = static_cast<int64_t>(M) * N;
  for (int64_t i = blockIdx.x * 256LL + threadIdx.x; i < total; i += gridDim.x * 256LL) {
    const int64_t m = i / N, n = i - m * N;
    float v = 0.f;
    for (int p = 0; p < splits; ++p) v += c[p * sps + m * ldc + n];
    Elem<T>::store(out, i, v);
  }
}

void sum_cast_slices(int dtype, const float* c, int splits, int64_t sps, int M, int N, int64_t ldc, void* out,
                     hipStream_t s) {
  if (M <= 0 || N <= 0) return;
  const int64_t total = static_cast<int64_t>(M) * N;
  const int blocks = static_cast<int>(std::min<int64_t>(4096, (total + 255) / 256));
  if (dtype == kF32)
    hipLaunchKernelGGL(sum_cast_kernel<float>, dim3(blocks), dim3(256), 0, s, c, splits, sps, M, N, ldc,
                       static_cast<float*>(out));
  else
    hipLaunchKernelGGL(sum_cast_kernel<bf16_t>, dim3(blocks), dim3(256), 0, s, c, splits, sps, M, N, ldc,
                       static_cast<bf16_t*>(out));
}

void sum_split_slices(float* c, int splits, int64_t sps, int M, int N, int64_t ldc, hipStream_t s) {
  if (splits <= 1 || M <= 0 || N <= 0) return;
  const int64_t total = static_cast<int64_t>(M) * N;
  const int blocks = static_cast<int>(std::min<int64_t>(2048, (total + 255) / 256));
  hipLaunchKernelGGL(sum_slices_kernel, dim3(blocks), dim3(256), 0, s, c, splits, sps, M, N, ldc);
}

namespace {

template <int MB, int NB, int AK, int NS, int DEPTH, int MINB>
void launch_out(const SkinnyArgs& sa, bool out_bf16, hipStream_t s) {
  // every one of the `splits` slices is written (an empty K piece writes zeros)
  dim3 grid((sa.N + 16 * NB - 1) / (16 * NB) * std::max(1, sa.m_groups), sa.Z, sa.splits);
  if (out_bf16)
    hipLaunchKernelGGL((skinny_kernel<MB, NB, AK, NS, DEPTH, MINB, bf16_t>), grid, dim3(256), 0, s, sa);
  else
    hipLaunchKernelGGL((skinny_kernel<MB, NB, AK, NS, DEPTH, MINB, float>), grid, dim3(256), 0, s, sa);
}

template <int MB, bool TILED, typename OutT>
void launch_dma_kernel(const SkinnyArgs& sa, hipStream_t s) {
  constexpr int KC = kTileK;
  dim3 grid((sa.N + kDmaCols - 1) / kDmaCols, sa.Z, sa.splits);
  constexpr int lds = DmaStage<KC, 16 * MB>::kLds;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(skinny_dma_kernel<MB, KC, OutT, TILED>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  hipLaunchKernelGGL((skinny_dma_kernel<MB, KC, OutT, TILED>), grid, dim3(kDmaThreads), lds, s, sa);
}

// weights in place (B0 / B1), or tiled (sa.Bt)
template <int MB>
void launch_dma(const SkinnyArgs& sa, bool out_bf16, hipStream_t s) {
  const bool tiled = sa.Bt != nullptr;
  if (out_bf16) {
    if (tiled) launch_dma_kernel<MB, true, bf16_t>(sa, s);
    else launch_dma_kernel<MB, false, bf16_t>(sa, s);
  } else {
    if (tiled) launch_dma_kernel<MB, true, float>(sa, s);
    else launch_dma_kernel<MB, false, float>(sa, s);
  }
}

template <int MB>
void launch_kind(const SkinnyArgs& sa, int kind, int ns, bool out_bf16, hipStream_t s) {
  if (kind == kABf16) {
    const Bf16Variant v = bf16_variant(sa.M, sa.N, sa.Z, sa.K);
    if (v == Bf16Variant::kWide && sa.N0 % 4 == 0) launch_dma<MB>(sa, out_bf16, s);
    else if (v == Bf16Variant::kWide) launch_out<MB, kWideNB, kABf16, 1, 3, 1>(sa, out_bf16, s);
    else if constexpr (MB >= 3) launch_out<MB, 2, kABf16, 1, 4, 2>(sa, out_bf16, s);  // narrow (M > 32)
    else launch_out<MB, 4, kABf16, 1, 3, 2>(sa, out_bf16, s);                         // base (M <= 32)
  } else if (kind == kAF32 || ns <= 1) {
    launch_out<MB, 4, kAF32, 1, 2, 1>(sa, out_bf16, s);
  } else {
    switch (ns) {
      case 2: launch_out<MB, 4, kAMerge, 2, 2, 1>(sa, out_bf16, s); break;
      case 3: launch_out<MB, 4, kAMerge, 3, 1, 1>(sa, out_bf16, s); break;
      case 4: launch_out<MB, 4, kAMerge, 4, 1, 1>(sa, out_bf16, s); break;
      default: launch_out<MB, 4, kAMerge, kMaxMerge, 1, 1>(sa, out_bf16, s); break;
    }
  }
}

void launch(const SkinnyArgs& sa, int kind, int ns, bool out_bf16, hipStream_t s) {
  if (sa.M <= 0 || sa.N <= 0 || sa.Z <= 0) return;
  switch ((sa.M + 15) / 16) {
    case 1: launch_kind<1>(sa, kind, ns, out_bf16, s); break;
    case 2: launch_kind<2>(sa, kind, ns, out_bf16, s); break;
    case 3: launch_kind<3>(sa, kind, ns, out_bf16, s); break;
    default: launch_kind<4>(sa, kind, ns, out_bf16, s); break;
  }
}

}  // namespace

namespace {
// out chunk i (16 bytes): slot p = i % 16 of row r of block b = i / (16 kTileRows),
// b = tile t x k block kb; it holds k = kTileK kb + 8 (p ^ (r & 15)) .. + 7 of
// weight row kTileRows t + r (zero past the rows or past k)
__global__ __launch_bounds__(256) void tile_weights_kernel(const uint16_t* __restrict__ w0, int64_t n0,
                                                           const uint16_t* __restrict__ w1, int64_t n1,
                                                           int64_t k, int64_t k_blocks,
                                                           uint4* __restrict__ out, int64_t n_chunks) {
  for (int64_t i = blockIdx.x * 256LL + threadIdx.x; i < n_chunks; i += gridDim.x * 256LL) {
    const int p = static_cast<int>(i & 15);
    const int64_t rb = i >> 4;
    const int r = static_cast<int>(rb % kTileRows);
    const int64_t blk = rb / kTileRows;
    const int64_t row = (blk / k_blocks) * kTileRows + r;
    const int64_t kk = (blk % k_blocks) * kTileK + 8 * (p ^ (r & 15));
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (row < n0 + n1 && kk < k) {
      const uint16_t* src = row < n0 ? w0 + row * k : w1 + (row - n0) * k;
      v = *reinterpret_cast<const uint4*>(src + kk);
    }
    out[i] = v;
  }
}
}  // namespace

int64_t tiled_weight_bytes(int64_t n_rows, int64_t k) {
  return (n_rows + kTileRows - 1) / kTileRows * ((k + kTileK - 1) / kTileK) * (kTileRows * kTileK * 2);
}

void tile_weights(const uint16_t* w0, int64_t n0, const uint16_t* w1, int64_t n1, int64_t k, uint16_t* out,
                  hipStream_t s) {
  const int64_t n_chunks = tiled_weight_bytes(n0 + n1, k) / 16;
  if (n_chunks <= 0) return;
  const int blocks = static_cast<int>(std::min<int64_t>(8192, (n_chunks + 255) / 256));
  hipLaunchKernelGGL(tile_weights_kernel, dim3(blocks), dim3(256), 0, s, w0, n0, w1, n1, k,
                     (k + kTileK - 1) / kTileK, reinterpret_cast<uint4*>(out), n_chunks);
}

void gemm_skinny_tiled(SkinnyArgs sa, bool out_bf16, hipStream_t s) {
  if (sa.M <= 0 || sa.M > 64 || sa.N <= 0 || sa.Z != 1) return;
  if (sa.splits < 1) sa.splits = 1;
  sa.k_per_split = k_per_split(sa.K, sa.splits);
  switch ((sa.M + 15) / 16) {
    case 1: launch_dma<1>(sa, out_bf16, s); break;
    case 2: launch_dma<2>(sa, out_bf16, s); break;
    case 3: launch_dma<3>(sa, out_bf16, s); break;
    default: launch_dma<4>(sa, out_bf16, s); break;
  }
}

void gemm_skinny(SkinnyArgs sa, bool a_f32, bool out_bf16, hipStream_t s) {
  if (sa.splits < 1) sa.splits = 1;
  sa.k_per_split = k_per_split(sa.K, sa.splits);
  launch(sa, a_f32 ? kAF32 : kABf16, 1, out_bf16, s);
}

int skinny_max_merge() { return kMaxMerge; }

void gemm_skinny_merged(SkinnyArgs sa, int n_merge, bool out_bf16, hipStream_t s) {
  sa.n_merge = n_merge;
  sa.splits = 1;
  sa.k_per_split = k_per_split(sa.K, 1);
  if (n_merge == 4 && out_bf16 && sa.M > 32 && sa.M <= 64 && sa.N == kMgCols && sa.K % 8 == 0 &&
      sa.Z * 2 >= 128) {
    // DMA-staged merge: two workgroups of 32 token rows per head
    sa.m_groups = 2;
    constexpr int lds = MergeStage<4>::kLds + kMgRows * 4 * 4;
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(merge_uv_kernel<4>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    hipLaunchKernelGGL(merge_uv_kernel<4>, dim3(2, sa.Z), dim3(256), lds, s, sa);
    return;
  }
  if (n_merge > 1 && sa.M > 32 && sa.M <= 64 && sa.N >= 128 && sa.Z * 2 >= 128) {
    // the merge reads n_merge partial rows per token row: two workgroups per
    // head take 32 token rows each, so every partial is read once and the
    // registers freed go to a deeper prefetch over 128 columns
    sa.m_groups = 2;
    switch (n_merge) {
      case 2: launch_out<2, 8, kAMerge, 2, 3, 1>(sa, out_bf16, s); break;
      case 3: launch_out<2, 8, kAMerge, 3, 2, 1>(sa, out_bf16, s); break;
      case 4: launch_out<2, 8, kAMerge, 4, 2, 1>(sa, out_bf16, s); break;
      default: launch_out<2, 8, kAMerge, kMaxMerge, 1, 1>(sa, out_bf16, s); break;
    }
    return;
  }
  launch(sa, n_merge <= 1 ? kAF32 : kAMerge, n_merge, out_bf16, s);
}

}  // namespace mla
