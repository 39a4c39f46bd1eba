// Batched strided GEMM used by the projection steps of the MLA path:
//   C[z][m][n] = Σ_k A[z][m][k] · B[z][k][n]
// A is k-contiguous (bf16, or fp32 split into a hi + lo pair of bf16 operands),
// B is either [n][k] (k-contiguous: the [out, in] projection weights, W_UV) or
// [k][n] (n-contiguous: W_UK, whose reduction dim is d_nope), C is fp32 or bf16.
//
// bf16 path: 256 threads = 4 wave64s in a 2x2 grid, each wave owning a
// (BM/2)x(BN/2) block of v_mfma_f32_16x16x32_bf16 tiles; A and B tiles are
// staged through LDS (k-contiguous, padded rows) with the next tile's global
// loads in flight while the current one is multiplied.
// fp32 path: plain LDS-tiled VALU kernel (small fp32 layers only).
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kBK = 64;        // k per LDS tile (two MFMA k-steps of 32)
constexpr int kPitch = kBK + 8;  // LDS row pitch in bf16 (16 B pad against bank conflicts)

// A chunk of 8 consecutive k.  bf16 A: the raw bits.  fp32 A: split into
// hi = bf16(a) and lo = bf16(a - hi), so hi·b + lo·b keeps ~16 mantissa bits of a.
template <bool A_F32>
__device__ __forceinline__ void load_a_chunk(const void* A, int64_t off, bool ok, uint4& hi,
                                             uint4& lo) {
  if (!ok) {
    hi = make_uint4(0, 0, 0, 0);
    lo = hi;
    return;
  }
  if constexpr (A_F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(A) + off);
    float4 a = p[0], b = p[1];
    float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float h0 = bf16_to_f32(f32_to_bf16(v[2 * i])), h1 = bf16_to_f32(f32_to_bf16(v[2 * i + 1]));
      h[i] = pack_bf16x2(h0, h1);
      l[i] = pack_bf16x2(v[2 * i] - h0, v[2 * i + 1] - h1);
    }
    hi = make_uint4(h[0], h[1], h[2], h[3]);
    lo = make_uint4(l[0], l[1], l[2], l[3]);
  } else {
    hi = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(A) + off);
  }
}

template <int BM, int BN, bool A_F32, bool B_KN, typename OutT>
__global__ __launch_bounds__(256) void gemm_bf16_mfma(GemmArgs g) {
  constexpr int WM = BM / 2, WN = BN / 2;     // per-wave block
  constexpr int TM = WM / 16, TN = WN / 16;   // MFMA tiles per wave
  constexpr int A_CHUNKS = BM * kBK / 8 / 256;  // 16-byte chunks per thread
  constexpr int B_CHUNKS = BN * kBK / 8 / 256;
  static_assert(A_CHUNKS >= 1 && B_CHUNKS >= 1, "tile too small");

  __shared__ __attribute__((aligned(16))) bf16_t sA[BM * kPitch];
  __shared__ __attribute__((aligned(16))) bf16_t sAlo[A_F32 ? BM * kPitch : 8];
  __shared__ __attribute__((aligned(16))) bf16_t sB[BN * kPitch];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int z = blockIdx.z;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;

  const int64_t a_base = static_cast<int64_t>(z) * g.sAz;
  const int64_t b_base = static_cast<int64_t>(z) * g.sBz;

  uint4 ra[A_CHUNKS], ralo[A_CHUNKS], rb[B_CHUNKS];

  auto load_tiles = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
      int c = tid + i * 256;
      int row = c / (kBK / 8), kc = (c % (kBK / 8)) * 8;
      int m = m0 + row, k = k0 + kc;
      bool ok = (m < g.M) && (k < g.K);
      load_a_chunk<A_F32>(g.A, a_base + static_cast<int64_t>(m) * g.sAm + k, ok, ra[i], ralo[i]);
    }
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) {
      int c = tid + i * 256;
      if constexpr (!B_KN) {
        int row = c / (kBK / 8), kc = (c % (kBK / 8)) * 8;
        int n = n0 + row, k = k0 + kc;
        bool ok = (n < g.N) && (k < g.K);
        rb[i] = ok ? *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(g.B) + b_base +
                                                      static_cast<int64_t>(n) * g.sBo + k)
                   : make_uint4(0, 0, 0, 0);
      } else {
        // chunk = 8 consecutive n at one k
        int krow = c / (BN / 8), nc = (c % (BN / 8)) * 8;
        int n = n0 + nc, k = k0 + krow;
        bool ok = (n < g.N) && (k < g.K);  // N % 8 == 0 is checked by the host
        rb[i] = ok ? *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(g.B) + b_base +
                                                      static_cast<int64_t>(k) * g.sBo + n)
                   : make_uint4(0, 0, 0, 0);
      }
    }
  };

  auto store_tiles = [&]() {
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
      int c = tid + i * 256;
      int row = c / (kBK / 8), kc = (c % (kBK / 8)) * 8;
      *reinterpret_cast<uint4*>(&sA[row * kPitch + kc]) = ra[i];
      if constexpr (A_F32) *reinterpret_cast<uint4*>(&sAlo[row * kPitch + kc]) = ralo[i];
    }
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) {
      int c = tid + i * 256;
      if constexpr (!B_KN) {
        int row = c / (kBK / 8), kc = (c % (kBK / 8)) * 8;
        *reinterpret_cast<uint4*>(&sB[row * kPitch + kc]) = rb[i];
      } else {
        int krow = c / (BN / 8), nc = (c % (BN / 8)) * 8;
        const bf16_t* v = reinterpret_cast<const bf16_t*>(&rb[i]);
#pragma unroll
        for (int e = 0; e < 8; ++e) sB[(nc + e) * kPitch + krow] = v[e];
      }
    }
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_tiles(0);
  for (int k0 = 0; k0 < g.K; k0 += kBK) {
    __syncthreads();
    store_tiles();
    __syncthreads();
    if (k0 + kBK < g.K) load_tiles(k0 + kBK);
#pragma unroll
    for (int ks = 0; ks < kBK / 32; ++ks) {
      const int kof = ks * 32 + 8 * (lane >> 4);
      bf16x8 af[TM], aflo[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int a_off = (wm * WM + i * 16 + (lane & 15)) * kPitch + kof;
        af[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&sA[a_off]));
        if constexpr (A_F32) aflo[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&sAlo[a_off]));
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        uint4 v = *reinterpret_cast<const uint4*>(&sB[(wn * WN + j * 16 + (lane & 15)) * kPitch + kof]);
        bfr[j] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
          if constexpr (A_F32)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aflo[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    }
  }

  OutT* C = static_cast<OutT*>(g.C) + static_cast<int64_t>(z) * g.sCz;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      int n = n0 + wn * WN + j * 16 + (lane & 15);
      if (n >= g.N) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        int m = m0 + wm * WM + i * 16 + 4 * (lane >> 4) + e;
        if (m < g.M) Elem<OutT>::store(C, static_cast<int64_t>(m) * g.sCm + n, acc[i][j][e]);
      }
    }
}

// Row n of the fp32 B[z][n][k] operand, from B or (columns n >= N0) from B1.
__device__ __forceinline__ const float* f32_b_row(const GemmArgs& g, int z, int n) {
  const bool second = g.B1 != nullptr && n >= g.N0;
  const float* base = static_cast<const float*>(second ? g.B1 : g.B) + static_cast<int64_t>(z) * g.sBz;
  return base + static_cast<int64_t>(second ? n - g.N0 : n) * g.sBo;
}

// fp32 VALU GEMM: 16x16 outputs per 256-thread block, k staged by 16.
template <bool B_KN>
__global__ __launch_bounds__(256) void gemm_f32_valu(GemmArgs g) {
  __shared__ float sA[16][17];
  __shared__ float sB[16][17];  // sB[n][k]
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int z = blockIdx.z;
  const int m = blockIdx.y * 16 + ty, n = blockIdx.x * 16 + tx;
  const float* A = static_cast<const float*>(g.A) + static_cast<int64_t>(z) * g.sAz;
  const float* B = static_cast<const float*>(g.B) + static_cast<int64_t>(z) * g.sBz;
  float acc = 0.f;
  for (int k0 = 0; k0 < g.K; k0 += 16) {
    int am = blockIdx.y * 16 + ty, ak = k0 + tx;
    sA[ty][tx] = (am < g.M && ak < g.K) ? A[static_cast<int64_t>(am) * g.sAm + ak] : 0.f;
    int bn = blockIdx.x * 16 + ty, bk = k0 + tx;
    float bv = 0.f;
    if (bn < g.N && bk < g.K)
      bv = B_KN ? B[static_cast<int64_t>(bk) * g.sBo + bn] : f32_b_row(g, z, bn)[bk];
    sB[ty][tx] = bv;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) acc = fmaf(sA[ty][kk], sB[tx][kk], acc);
    __syncthreads();
  }
  if (m < g.M && n < g.N)
    static_cast<float*>(g.C)[static_cast<int64_t>(z) * g.sCz + static_cast<int64_t>(m) * g.sCm + n] = acc;
}

// fp32 product of a few rows (M <= kSmallM): one launch of latency, no k
// staging.  B [n][k]: each wave computes four output columns for all rows, its
// lanes striding k (coalesced rows of A and B), then a shuffle sum per output.
// B [k][n]: each thread computes one column over k, the wave's loads of a B row
// coalesced.
constexpr int kSmallM = 4;

template <bool B_KN>
__global__ __launch_bounds__(256) void gemm_f32_small(GemmArgs g) {
  const int z = blockIdx.z;
  const float* A = static_cast<const float*>(g.A) + static_cast<int64_t>(z) * g.sAz;
  float* C = static_cast<float*>(g.C) + static_cast<int64_t>(z) * g.sCz;
  if constexpr (!B_KN) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nb = (blockIdx.x * 4 + wave) * 4;  // the wave's first column
    const float* brow[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) brow[c] = f32_b_row(g, z, min(nb + c, g.N - 1));
    float acc[4][kSmallM];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int m = 0; m < kSmallM; ++m) acc[c][m] = 0.f;
    for (int k = lane; k < g.K; k += 64) {
      float a[kSmallM];
#pragma unroll
      for (int m = 0; m < kSmallM; ++m) a[m] = m < g.M ? A[static_cast<int64_t>(m) * g.sAm + k] : 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float w = brow[c][k];
#pragma unroll
        for (int m = 0; m < kSmallM; ++m) acc[c][m] = fmaf(a[m], w, acc[c][m]);
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int m = 0; m < kSmallM; ++m) {
        float v = acc[c][m];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
        if (lane == 0 && m < g.M && nb + c < g.N) C[static_cast<int64_t>(m) * g.sCm + nb + c] = v;
      }
  } else {
    const int n = blockIdx.x * 256 + threadIdx.x;
    if (n >= g.N) return;
    const float* B = static_cast<const float*>(g.B) + static_cast<int64_t>(z) * g.sBz;
    float acc[kSmallM];
#pragma unroll
    for (int m = 0; m < kSmallM; ++m) acc[m] = 0.f;
    for (int k = 0; k < g.K; ++k) {
      const float b = B[static_cast<int64_t>(k) * g.sBo + n];
#pragma unroll
      for (int m = 0; m < kSmallM; ++m)
        if (m < g.M) acc[m] = fmaf(A[static_cast<int64_t>(m) * g.sAm + k], b, acc[m]);
    }
#pragma unroll
    for (int m = 0; m < kSmallM; ++m)
      if (m < g.M) C[static_cast<int64_t>(m) * g.sCm + n] = acc[m];
  }
}

// ---- few-token product with an n-contiguous weight (q_lat = q_nope · W_UK) ----
// For M <= 64 rows of fp32 A and B[z] = [K][N] bf16 (n contiguous): one
// workgroup per (z, 256-column slice of N).  A is split once into hi + lo bf16
// rows in LDS (rows padded by 16 bytes: the 16 rows of a fragment read fall on
// distinct banks); the [K][256] slice of B goes to LDS with its 32-byte column
// units XOR-swizzled by f(k) = (k & 3) + 4((k >> 3) & 1), so the eight rows one
// half-wave of a transposed read touches land on distinct banks.  B fragments
// come from ds_read_b64_tr_b16 (lane n gets 4 consecutive k of column n); wave w
// computes columns [64w, 64w + 64) of the slice for all M rows, K in chunks of
// 128 staged one at a time.
constexpr int kUkCols = 256;                  // columns per workgroup
constexpr int kUkK = 128;                     // k per staged chunk
constexpr int kUkBPitch = kUkCols * 2;        // 512 B per B row (swizzled, unpadded)
constexpr int kUkAPitch = kUkK * 2 + 16;      // 272 B per A row
constexpr int kUkLds = kUkK * kUkBPitch + 2 * 64 * kUkAPitch;

typedef short uk_s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uk_s16x4 uk_lds_s16x4;

__device__ __forceinline__ int uk_unit(int k, int u) { return u ^ ((k & 3) + 4 * ((k >> 3) & 1)); }

template <int MB, typename OutT>
__global__ __launch_bounds__(256) void gemm_uk_kernel(GemmArgs g) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char* sB = smem;
  unsigned char* sAh = smem + kUkK * kUkBPitch;
  unsigned char* sAl = sAh + 64 * kUkAPitch;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * kUkCols;
  const int z = blockIdx.y;
  const float* A = static_cast<const float*>(g.A) + static_cast<int64_t>(z) * g.sAz;
  const bf16_t* B = static_cast<const bf16_t*>(g.B) + static_cast<int64_t>(z) * g.sBz;

  f32x4 acc[MB][4];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < g.K; k0 += kUkK) {
    if (k0 > 0) __syncthreads();  // the previous chunk is consumed
    // B chunk: rows k0 .. k0+127, 32 chunks of 16 B per row; A chunk: rows
    // 0 .. 16MB-1, 32 float4 per row.  Every load is issued before any store,
    // from a clamped (valid) address, and zeroed past K, N or M afterwards.
    constexpr int kBLoads = kUkK * 32 / 256, kALoads = MB * 16 * 32 / 256;
    uint4 bv[kBLoads];
    float4 av[kALoads];
#pragma unroll
    for (int i = 0; i < kBLoads; ++i) {
      const int c = tid + 256 * i;
      const int k = k0 + (c >> 5), n = n0 + (c & 31) * 8;
      bv[i] = *reinterpret_cast<const uint4*>(B + static_cast<int64_t>(min(k, g.K - 1)) * g.sBo + min(n, g.N - 8));
    }
#pragma unroll
    for (int i = 0; i < kALoads; ++i) {
      const int c = tid + 256 * i;
      const int m = c >> 5, k = k0 + (c & 31) * 4;
      av[i] = *reinterpret_cast<const float4*>(A + static_cast<int64_t>(min(m, g.M - 1)) * g.sAm + min(k, g.K - 4));
    }
#pragma unroll
    for (int i = 0; i < kBLoads; ++i) {
      const int c = tid + 256 * i;
      const int kr = c >> 5, ch = c & 31;
      const bool ok = k0 + kr < g.K && n0 + ch * 8 < g.N;
      *reinterpret_cast<uint4*>(sB + kr * kUkBPitch + (uk_unit(kr, ch >> 1) * 2 + (ch & 1)) * 16) =
          ok ? bv[i] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kALoads; ++i) {
      const int c = tid + 256 * i;
      const int m = c >> 5, kc = (c & 31) * 4;
      const float4 a = (m < g.M && k0 + kc < g.K) ? av[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      const uint32_t h0 = pack_bf16x2(a.x, a.y), h1 = pack_bf16x2(a.z, a.w);
      const uint32_t l0 = pack_bf16x2(a.x - __uint_as_float(h0 << 16), a.y - __uint_as_float(h0 & 0xFFFF0000u));
      const uint32_t l1 = pack_bf16x2(a.z - __uint_as_float(h1 << 16), a.w - __uint_as_float(h1 & 0xFFFF0000u));
      *reinterpret_cast<uint2*>(sAh + m * kUkAPitch + kc * 2) = make_uint2(h0, h1);
      *reinterpret_cast<uint2*>(sAl + m * kUkAPitch + kc * 2) = make_uint2(l0, l1);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kUkK / 32; ++ks) {
      bf16x8 ah[MB], al[MB], bf[4];
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int off = (i * 16 + l16) * kUkAPitch + (ks * 32 + lg * 8) * 2;
        ah[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(sAh + off));
        al[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(sAl + off));
      }
      // lane s of each 16-lane group addresses row base + s/4, columns c0 + 4(s%4)..+3
      // of its 16-column unit; it receives column c0 + s at rows base..base+3
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int u = wave * 4 + j;  // 16-column unit within the slice (32 B)
        const int r_lo = ks * 32 + lg * 8 + (l16 >> 2), r_hi = r_lo + 4;
        const int cb = (l16 & 3) * 8;  // byte offset of columns 4(s%4) within the unit
        const uk_s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (uk_lds_s16x4*)(sB + r_lo * kUkBPitch + uk_unit(r_lo, u) * 32 + cb));
        const uk_s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (uk_lds_s16x4*)(sB + r_hi * kUkBPitch + uk_unit(r_hi, u) * 32 + cb));
        bf[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[i], bf[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[i], bf[j], acc[i][j], 0, 0, 0);
        }
    }
  }

  // lane holds C[m = 16i + 4lg + e][n = n0 + 64w + 16j + l16]
  OutT* C = static_cast<OutT*>(g.C) + static_cast<int64_t>(z) * g.sCz;
  if constexpr (sizeof(OutT) == 2) {
    // bf16 out: the tile goes through LDS (over the B slice, once every wave is
    // done with it) so each lane stores 16 contiguous bytes of one row
    __syncthreads();
    bf16_t* tile = reinterpret_cast<bf16_t*>(sB);  // [MB * 16 rows][kUkCols]
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          tile[(i * 16 + lg * 4 + e) * kUkCols + wave * 64 + j * 16 + l16] = f32_to_bf16(acc[i][j][e]);
    __syncthreads();
    constexpr int kChunks = MB * 16 * kUkCols / 8;  // 16-byte chunks of the tile
#pragma unroll
    for (int c = tid; c < kChunks; c += 256) {
      const int m = c / (kUkCols / 8), n = n0 + (c % (kUkCols / 8)) * 8;
      if (m < g.M && n < g.N)
        *reinterpret_cast<uint4*>(C + static_cast<int64_t>(m) * g.sCm + n) =
            *reinterpret_cast<const uint4*>(tile + m * kUkCols + (n - n0));
    }
  } else {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + wave * 64 + j * 16 + l16;
        if (n >= g.N) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = i * 16 + lg * 4 + e;
          if (m < g.M) Elem<OutT>::store(C, static_cast<int64_t>(m) * g.sCm + n, acc[i][j][e]);
        }
      }
  }
}

template <int MB>
void launch_uk(const GemmArgs& g, bool out_bf16, hipStream_t s) {
  dim3 grid((g.N + kUkCols - 1) / kUkCols, g.Z);
  if (out_bf16) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_uk_kernel<MB, bf16_t>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, kUkLds);
    hipLaunchKernelGGL((gemm_uk_kernel<MB, bf16_t>), grid, dim3(256), kUkLds, s, g);
  } else {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_uk_kernel<MB, float>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, kUkLds);
    hipLaunchKernelGGL((gemm_uk_kernel<MB, float>), grid, dim3(256), kUkLds, s, g);
  }
}

template <int BM, int BN, bool A_F32, bool B_KN>
void launch_bf16(const GemmArgs& g, bool out_bf16, hipStream_t s) {
  dim3 grid((g.N + BN - 1) / BN, (g.M + BM - 1) / BM, g.Z);
  if (out_bf16)
    hipLaunchKernelGGL((gemm_bf16_mfma<BM, BN, A_F32, B_KN, bf16_t>), grid, dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL((gemm_bf16_mfma<BM, BN, A_F32, B_KN, float>), grid, dim3(256), 0, s, g);
}

template <int BM, int BN>
void dispatch_bf16(const GemmArgs& g, bool a_f32, bool b_kn, bool out_bf16, hipStream_t s) {
  if (a_f32) {
    if (b_kn) launch_bf16<BM, BN, true, true>(g, out_bf16, s);
    else launch_bf16<BM, BN, true, false>(g, out_bf16, s);
  } else {
    if (b_kn) launch_bf16<BM, BN, false, true>(g, out_bf16, s);
    else launch_bf16<BM, BN, false, false>(g, out_bf16, s);
  }
}

}  // namespace

void gemm_f16_out(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.Z <= 0) return;
  const int64_t tiles128 = static_cast<int64_t>((g.M + 127) / 128) * ((g.N + 127) / 128) * g.Z;
  if (g.M >= 256 && tiles128 >= 512) {
    dim3 grid((g.N + 127) / 128, (g.M + 127) / 128, g.Z);
    hipLaunchKernelGGL((gemm_bf16_mfma<128, 128, false, false, _Float16>), grid, dim3(256), 0, s, g);
  } else {
    dim3 grid((g.N + 63) / 64, (g.M + 63) / 64, g.Z);
    hipLaunchKernelGGL((gemm_bf16_mfma<64, 64, false, false, _Float16>), grid, dim3(256), 0, s, g);
  }
}

void gemm(const GemmArgs& g, int dtype, bool a_f32, bool b_kn, bool out_bf16, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.Z <= 0) return;
  if (dtype == kF32) {
    if (g.M <= kSmallM) {
      const dim3 grid(b_kn ? (g.N + 255) / 256 : (g.N + 15) / 16, 1, g.Z);
      if (b_kn) hipLaunchKernelGGL(gemm_f32_small<true>, grid, dim3(256), 0, s, g);
      else hipLaunchKernelGGL(gemm_f32_small<false>, grid, dim3(256), 0, s, g);
      return;
    }
    dim3 grid((g.N + 15) / 16, (g.M + 15) / 16, g.Z);
    if (b_kn) hipLaunchKernelGGL(gemm_f32_valu<true>, grid, dim3(256), 0, s, g);
    else hipLaunchKernelGGL(gemm_f32_valu<false>, grid, dim3(256), 0, s, g);
    return;
  }
  if (a_f32 && b_kn && g.M <= 64 && g.K % 32 == 0 && g.N % 8 == 0 && g.sBo % 8 == 0 && g.sAm % 4 == 0 &&
      g.sAz % 4 == 0 && g.sCm % 8 == 0 && g.sCz % 8 == 0) {
    // few rows against an n-contiguous weight: the transposed-read kernel
    switch ((g.M + 15) / 16) {
      case 1: launch_uk<1>(g, out_bf16, s); break;
      case 2: launch_uk<2>(g, out_bf16, s); break;
      case 3: launch_uk<3>(g, out_bf16, s); break;
      default: launch_uk<4>(g, out_bf16, s); break;
    }
    return;
  }
  // Large problems: 128x128 tiles; otherwise 64x64 for more blocks.
  int64_t tiles128 = static_cast<int64_t>((g.M + 127) / 128) * ((g.N + 127) / 128) * g.Z;
  if (g.M >= 256 && tiles128 >= 512)
    dispatch_bf16<128, 128>(g, a_f32, b_kn, out_bf16, s);
  else
    dispatch_bf16<64, 64>(g, a_f32, b_kn, out_bf16, s);
}

}  // namespace mla
