// bf16 MFMA causal prefill over the latent cache (absorbed form).
//
// Every query head of a token reads the same cached rows [c ; kr] (MLA
// principle page, section on matrix absorption: the score is q_lat·c + q_pe·kr,
// eq. (4) accumulates P·c), so attention over the latent cache is multi-query
// attention with K = [c ; kr] and V = c.  Causal rule (nanowhale page, SDPA
// with is_causal): token t attends to the rows cu[b] .. t of its sequence.
//
// Workgroup = 4 wave64s when two workgroups' rings fit in a CU's LDS (two per
// CU, each with its own barriers), else 8; each wave's 16 MFMA columns are
// (token, head) pairs
// (one token with its H = 16 heads, or 16/H tokens of H heads; see below).
// The workgroup streams
// the union of its tokens' key ranges in 32-row tiles through a 4-buffer LDS
// ring (global_load_lds_dwordx4; 16-byte chunks XOR-swizzled by 2·((row / 2) mod 4) within
// groups of eight so fragment reads spread over the banks).  Per tile and wave:
//   - score Sᵀ[32 keys x 16 columns]: two 16x16 blocks of
//     v_mfma_f32_16x16x32_bf16 over the whole row (K = r + G·d_rope), key rows
//     as the A operand from LDS, the token's Qᵀ as the B operand in registers
//     (q_lat, the head's rotary-group q_pe, zero elsewhere);
//   - causal / sequence mask (only on tiles that cross a column's sequence
//     start or its own token), softmax against a per-column reference: the max
//     of the first tile where the column has a valid key, base 2.  No running
//     max is kept: a pass whose weights pass 2^64 (seen in the row sums) is
//     redone after a max-only scan with each column's true max, so O is never
//     rescaled;
//   - PV: O[16 columns x r] += P[16 x 32]·C[32 x r], P straight from the softmax
//     registers as the A operand (the product's K order is the order in which
//     a lane holds its keys), C read transposed from the tile with
//     ds_read_b64_tr_b16 at the matching row bases.
// Blocks of later tokens (longer key ranges) are dispatched first.
// Output: normalised o_ [n_tokens, H, r] fp32; or, as a one-split softmax state
// for a caller that still folds in more terms (the V4 variant's attention
// sink), o_ in bf16 with its (reference, row sum) pair per (token, head).
// With H < 16 heads (H dividing 16) the 16 MFMA columns of a wave are 16/H
// consecutive tokens times H heads, each lane masking for its own column's
// token, and a workgroup covers 8·16/H tokens.  The V4
// variant (nanowhale page: one KV head of 512 dims used as key and value) runs
// the same kernel with r = row width = 512 and no separate rotary key; there
// the weights enter PV as a bf16 hi + lo pair (two MFMAs), since bf16 weights
// against the bf16 rows that are both key and value leave too little margin.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "lds_dma.h"
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kHeads = 16;          // query heads per token (one MFMA N block)
constexpr int kTL = 32;             // key rows per tile
constexpr int kStages = 4;
constexpr float kLog2e = 1.4426950408889634f;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

// Swizzle key of tile row r: the 16-byte chunks of a row are XORed within
// groups of eight by 2·((r / 2) mod 4).  On gfx950 a ds_read_b128 is served
// 16 lanes at a time, lanes 0-7 with 24-31 (and 8-15 with 16-23, likewise
// above 32), and a ds_read_b64_tr_b16 32 lanes at a time; with rows whose
// length is 128 bytes past a multiple of 256, this key keeps both the score's
// fragment reads (rows l16, chunk 4ks + lg) and the transposed PV reads (rows
// 4lg + l16/4, a 32-byte pair of chunks each) on distinct banks.  The key
// (r / 2) mod 8 left every transposed read two-way conflicted.
__device__ __forceinline__ int row_key(int r) { return ((r >> 1) & 3) << 1; }
// LDS chunk slot of 16-byte chunk c of tile row r (an involution for fixed r).
__device__ __forceinline__ int swz(int c, int r) { return (c & ~7) | ((c ^ row_key(r)) & 7); }

template <int R, int RW>
struct PShape {
  static_assert(R % 16 == 0 && RW % 32 == 0 && RW >= R, "row layout");
  static constexpr int kRowBytes = RW * 2;
  static constexpr int kRowChunks = kRowBytes / 16;
  static_assert(kRowChunks % 8 == 0, "swizzle groups of eight chunks");
  static constexpr int kTileBytes = kTL * kRowBytes;
  static_assert(kTileBytes % 1024 == 0, "whole 1 KB copies");
  static constexpr int kDmaOps = kTileBytes / 1024;
  // the setup scratch and the restart flags alias the start of the ring, which
  // is idle at those moments
  static constexpr int kLdsBytes = kStages * kTileBytes;
  // two waves per SIMD: two workgroups of 4 waves per CU when two rings fit in
  // its 160 KB of LDS (they then keep separate barriers and overlap each
  // other's MFMA and softmax phases), else one of 8
  static constexpr int kBlocksPerCU = 2 * kLdsBytes <= 160 * 1024 ? 2 : 1;
  static constexpr int kWaves = 8 / kBlocksPerCU;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kDmaPerWave = (kDmaOps + kWaves - 1) / kWaves;
  static_assert(3 * kDmaPerWave < 64, "vmcnt range");
  static constexpr int kSteps = RW / 32;     // score k-steps
  static constexpr int kNB = R / 16;         // PV column blocks
  static constexpr bool kSplitP = RW == R;   // K = V rows: weights as hi + lo bf16
  static constexpr int kLA = kSplitP ? 2 : 3;  // C fragments in flight
  static_assert(kTileBytes >= 8 * kWaves, "scratch in the ring");
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
};

template <int N, int PerWave>
__device__ __forceinline__ void wait_tiles_after() {
  wait_vmcnt<N * PerWave>();
}

template <int R, int RW>
__global__ __launch_bounds__((PShape<R, RW>::kThreads), (PShape<R, RW>::kBlocksPerCU)) void prefill_mfma_kernel(
    const bf16_t* __restrict__ q_lat, const bf16_t* __restrict__ q_pe,
    const bf16_t* __restrict__ cache, const int64_t* __restrict__ cu, int batch, int64_t n_tokens,
    int n_heads, int n_groups, int d_rope, float scale, float* __restrict__ o_out,
    bf16_t* __restrict__ part_o, float* __restrict__ part_ml) {
  using S = PShape<R, RW>;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  int64_t* range = reinterpret_cast<int64_t*>(smem);  // [S::kWaves] setup scratch (ring not yet in use)
  int* flags = reinterpret_cast<int*>(smem);          // restart flags (ring idle between passes)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;

  // ---- MFMA column l16 of this wave is (token t, head hc): token slot l16 / H
  // of the wave's 16/H tokens.  Its key rows are [seq_lo, t].
  const int tpw = kHeads / n_heads;
  const int64_t block_tokens = static_cast<int64_t>(S::kWaves) * tpw;
  const int64_t n_blocks = (n_tokens + block_tokens - 1) / block_tokens;
  const int64_t block = n_blocks - 1 - blockIdx.x;  // longest key ranges first
  const int64_t wave_t0 = block * block_tokens + static_cast<int64_t>(wave) * tpw;
  const int hc = l16 % n_heads;
  const int64_t t = wave_t0 + l16 / n_heads;
  const bool active = t < n_tokens;
  const int64_t last_t = min(block * block_tokens + block_tokens - 1, n_tokens - 1);
  int64_t seq_lo = last_t;
  if (active) {
    int lo = 0, hi = batch;  // largest b with cu[b] <= t
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (cu[mid] <= t) lo = mid;
      else hi = mid;
    }
    seq_lo = cu[lo];
  }
  // the workgroup's key range: union of its tokens' ranges
  int64_t wave_lo = seq_lo;
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) wave_lo = min(wave_lo, static_cast<int64_t>(__shfl_xor(wave_lo, d, 64)));
  if (lane == 0) range[wave] = wave_lo;
  __syncthreads();
  int64_t k_lo = range[0];
#pragma unroll
  for (int w = 1; w < S::kWaves; ++w) k_lo = min(k_lo, range[w]);
  const int64_t k_hi = last_t;
  const int n_tiles = static_cast<int>((k_hi - k_lo + kTL) / kTL);
  __syncthreads();  // range[] read everywhere before it is reused as flags

  const char* cache_c = reinterpret_cast<const char*>(cache);
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u8*)smem));

  // ---- tile copy: copy j fills LDS chunks [64j, 64j + 64); chunk L holds global
  // chunk L ^ row_key(row) of row L / kRowChunks; rows past k_hi read row k_hi
  // per-lane source offsets of this wave's copies: with a row of chunks that
  // is no power of two (a real divide), computed once for a full tile and
  // again only for a ragged last tile; otherwise per tile (shifts, no
  // registers held)
  auto dma_offsets = [&](int valid, uint32_t (&off)[S::kDmaPerWave]) {
    int ln = lane;
    __asm__ volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < S::kDmaPerWave; ++i) {
      const int j = min(wave + S::kWaves * i, S::kDmaOps - 1);  // duplicates of the last copy are benign
      const int L = j * 64 + ln;
      const int r = L / S::kRowChunks;
      const int g = r < valid ? (L ^ row_key(r)) : (valid - 1) * S::kRowChunks + (L & 7);
      off[i] = static_cast<uint32_t>(g * 16);
    }
  };
  constexpr bool kHoist = (S::kRowChunks & (S::kRowChunks - 1)) != 0;
  uint32_t full_off[S::kDmaPerWave];
  if constexpr (kHoist) dma_offsets(kTL, full_off);
  auto issue_tile = [&](int tt) {
    const int64_t tile_row = k_lo + static_cast<int64_t>(tt) * kTL;
    const int valid = static_cast<int>(min<int64_t>(kTL, k_hi + 1 - tile_row));
    const char* tbase = cache_c + tile_row * S::kRowBytes;
    const uint32_t dst = lds0 + (tt % kStages) * S::kTileBytes;
    if constexpr (kHoist) {
      uint32_t off[S::kDmaPerWave];
#pragma unroll
      for (int i = 0; i < S::kDmaPerWave; ++i) off[i] = full_off[i];
      if (valid < kTL) dma_offsets(valid, off);  // uniform branch, last tile only
#pragma unroll
      for (int i = 0; i < S::kDmaPerWave; ++i) {
        const int j = min(wave + S::kWaves * i, S::kDmaOps - 1);
        global_to_lds16(tbase, off[i], __builtin_amdgcn_readfirstlane(dst + j * 1024));
      }
    } else {
      int ln = lane;
      __asm__ volatile("" : "+v"(ln));
#pragma unroll
      for (int i = 0; i < S::kDmaPerWave; ++i) {
        const int j = min(wave + S::kWaves * i, S::kDmaOps - 1);  // duplicates of the last copy are benign
        const int L = j * 64 + ln;
        const int r = L / S::kRowChunks;
        const int g = r < valid ? (L ^ row_key(r)) : (valid - 1) * S::kRowChunks + (L & 7);
        global_to_lds16(tbase, static_cast<uint32_t>(g * 16), __builtin_amdgcn_readfirstlane(dst + j * 1024));
      }
    }
  };
  auto wait_tile = [&](int tt, int last_issued) {
    switch (last_issued - tt) {
      case 0: wait_tiles_after<0, S::kDmaPerWave>(); break;
      case 1: wait_tiles_after<1, S::kDmaPerWave>(); break;
      default: wait_tiles_after<2, S::kDmaPerWave>(); break;
    }
  };

  // ---- Qᵀ of the columns: B operand, lane = column l16, k = 32ks + 8lg + e
  const int64_t tq = active ? t : 0;
  const int per_group = n_heads / n_groups;
  bf16x8 qf[S::kSteps];
#pragma unroll
  for (int ks = 0; ks < S::kSteps; ++ks) {
    const int k0 = ks * 32 + lg * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (k0 < R) {
      v = *reinterpret_cast<const uint4*>(q_lat + (tq * n_heads + hc) * R + k0);
    } else {
      const int g = (k0 - R) / d_rope, j0 = (k0 - R) - g * d_rope;
      if (g == hc / per_group)
        v = *reinterpret_cast<const uint4*>(q_pe + (tq * n_heads + hc) * d_rope + j0);
    }
    qf[ks] = __builtin_bit_cast(bf16x8, v);
  }
  const float qk_scale = scale * kLog2e;
  wait_vmcnt<0>();  // Q landed before any tile copy is in flight

  const int a_off0 = l16 * S::kRowBytes, a_off1 = (16 + l16) * S::kRowBytes;
  const int x_even = (lg ^ row_key(l16)) & 7;
  const int x_odd = ((4 + lg) ^ row_key(l16)) & 7;
  const int r_lo = lg * 4 + (l16 >> 2), r_hi = 16 + r_lo;
  const int c_sub = (l16 & 1) * 8, c_half = (l16 & 3) >> 1;

  // Softmax state of column l16 (base 2): the reference is the max of the
  // column's first tile with a valid key; no running max is kept.  A pass in
  // which a weight passes 2^64 (its row sum then exceeds 2^64, or is inf/NaN)
  // is redone after a max-only scan with each column's true max.
  constexpr float kNoRef = -1e30f;   // reference before a column's first valid key
  const bf16x2_t ones = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);  // row sums by v_dot2
  float m_ref = kNoRef;
  float m_lane = -INFINITY, l_lane = 0.f;
  f32x4 o[S::kNB];

  // the wave's tiles need the mask only where they cross a column's sequence
  // start or its own token (or some column is past the last token)
  int64_t lo_max = active ? seq_lo : INT64_MAX;
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) lo_max = max(lo_max, static_cast<int64_t>(__shfl_xor(lo_max, d, 64)));
  const bool all_active = __builtin_amdgcn_ballot_w64(!active) == 0;
  auto needs_mask = [&](int64_t row0) { return !all_active || row0 < lo_max || row0 + kTL - 1 > wave_t0; };
  auto mask = [&](f32x4 (&s)[2], int64_t row0) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t kr = row0 + rb * 16 + lg * 4 + i;
        s[rb][i] = (active && kr >= seq_lo && kr <= t) ? s[rb][i] : -INFINITY;
      }
  };
  auto raw_max = [&](const f32x4 (&s)[2]) {
    return fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                 fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
  };
  auto ref_missing = [&]() { return __builtin_amdgcn_ballot_w64(active && m_ref == kNoRef) != 0; };

  auto run_pass = [&](auto scan_c) {
    constexpr bool kScan = decltype(scan_c)::value;
#pragma unroll
    for (int nb = 0; nb < S::kNB; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_lane = -INFINITY;
    l_lane = 0.f;
    bool need_ref = !kScan && ref_missing();

#pragma unroll
    for (int tt = 0; tt < kStages - 1; ++tt)
      if (tt < n_tiles) issue_tile(tt);
    int issued = min(kStages - 1, n_tiles) - 1;

    for (int tt = 0; tt < n_tiles; ++tt) {
      wait_tile(tt, issued);
      lds_barrier();  // tile tt landed everywhere; tile tt-1's buffer is free
      if (tt + kStages - 1 < n_tiles) {
        issue_tile(tt + kStages - 1);
        issued = tt + kStages - 1;
      }
      const unsigned char* tb = smem + (tt % kStages) * S::kTileBytes;

      // score: s[rb] = keys 16rb + 4lg + i of column l16
      f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      auto frag = [&](int ks, int off) {
        const int coff = (ks >> 1) * 128 + ((ks & 1) ? x_odd : x_even) * 16;
        return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(tb + off + coff));
      };
      bf16x8 fa[2][2];
      fa[0][0] = frag(0, a_off0);
      fa[0][1] = frag(0, a_off1);
      fa[1][0] = frag(1, a_off0);
      fa[1][1] = frag(1, a_off1);
#pragma unroll
      for (int ks = 0; ks < S::kSteps; ++ks) {
        s[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[ks & 1][0], qf[ks], s[0], 0, 0, 0);
        s[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[ks & 1][1], qf[ks], s[1], 0, 0, 0);
        if (ks + 2 < S::kSteps) {
          fa[ks & 1][0] = frag(ks + 2, a_off0);
          fa[ks & 1][1] = frag(ks + 2, a_off1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }

      // mask (each column's sequence rows up to its token), reference, weights
      const int64_t row0 = k_lo + static_cast<int64_t>(tt) * kTL;
      if (needs_mask(row0)) mask(s, row0);
      if constexpr (kScan) {
        m_lane = fmaxf(m_lane, raw_max(s));
        continue;
      }
      if (need_ref) {  // uniform; only until every column has met a valid key
        float tmax = raw_max(s);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        if (m_ref == kNoRef && tmax != -INFINITY) m_ref = tmax * qk_scale;
        need_ref = ref_missing();
      }
      const float neg = -m_ref;
      uint32_t w[4], wl[4];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const f32x4 v = s[rb];
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(v[i], qk_scale, neg));
        w[2 * rb] = pack_bf16x2(p[0], p[1]);
        w[2 * rb + 1] = pack_bf16x2(p[2], p[3]);
        // the row sum takes the bf16 weights the PV product uses
        l_lane = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[2 * rb]), ones, l_lane, false);
        l_lane = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[2 * rb + 1]), ones, l_lane, false);
        if constexpr (S::kSplitP) {
          const float h0 = __uint_as_float(w[2 * rb] << 16), h1 = __uint_as_float(w[2 * rb] & 0xFFFF0000u);
          const float h2 = __uint_as_float(w[2 * rb + 1] << 16), h3 = __uint_as_float(w[2 * rb + 1] & 0xFFFF0000u);
          wl[2 * rb] = pack_bf16x2(p[0] - h0, p[1] - h1);
          wl[2 * rb + 1] = pack_bf16x2(p[2] - h2, p[3] - h3);
          l_lane = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, wl[2 * rb]), ones, l_lane, false);
          l_lane = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, wl[2 * rb + 1]), ones, l_lane, false);
        }
      }
      const bf16x8 pa = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
      const bf16x8 pl = __builtin_bit_cast(bf16x8, make_uint4(wl[0], wl[1], wl[2], wl[3]));
      (void)pl;

      // PV: O[column][16nb + col] += P[column][keys]·C[keys][cols], K order as held
      auto cfrag = [&](int nb) {
        const int chunk = nb * 2 + c_half;
        const unsigned char* plo = tb + r_lo * S::kRowBytes + swz(chunk, r_lo) * 16 + c_sub;
        const unsigned char* phi = tb + r_hi * S::kRowBytes + swz(chunk, r_hi) * 16 + c_sub;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(plo));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(phi));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      constexpr int kLA = S::kLA;
      bf16x8 cf[kLA];
#pragma unroll
      for (int q = 0; q < kLA; ++q) cf[q] = cfrag(q);
#pragma unroll
      for (int nb = 0; nb < S::kNB; ++nb) {
        o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, cf[nb % kLA], o[nb], 0, 0, 0);
        if constexpr (S::kSplitP) o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, cf[nb % kLA], o[nb], 0, 0, 0);
        if (nb + kLA < S::kNB) cf[nb % kLA] = cfrag(nb + kLA);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    lds_barrier();  // every wave is done with the ring before another pass refills it
  };

  for (int pass = 0;; ++pass) {  // one weighing pass, or (rarely) two with a scan between
    run_pass(std::false_type{});
    if (pass == 1) break;
    const bool wave_over = __builtin_amdgcn_ballot_w64(!(l_lane <= 1.8e19f)) != 0;  // 2^64; every lane votes
    if (lane == 0) flags[wave] = wave_over ? 1 : 0;
    lds_barrier();
    int any = 0;
#pragma unroll
    for (int w = 0; w < S::kWaves; ++w) any |= flags[w];
    if (any == 0) break;
    lds_barrier();  // the flags are read everywhere before the scan refills the ring
    run_pass(std::true_type{});
    float mx = fmaxf(m_lane, __shfl_xor(m_lane, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    m_ref = mx == -INFINITY ? kNoRef : mx * qk_scale;
  }

  // ---- epilogue: l per column (lanes with l16 = column), O[column 4lg + i][16nb + l16]
  float l = l_lane;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = lg * 4 + i;
    const float lh = __shfl(l, c, 64);
    const float mh = __shfl(m_ref, c, 64);
    const int64_t tc = wave_t0 + c / n_heads;
    if (tc >= n_tokens) continue;
    const float inv = 1.f / lh;
    const int64_t row = tc * n_heads + c % n_heads;
    if (part_o != nullptr) {
      bf16_t* dst = part_o + row * R + l16;
#pragma unroll
      for (int nb = 0; nb < S::kNB; ++nb) dst[nb * 16] = f32_to_bf16(o[nb][i] * inv);
      if (l16 == 0) {
        part_ml[row * 2] = mh;
        part_ml[row * 2 + 1] = lh;
      }
    } else {
      float* dst = o_out + row * R + l16;
#pragma unroll
      for (int nb = 0; nb < S::kNB; ++nb) dst[nb * 16] = o[nb][i] * inv;
    }
  }
}

template <int R, int RW>
void launch(const AttnShape& sh, const void* q_lat, const void* q_pe, const void* cache,
            const int64_t* cu, int batch, int64_t n_tokens, float* o_out, void* part_o, float* part_ml,
            hipStream_t s) {
  using S = PShape<R, RW>;
  auto kern = prefill_mfma_kernel<R, RW>;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                      S::kLdsBytes);
  const int64_t block_tokens = static_cast<int64_t>(S::kWaves) * (kHeads / sh.H);
  const int64_t n_blocks = (n_tokens + block_tokens - 1) / block_tokens;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(n_blocks)), dim3(S::kThreads), S::kLdsBytes, s,
                     static_cast<const bf16_t*>(q_lat), static_cast<const bf16_t*>(q_pe),
                     static_cast<const bf16_t*>(cache), cu, batch, n_tokens, sh.H, sh.G, sh.d_rope, sh.scale,
                     o_out, static_cast<bf16_t*>(part_o), part_ml);
}

// Compiled shapes: (latent r, row width r + G*d_rope) with up to 16 query heads.
#define MLA_PREFILL_SHAPES(X)                                                   \
  X(256, 320) /* r = 256, one 64-wide rotary key (Zebra MLA layers)          */ \
  X(512, 512) /* one 512-wide KV head as key and value (DeepSeek-V4 variant) */

}  // namespace

bool prefill_mfma_supported(const AttnShape& sh) {
  if (sh.H < 1 || kHeads % sh.H != 0 || sh.d_rope % 8 != 0 || sh.H % sh.G != 0) return false;
#define MLA_MATCH(R_, RW_) \
  if (sh.r == R_ && sh.row_w == RW_) return true;
  MLA_PREFILL_SHAPES(MLA_MATCH)
#undef MLA_MATCH
  return false;
}

void prefill_mfma(const AttnShape& sh, const void* q_lat, const void* q_pe, const void* cache,
                  const int64_t* cu, int batch, int64_t n_tokens, int max_len, float* o_out,
                  void* part_o, float* part_ml, hipStream_t s) {
  (void)max_len;
  if (n_tokens <= 0 || batch <= 0) return;
#define MLA_LAUNCH(R_, RW_)                                                          \
  if (sh.r == R_ && sh.row_w == RW_) {                                               \
    launch<R_, RW_>(sh, q_lat, q_pe, cache, cu, batch, n_tokens, o_out, part_o, part_ml, s); \
    return;                                                                          \
  }
  MLA_PREFILL_SHAPES(MLA_LAUNCH)
#undef MLA_LAUNCH
}

}  // namespace mla
