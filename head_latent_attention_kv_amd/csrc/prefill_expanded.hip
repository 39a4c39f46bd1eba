// bf16 MFMA causal prefill in the original (non-absorbed) order.
//
// MLA principle page, section "原始顺序" eqs. (1)-(2): the latent rows are first
// up-projected, k_nope = W_UK·c and v = W_UV·c per head, and attention then runs
// as ordinary multi-head attention with the key [k_nope ; kr] (kr: the cached
// rotary key of the head's group) and the query [q_nope ; q_pe].  For a long
// prefill this order is the cheaper one: per (query, key, head) it costs
// 2(d_nope + d_rope) + 2 d_v flops against 2(r + d_rope) + 2r for the absorbed
// form, and the up-projection is paid once per key row, not once per query.
// Causal rule (nanowhale page, SDPA with is_causal): token t attends to the
// rows cu[b] .. t of its own sequence.
//
// Inputs: k_nope [H, T, 128] and vᵀ [H, 128, T_pad] in fp16 (expanded by the
// caller; T_pad = T rounded up to 32, the pad columns zero), the rotary keys
// straight from the bf16 latent cache rows, q_nope [T, H, 128] and q_pe
// [T, H, DR] in bf16.  Output [T, H, 128] bf16.
// Precision: this order rounds two intermediates the absorbed order does not
// (the expanded keys and values), so they, q_nope and the weights P are fp16
// inside the kernel (11 significant bits against bf16's 8, same MFMA rate).
// The rotary part of the score stays bf16; both parts accumulate into one
// fp32 tile.  fp16 bounds |k_nope|, |v| and |q_nope| to 65504.
//
// Workgroup = W wave64s on 256 consecutive query tokens of one head; each wave
// owns 256/W queries (8/W 32-wide MFMA column blocks): with W = 4 every K or V
// fragment read from LDS feeds two MFMAs, with W = 8 two waves share each SIMD
// and hide each other's LDS and softmax latencies.  Per 32-key tile:
//   - Sᵀ[32 keys x 64 queries] = K·Qᵀ with v_mfma_f32_32x32x16_bf16: key rows
//     as the A operand from LDS, Qᵀ as the B operand held in registers.  In
//     this orientation a lane owns one query column, so the row max is a
//     lane-local max and the softmax needs no cross-lane traffic.  The A
//     operand's rows are a permutation of the tile's keys chosen so that each
//     lane's 16 accumulator values are 16 consecutive keys;
//   - softmax against one reference per query (base 2): the max of the first
//     tile in which the query has a valid key.  No running max is kept: a
//     weight past fp16's range (a later score about 16 or more above the
//     reference, in log2 units) turns the row sum into inf, and such a pass is
//     redone after a max-only scan with each query's true max.  O is never
//     rescaled and stays in the matrix accumulators for the whole pass;
//   - Oᵀ[128 dims x 64 queries] += Vᵀ·Pᵀ: the fp16 weights go straight from the
//     score registers into the B operand, so each lane contributes 8
//     consecutive keys per MFMA, and a Vᵀ fragment is one 16-byte read of a
//     vᵀ row (the V tile is staged transposed, [128 dims][32 keys]).
// Key tiles are aligned to 32 keys, so every vᵀ chunk is 16-byte aligned.
// The score of tile t+1 is issued before the softmax and PV of tile t, so the
// matrix cores stay busy while the softmax runs.
// Tiles stream HBM -> LDS with global_load_lds_dwordx4 through a 4-stage ring;
// each tile's 20 one-KB copies are spread over the waves.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "lds_dma.h"
#include "mla_device.h"
#include "mla_internal.h"



namespace mla {

namespace {

// waves per workgroup and 32-query blocks per wave: 8 x 1, one workgroup of
// 256 queries per CU (two workgroups of 4 x 1 per CU, with separate barriers,
// and 4 x 2 with one wave per SIMD are both slower)
constexpr int kWavesFA = 8;
constexpr int kQBFA = 1;
constexpr int kDN = 128;            // d_nope (key/query dims without position)
constexpr int kDV = 128;            // d_v
constexpr int kBN = 32;             // keys per tile
constexpr int kStages = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNoMax = -1e30f;    // reference before a query's first valid key

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;

template <int DR>
struct FShape {
  static_assert(DR == 64, "rotary width (the chunk keys assume 128-byte rotary rows)");
  static constexpr int kKnBytes = kBN * kDN * 2;
  static constexpr int kKrBytes = kBN * DR * 2;
  static constexpr int kVBytes = kBN * kDV * 2;
  static constexpr int kKrOff = kKnBytes;
  static constexpr int kVOff = kKnBytes + kKrBytes;
  static constexpr int kStageBytes = kVOff + kVBytes;
  static constexpr int kKnOps = kKnBytes / 1024;
  static constexpr int kKrOps = kKrBytes / 1024;
  static constexpr int kVOps = kVBytes / 1024;
  static constexpr int kOps = kKnOps + kKrOps + kVOps;
  static constexpr int kKrChunks = DR / 8;          // 16-byte chunks of a rotary row
  static constexpr int kKS = (kDN + DR) / 16;       // score k-steps
  // the restart flags alias the start of the ring (idle between passes)
  static constexpr int kLdsBytes = kStages * kStageBytes;
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
};

// Score row r of the A operand holds key kperm(r) of the tile: the accumulator
// rows 8a + 4h + b that lane half h holds (a, b < 4) are keys 16h + 4a + b.
__device__ __forceinline__ int kperm(int r) { return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3); }

// XOR keys of the 16-byte chunk slots, so that the 16 (or 8) lanes a fragment
// read serves at once land on distinct banks.  Lanes 16g .. 16g+15 of a score
// read take key rows with bits {0, 1, 2, 4} varying (bit 3 = g); lanes 16g ..
// 16g+15 of a vᵀ read take dim rows 16g' .. 16g'+15.
__device__ __forceinline__ int kn_key(int row) {  // 256-byte rows: a 4-bit key
  return (row & 3) | ((row >> 2) & 4) | ((row << 1) & 8);
}
__device__ __forceinline__ int kr_key(int row) {  // 128-byte rows: a 3-bit key
  return ((row >> 1) & 1) | (((row >> 4) & 1) << 1) | (((row ^ (row >> 2)) & 1) << 2);
}
__device__ __forceinline__ int v_key(int row) {   // 64-byte rows: a 2-bit key
  return (((row >> 2) ^ (row >> 1)) & 1) | ((((row >> 3) ^ (row >> 1)) & 1) << 1);
}

__device__ __forceinline__ float swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Eight bf16 values (raw bits) -> fp16, through fp32 (round to nearest even).
__device__ __forceinline__ f16x8 bf16x8_to_f16(uint4 u) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  f16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 h = __builtin_convertvector(f32x2{__uint_as_float(w[i] << 16), __uint_as_float(w[i] & 0xFFFF0000u)}, f16x2);
    r[2 * i] = h[0];
    r[2 * i + 1] = h[1];
  }
  return r;
}

template <int N, int PerWave>
__device__ __forceinline__ void wait_tiles_after() {
  wait_vmcnt<N * PerWave>();
}

template <int DR, int W, int QB>
__global__ __launch_bounds__(64 * W, 8 / W) void prefill_fa_kernel(
    const bf16_t* __restrict__ q_nope, const bf16_t* __restrict__ q_pe,
    const _Float16* __restrict__ k_nope, const _Float16* __restrict__ v,
    const bf16_t* __restrict__ cache, const int64_t* __restrict__ cu, int batch, int n_tokens,
    int t_pad, int n_heads, int heads_per_group, int row_w, int r, float scale, bf16_t* __restrict__ out) {
  using S = FShape<DR>;
  constexpr int kQB = QB;             // 32-query column blocks per wave
  constexpr int kQW = 32 * kQB;       // queries per wave
  constexpr int kBM = W * kQW;        // queries per workgroup
  static_assert(S::kKnOps % W == 0 && S::kVOps % W == 0, "wave split");
  // tile copies per wave: the first kOps % W waves take one more
  constexpr int kOpsHi = (S::kOps + W - 1) / W, kOpsLo = S::kOps / W;
  static_assert(3 * kOpsHi < 64, "vmcnt range");
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int head = blockIdx.y;
  const int n_qt = (n_tokens + kBM - 1) / kBM;
  const int q0 = (n_qt - 1 - static_cast<int>(blockIdx.x)) * kBM;  // longest key ranges first
  const int qw0 = q0 + wave * kQW;

  auto seq_start = [&](int t) {  // cu[b] of the sequence holding token t
    int lo = 0, hi = batch;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (cu[mid] <= t) lo = mid;
      else hi = mid;
    }
    return static_cast<int>(cu[lo]);
  };

  // ---- key range of the workgroup and of this wave (tiles of kBN rows from k_lo,
  // aligned down to a multiple of kBN; keys before the sequence are masked)
  const int k_lo = seq_start(q0) & ~(kBN - 1);
  const int k_hi = min(q0 + kBM - 1, n_tokens - 1);
  const int n_tiles = (k_hi - k_lo + kBN) / kBN;
  const bool wave_on = qw0 < n_tokens;
  const int qwl = min(qw0 + kQW - 1, n_tokens - 1);
  const int start_last = wave_on ? seq_start(qwl) : k_lo;

  // ---- this lane's queries (column l32 of each 32-query block)
  int qv[kQB], qst[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    qv[qb] = qw0 + 32 * qb + l32;
    qst[qb] = seq_start(min(qv[qb], n_tokens - 1));
  }

  // ---- Qᵀ as B fragments: column = query, k = dims 16ks + 8hh + e; the
  // no-position part converted to fp16 (exact for bf16 values of moderate range)
  constexpr int kKN = kDN / 16;       // k-steps of the no-position part
  constexpr int kKR = S::kKS - kKN;   // k-steps of the rotary part
  f16x8 qn[kQB][kKN];
  bf16x8 qr[kQB][kKR];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const int64_t qrow = static_cast<int64_t>(min(qv[qb], n_tokens - 1)) * n_heads + head;
#pragma unroll
    for (int ks = 0; ks < kKN; ++ks) {
      qn[qb][ks] = bf16x8_to_f16(*reinterpret_cast<const uint4*>(q_nope + qrow * kDN + ks * 16 + hh * 8));
    }
#pragma unroll
    for (int ks = 0; ks < kKR; ++ks)
      qr[qb][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(q_pe + qrow * DR + ks * 16 + hh * 8));
  }
  const float qk = scale * kLog2e;
  wait_vmcnt<0>();  // queries and sequence bounds landed before any tile copy is in flight

  // ---- tile copies.  LDS chunk slot p of a row holds global chunk p ^ key(row);
  // key rows past k_hi repeat row k_hi, and vᵀ columns past T are the zero pad
  // (finite values, masked out).
  const char* kn_head = reinterpret_cast<const char*>(k_nope + static_cast<int64_t>(head) * n_tokens * kDN);
  const char* v_head = reinterpret_cast<const char*>(v + static_cast<int64_t>(head) * kDV * t_pad);
  const uint32_t vt_row = static_cast<uint32_t>(t_pad) * 2;  // 128 rows of it fit 32 bits (host check)
  const char* kr_col = reinterpret_cast<const char*>(cache) +
                       static_cast<int64_t>(r + (head / heads_per_group) * DR) * 2;
  const int row_bytes = row_w * 2;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u8*)smem));

  // Per-lane source offsets of this wave's copies, computed once: row clamping
  // (rows past k_hi repeat row k_hi) changes them only in a ragged last tile.
  constexpr int kKnW = S::kKnOps / W, kVW = S::kVOps / W, kKrW = (S::kKrOps + W - 1) / W;
  auto dma_offsets = [&](int valid, uint32_t (&okn)[kKnW], uint32_t (&ov)[kVW], uint32_t (&okr)[kKrW]) {
    int ln = lane;
    __asm__ volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < kKnW; ++i) {
      const int L = (wave + W * i) * 64 + ln;
      const int row = L >> 4, p = L & 15;
      okn[i] = static_cast<uint32_t>(min(row, valid - 1) * (kDN * 2) + ((p ^ kn_key(row)) << 4));
    }
#pragma unroll
    for (int i = 0; i < kVW; ++i) {  // vᵀ: 128 dim rows of 64 bytes (32 keys)
      const int L = (wave + W * i) * 64 + ln;
      const int row = L >> 2, p = L & 3;
      ov[i] = static_cast<uint32_t>(row) * vt_row + static_cast<uint32_t>((p ^ v_key(row)) << 4);
    }
#pragma unroll
    for (int i = 0; i < kKrW; ++i) {
      const int L = (wave + W * i) * 64 + ln;
      const int row = L / S::kKrChunks, p = L % S::kKrChunks;
      okr[i] = static_cast<uint32_t>(min(row, valid - 1) * row_bytes + ((p ^ kr_key(row)) << 4));
    }
  };
  uint32_t full_kn[kKnW], full_v[kVW], full_kr[kKrW];
  dma_offsets(kBN, full_kn, full_v, full_kr);

  auto issue_tile = [&](int tt) {
    const int kt0 = k_lo + tt * kBN;
    const int valid = min(kBN, k_hi + 1 - kt0);
    const uint32_t dst = lds0 + (tt % kStages) * S::kStageBytes;
    const char* kn_t = kn_head + static_cast<int64_t>(kt0) * (kDN * 2);
    const char* v_t = v_head + static_cast<int64_t>(kt0) * 2;
    const char* kr_t = kr_col + static_cast<int64_t>(kt0) * row_bytes;
    uint32_t okn[kKnW], ov[kVW], okr[kKrW];
#pragma unroll
    for (int i = 0; i < kKnW; ++i) okn[i] = full_kn[i];
#pragma unroll
    for (int i = 0; i < kVW; ++i) ov[i] = full_v[i];
#pragma unroll
    for (int i = 0; i < kKrW; ++i) okr[i] = full_kr[i];
    if (valid < kBN) dma_offsets(valid, okn, ov, okr);  // uniform branch, last tile only
#pragma unroll
    for (int i = 0; i < kKnW; ++i)
      global_to_lds16(kn_t, okn[i], __builtin_amdgcn_readfirstlane(dst + (wave + W * i) * 1024));
#pragma unroll
    for (int i = 0; i < kVW; ++i)
      global_to_lds16(v_t, ov[i], __builtin_amdgcn_readfirstlane(dst + S::kVOff + (wave + W * i) * 1024));
#pragma unroll
    for (int i = 0; i < kKrW; ++i)
      if (wave + W * i < S::kKrOps)
        global_to_lds16(kr_t, okr[i], __builtin_amdgcn_readfirstlane(dst + S::kKrOff + (wave + W * i) * 1024));
  };
  const bool ops_hi = wave < S::kOps % W || S::kOps % W == 0;
  auto wait_tile = [&](int tt, int last_issued) {
    const int d = last_issued - tt;
    if (ops_hi) {
      if (d == 0) wait_tiles_after<0, kOpsHi>();
      else if (d == 1) wait_tiles_after<1, kOpsHi>();
      else wait_tiles_after<2, kOpsHi>();
    } else {
      if (d == 0) wait_tiles_after<0, kOpsLo>();
      else if (d == 1) wait_tiles_after<1, kOpsLo>();
      else wait_tiles_after<2, kOpsLo>();
    }
  };

  // ---- fragment addressing (byte offsets inside a stage)
  // K: lane reads key row kperm(l32), dims 16ks + 8hh .. +7
  const int krow = kperm(l32);
  const int kn_base = krow * (kDN * 2);
  const int kn_x = kn_key(krow);
  const int kr_base = S::kKrOff + krow * (DR * 2);
  const int kr_x = kr_key(krow);
  auto kfrag = [&](const unsigned char* st, int ks) {
    int off;
    if (ks < kDN / 16) off = kn_base + (((2 * ks + hh) ^ kn_x) << 4);
    else off = kr_base + (((2 * (ks - kDN / 16) + hh) ^ kr_x) << 4);
    return *reinterpret_cast<const uint4*>(st + off);
  };
  // Vᵀ: lane reads dim row 32db + l32 at keys 16hh + 8s2 .. +7 (chunk 2hh + s2);
  // the row's key depends on l32 only (32db keeps bits 0..3)
  const int v_x = v_key(l32);
  auto vfrag = [&](const unsigned char* st, int db, int s2) {
    const int off = S::kVOff + (32 * db + l32) * (kBN * 2) + (((2 * hh + s2) ^ v_x) << 4);
    return *reinterpret_cast<const f16x8*>(st + off);
  };

  // Sᵀ[qb][i]: key 16hh + i of the tile, query qv[qb]
  auto score = [&](const unsigned char* st, f32x16 (&sc)[kQB]) {
    const f32x16 z = {};
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) sc[qb] = z;
    constexpr int kPF = 2;  // K fragments in flight
    uint4 kf[kPF];
#pragma unroll
    for (int i = 0; i < kPF - 1; ++i) kf[i] = kfrag(st, i);
#pragma unroll
    for (int ks = 0; ks < S::kKS; ++ks) {
      if (ks + kPF - 1 < S::kKS) kf[(ks + kPF - 1) % kPF] = kfrag(st, ks + kPF - 1);
      if (ks < kKN) {
        const f16x8 a = __builtin_bit_cast(f16x8, kf[ks % kPF]);
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
          sc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qn[qb][ks], sc[qb], 0, 0, 0);
      } else {
        const bf16x8 a = __builtin_bit_cast(bf16x8, kf[ks % kPF]);
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
          sc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qr[qb][ks - kKN], sc[qb], 0, 0, 0);
      }
    }
  };
  auto mask = [&](f32x16 (&sc)[kQB], int kt0) {
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kt0 + 16 * hh + i;
        sc[qb][i] = (key >= qst[qb] && key <= qv[qb]) ? sc[qb][i] : -INFINITY;
      }
  };

  float m_ref[kQB];  // reference per query (base 2), equal in both lane halves
  float m_lane[kQB], l_run[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) m_ref[qb] = kNoMax;
  f32x16 o[kQB][4];
  const f16x2 ones = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};  // row sum of the fp16 weights

  auto lane_max = [&](const f32x16& s) {
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    return mx;
  };
  // The reference of a query is set at its first tile with a valid key.
  auto set_ref = [&](const f32x16 (&sc)[kQB]) {
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const float m = swap_max(lane_max(sc[qb])) * qk;
      m_ref[qb] = (m_ref[qb] == kNoMax && m != -INFINITY) ? m : m_ref[qb];
    }
  };
  auto ref_missing = [&]() {
    bool miss = false;
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) miss = miss || m_ref[qb] == kNoMax;
    return __builtin_amdgcn_ballot_w64(miss) != 0;
  };
  // running max of the scores (the rare max-only pass)
  auto scan_max = [&](const f32x16 (&sc)[kQB]) {
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) m_lane[qb] = fmaxf(m_lane[qb], lane_max(sc[qb]));
  };
  // w[qb][k]: fp16 pair (p_2k, p_2k+1) of query block qb
  uint32_t w[kQB][8];
  auto weights = [&](const f32x16 (&sc)[kQB]) {
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const f32x16 s = sc[qb];
      const float neg = -m_ref[qb];
      float acc = l_run[qb];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * k], qk, neg));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * k + 1], qk, neg));
        const f16x2 ph = __builtin_convertvector(f32x2{p0, p1}, f16x2);
        w[qb][k] = __builtin_bit_cast(uint32_t, ph);
        acc = __builtin_amdgcn_fdot2(ph, ones, acc, false);
      }
      l_run[qb] = acc;
    }
  };
  auto pv = [&](const unsigned char* st) {
    f16x8 pb[kQB][2];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        pb[qb][s2] = __builtin_bit_cast(
            f16x8, make_uint4(w[qb][4 * s2], w[qb][4 * s2 + 1], w[qb][4 * s2 + 2], w[qb][4 * s2 + 3]));
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const f16x8 a = vfrag(st, db, s2);
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
          o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb[qb][s2], o[qb][db], 0, 0, 0);
      }
  };

  // Passes: 0 weighs every tile against the first-tile reference.  A weight
  // past fp16's range (a later score more than ~2^16 above the reference)
  // turns the row sum into inf; then pass 1 scans the true max of every
  // query and pass 2 weighs again against it.  All waves take the same passes.
  int* flags = reinterpret_cast<int*>(smem);  // restart flags, in the idle ring between passes
  auto tile_scores = [&](int t, f32x16 (&sc)[kQB]) { score(smem + (t % kStages) * S::kStageBytes, sc); };
  // One pass over the workgroup's tiles: weights and PV, or (kScan) the running
  // max only.  Every active wave takes every tile of the workgroup's range:
  // tiles outside its own queries' ranges are masked out (a few tiles per
  // workgroup).  Iteration t issues the scores of tile t+1 before the softmax
  // and PV of tile t, so the matrix core has work while the softmax runs.
  auto run_pass = [&](auto scan_c) {
    constexpr bool kScan = decltype(scan_c)::value;
    bool need_ref = !kScan && ref_missing();
#pragma unroll
    for (int tt = 0; tt < kStages - 1; ++tt)
      if (tt < n_tiles) issue_tile(tt);
    int issued = min(kStages - 1, n_tiles) - 1;
    wait_tile(0, issued);
    lds_barrier();
    f32x16 sa[kQB], sb[kQB];
    if (wave_on) tile_scores(0, sa);
    auto iter = [&](int t, f32x16 (&cur)[kQB], f32x16 (&nxt)[kQB]) {
      if (t + 1 < n_tiles) wait_tile(t + 1, issued);
      lds_barrier();  // tile t+1 landed everywhere; tile t-1's buffer is free
      if (t + kStages - 1 < n_tiles) {
        issue_tile(t + kStages - 1);
        issued = t + kStages - 1;
      }
      if (!wave_on) return;
      const int kt0 = k_lo + t * kBN;
      if (kt0 + kBN - 1 > qw0 || kt0 < start_last) mask(cur, kt0);
      if constexpr (kScan) {
        scan_max(cur);
        tile_scores(t + 1, nxt);
      } else {
        if (need_ref) {  // uniform; only until every query of the wave has met a valid key
          set_ref(cur);
          need_ref = ref_missing();
        }
        tile_scores(t + 1, nxt);  // past the last tile this reads a stale buffer; unused
        weights(cur);
        pv(smem + (t % kStages) * S::kStageBytes);
      }
    };
    for (int t = 0; t < n_tiles; t += 2) {
      iter(t, sa, sb);
      if (t + 1 < n_tiles) iter(t + 1, sb, sa);
    }
    lds_barrier();  // every wave is done with the ring before another pass refills it
  };

  // Pass 0 weighs every tile against the first-tile reference.  A weight past
  // fp16's range (a later score about 16 or more above the reference, log2
  // units) turns the row sum into inf; then a max-only pass finds every
  // query's true max and a last pass weighs again against it.  All waves take
  // the same passes.
  auto reset = [&]() {
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      m_lane[qb] = -INFINITY;
      l_run[qb] = 0.f;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[qb][db] = f32x16{};
    }
  };
  reset();
  run_pass(std::false_type{});
  bool over = false;
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) over = over || !(l_run[qb] <= 3.0e38f);
  const bool wave_over = __builtin_amdgcn_ballot_w64(over) != 0;  // every lane votes
  if (lane == 0) flags[wave] = wave_on && wave_over ? 1 : 0;
  lds_barrier();
  int any = 0;
#pragma unroll
  for (int i = 0; i < W; ++i) any |= flags[i];
  if (any != 0) {
    lds_barrier();  // the flags are read everywhere before the scan refills the ring
    reset();
    run_pass(std::true_type{});
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const float m = swap_max(m_lane[qb]) * qk;
      m_ref[qb] = m == -INFINITY ? kNoMax : m;
    }
    reset();
    run_pass(std::false_type{});
  }

  // ---- epilogue: Oᵀ[qb][db][i] is dim 32db + 8(i/4) + 4hh + (i%4) of query qv[qb]
  if (!wave_on) return;
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    if (qv[qb] >= n_tokens) continue;
    const float l = swap_sum(l_run[qb]);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    bf16_t* dst = out + (static_cast<int64_t>(qv[qb]) * n_heads + head) * kDV + 4 * hh;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x16 a = o[qb][db];
        const uint2 pk = make_uint2(pack_bf16x2(a[4 * j] * inv, a[4 * j + 1] * inv),
                                    pack_bf16x2(a[4 * j + 2] * inv, a[4 * j + 3] * inv));
        *reinterpret_cast<uint2*>(dst + 32 * db + 8 * j) = pk;
      }
  }
}

template <int DR, int W, int QB>
void launch_fa(const AttnShape& sh, const void* q_nope, const void* q_pe, const void* k_nope,
               const void* v, const void* cache, const int64_t* cu, int batch, int n_tokens,
               void* out, hipStream_t s) {
  const int t_pad = static_cast<int>(prefill_expanded_vt_cols(n_tokens));
  using S = FShape<DR>;
  auto kern = prefill_fa_kernel<DR, W, QB>;
  constexpr int kBM = W * 32 * QB;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                      S::kLdsBytes);
  const int n_qt = (n_tokens + kBM - 1) / kBM;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(n_qt), static_cast<unsigned>(sh.H)), dim3(64 * W),
                     S::kLdsBytes, s, static_cast<const bf16_t*>(q_nope), static_cast<const bf16_t*>(q_pe),
                     static_cast<const _Float16*>(k_nope), static_cast<const _Float16*>(v),
                     static_cast<const bf16_t*>(cache), cu, batch, n_tokens, t_pad, sh.H, sh.H / sh.G, sh.row_w,
                     sh.r, sh.scale, static_cast<bf16_t*>(out));
}

}  // namespace

int64_t prefill_expanded_vt_cols(int64_t n_tokens) { return (n_tokens + kBN - 1) / kBN * kBN; }

namespace {
__global__ __launch_bounds__(256) void vt_pad_kernel(_Float16* __restrict__ vt, int64_t rows, int64_t cols,
                                                     int64_t n_tokens) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (row >= rows) return;
  for (int64_t c = n_tokens; c < cols; ++c) vt[row * cols + c] = static_cast<_Float16>(0.f);
}
}  // namespace

void prefill_expanded_vt_pad(void* vt, int64_t rows, int64_t n_tokens, hipStream_t s) {
  const int64_t cols = prefill_expanded_vt_cols(n_tokens);
  if (cols == n_tokens || rows <= 0) return;
  hipLaunchKernelGGL(vt_pad_kernel, dim3(static_cast<unsigned>((rows + 255) / 256)), dim3(256), 0, s,
                     static_cast<_Float16*>(vt), rows, cols, n_tokens);
}

bool prefill_expanded_supported(const AttnShape& sh, int d_nope, int d_v) {
  return d_nope == kDN && d_v == kDV && sh.d_rope == 64 && sh.H % sh.G == 0 && sh.H <= 65535 &&
         sh.row_w % 8 == 0 && sh.r % 8 == 0;
}

void prefill_expanded(const AttnShape& sh, const void* q_nope, const void* q_pe, const void* k_nope,
                      const void* v, const void* cache, const int64_t* cu, int batch, int64_t n_tokens,
                      void* out, hipStream_t s) {
  if (n_tokens <= 0 || batch <= 0) return;
  launch_fa<64, kWavesFA, kQBFA>(sh, q_nope, q_pe, k_nope, v, cache, cu, batch, static_cast<int>(n_tokens), out, s);
}

}  // namespace mla
