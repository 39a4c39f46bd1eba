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
// Inputs: k_nope [H, T, 128] and v [H, T, 128] in fp16 (expanded by the
// caller), the rotary keys straight from the bf16 latent cache rows, q_nope
// [T, H, 128] and q_pe [T, H, DR] in bf16.  Output [T, H, 128] bf16.
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
//     lane-local max and the softmax needs no cross-lane traffic;
//   - softmax against one reference per query (base 2): the max of the first
//     tile in which the query has a valid key, with 2^15 of headroom (P is
//     fp16).  A pass
//     in which some later score passes the headroom is redone with each
//     query's true max, so O is never rescaled and stays in the matrix
//     accumulators for the whole pass;
//   - Oᵀ[128 dims x 64 queries] += Vᵀ·Pᵀ: the fp16 weights go straight from the
//     score registers into the B operand (the product's K order is the order
//     in which a lane holds its keys); Vᵀ fragments are transposed reads
//     (ds_read_b64_tr_b16) of the V tile at the matching key rows.
// The score of tile t+1 is issued before the softmax and PV of tile t, so the
// matrix cores stay busy while the softmax runs.
// Tiles stream HBM -> LDS with global_load_lds_dwordx4 through a 4-stage ring;
// each tile's 20 one-KB copies are spread over the waves.
#include <math.h>

#include <algorithm>

#include "lds_dma.h"
#include "mla_device.h"
#include "mla_internal.h"

#ifndef MLA_PREFILL_FA_WAVES
#define MLA_PREFILL_FA_WAVES 8  // waves per workgroup (4: one per SIMD, 8: two per SIMD)
#endif

namespace mla {

namespace {

constexpr int kDN = 128;            // d_nope (key/query dims without position)
constexpr int kDV = 128;            // d_v
constexpr int kBM = 256;            // queries per workgroup
constexpr int kBN = 32;             // keys per tile
constexpr int kStages = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSlack = 15.f;      // headroom (base 2) of the reference: P <= 2^15 fits fp16
constexpr float kNoMax = -1e30f;    // reference before a query's first valid key

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

template <int DR>
struct FShape {
  static_assert(DR % 16 == 0 && DR >= 64 && DR <= 128, "rotary width");
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
  static constexpr int kKrRowsPer256 = 16 / kKrChunks;
  static constexpr int kKS = (kDN + DR) / 16;       // score k-steps
  static constexpr int kFlagsOff = kStages * kStageBytes;
  static constexpr int kLdsBytes = kFlagsOff + 64;
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
};

// XOR keys of the 16-byte chunk slots.  A fragment read of 16 key rows at one
// chunk (k_nope, rotary key) and a transposed read of 4 V rows x 2 chunks then
// land on distinct banks.
__device__ __forceinline__ int kn_key(int row) { return row & 15; }
template <int DR>
__device__ __forceinline__ int kr_key(int row) {
  using S = FShape<DR>;
  return (row / S::kKrRowsPer256) & (S::kKrChunks - 1);
}
__device__ __forceinline__ int v_key(int row) { return 4 * (row & 3); }

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

template <int DR, int W>
__global__ __launch_bounds__(64 * W, 1) void prefill_fa_kernel(
    const bf16_t* __restrict__ q_nope, const bf16_t* __restrict__ q_pe,
    const _Float16* __restrict__ k_nope, const _Float16* __restrict__ v,
    const bf16_t* __restrict__ cache, const int64_t* __restrict__ cu, int batch, int n_tokens,
    int n_heads, int heads_per_group, int row_w, int r, float scale, bf16_t* __restrict__ out) {
  using S = FShape<DR>;
  constexpr int kQB = 8 / W;          // 32-query column blocks per wave
  constexpr int kQW = 32 * kQB;       // queries per wave
  static_assert(W * kQW == kBM && S::kKnOps % W == 0 && S::kVOps % W == 0, "wave split");
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

  // ---- key range of the workgroup and of this wave (tiles of kBN rows from k_lo)
  const int k_lo = seq_start(q0);
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
  // rows past k_hi repeat row k_hi (finite values, masked out).
  const char* kn_head = reinterpret_cast<const char*>(k_nope + static_cast<int64_t>(head) * n_tokens * kDN);
  const char* v_head = reinterpret_cast<const char*>(v + static_cast<int64_t>(head) * n_tokens * kDV);
  const char* kr_col = reinterpret_cast<const char*>(cache) +
                       static_cast<int64_t>(r + (head / heads_per_group) * DR) * 2;
  const int row_bytes = row_w * 2;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u8*)smem));

  auto issue_tile = [&](int tt) {
    const int kt0 = k_lo + tt * kBN;
    const int valid = min(kBN, k_hi + 1 - kt0);
    const uint32_t dst = lds0 + (tt % kStages) * S::kStageBytes;
    int ln = lane;
    __asm__ volatile("" : "+v"(ln));
    const char* kn_t = kn_head + static_cast<int64_t>(kt0) * (kDN * 2);
    const char* v_t = v_head + static_cast<int64_t>(kt0) * (kDV * 2);
    const char* kr_t = kr_col + static_cast<int64_t>(kt0) * row_bytes;
#pragma unroll
    for (int i = 0; i < S::kKnOps / W; ++i) {
      const int j = wave + W * i;
      const int L = j * 64 + ln;
      const int row = L >> 4, p = L & 15;
      const int rr = min(row, valid - 1);
      global_to_lds16(kn_t, static_cast<uint32_t>(rr * (kDN * 2) + ((p ^ kn_key(row)) << 4)),
                      __builtin_amdgcn_readfirstlane(dst + j * 1024));
    }
#pragma unroll
    for (int i = 0; i < S::kVOps / W; ++i) {
      const int j = wave + W * i;
      const int L = j * 64 + ln;
      const int row = L >> 4, p = L & 15;
      const int rr = min(row, valid - 1);
      global_to_lds16(v_t, static_cast<uint32_t>(rr * (kDV * 2) + ((p ^ v_key(row)) << 4)),
                      __builtin_amdgcn_readfirstlane(dst + S::kVOff + j * 1024));
    }
#pragma unroll
    for (int i = 0; i < (S::kKrOps + W - 1) / W; ++i) {
      const int j = wave + W * i;
      if (j < S::kKrOps) {
        const int L = j * 64 + ln;
        const int row = L / S::kKrChunks, p = L % S::kKrChunks;
        const int rr = min(row, valid - 1);
        global_to_lds16(kr_t, static_cast<uint32_t>(rr * row_bytes + ((p ^ kr_key<DR>(row)) << 4)),
                        __builtin_amdgcn_readfirstlane(dst + S::kKrOff + j * 1024));
      }
    }
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
  // K: lane reads key row l32, dims 16ks + 8hh .. +7
  const int kn_base = l32 * (kDN * 2);
  const int kn_x = kn_key(l32);
  const int kr_base = S::kKrOff + l32 * (DR * 2);
  const int kr_x = kr_key<DR>(l32);
  auto kfrag = [&](const unsigned char* st, int ks) {
    int off;
    if (ks < kDN / 16) off = kn_base + (((2 * ks + hh) ^ kn_x) << 4);
    else off = kr_base + (((2 * (ks - kDN / 16) + hh) ^ kr_x) << 4);
    return *reinterpret_cast<const uint4*>(st + off);
  };
  // Vᵀ: lane (group g = lane / 16, s = lane % 16) addresses row 4hh + s/4 (+ 16 ks2,
  // + 8 for the second read), dims 32db + 16(g & 1) + 4(s & 3); it receives dim
  // 32db + l32 at 4 consecutive key rows.
  const int vs = lane & 15;
  const int v_row = 4 * hh + (vs >> 2);
  const int v_x = v_key(v_row);
  const int v_chunk = 2 * ((lane >> 4) & 1) + ((vs & 3) >> 1);
  const int v_sub = 8 * (vs & 1);
  auto vfrag = [&](const unsigned char* st, int db, int ks2) {
    const int col = ((((4 * db) + v_chunk) ^ v_x) << 4) + v_sub;
    const unsigned char* plo = st + S::kVOff + (16 * ks2 + v_row) * (kDV * 2) + col;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(plo));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(plo + 8 * (kDV * 2)));
    return __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // Sᵀ[qb][i]: key 8(i/4) + 4hh + (i%4) of the tile, query qv[qb]
  auto score = [&](const unsigned char* st, f32x16 (&sc)[kQB]) {
    const f32x16 z = {};
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) sc[qb] = z;
    uint4 kf[2];
    kf[0] = kfrag(st, 0);
#pragma unroll
    for (int ks = 0; ks < S::kKS; ++ks) {
      if (ks + 1 < S::kKS) kf[(ks + 1) & 1] = kfrag(st, ks + 1);
      if (ks < kKN) {
        const f16x8 a = __builtin_bit_cast(f16x8, kf[ks & 1]);
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
          sc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qn[qb][ks], sc[qb], 0, 0, 0);
      } else {
        const bf16x8 a = __builtin_bit_cast(bf16x8, kf[ks & 1]);
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
        const int key = kt0 + 8 * (i >> 2) + 4 * hh + (i & 3);
        sc[qb][i] = (key >= qst[qb] && key <= qv[qb]) ? sc[qb][i] : -INFINITY;
      }
  };

  float m_ref[kQB];  // reference per query (base 2), equal in both lane halves
  float m_lane[kQB], l_run[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) m_ref[qb] = kNoMax;
  bool over;
  f32x16 o[kQB][4];
  const f16x2 ones = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};  // row sum of the fp16 weights

  // max of the tile's scores per query; the reference is set at the query's
  // first tile with a valid key
  auto tile_max = [&](const f32x16 (&sc)[kQB]) {
    float lmax[kQB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const f32x16 s = sc[qb];
      float mx = s[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
      lmax[qb] = mx;
      m_lane[qb] = fmaxf(m_lane[qb], mx);
    }
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const float m = swap_max(lmax[qb]) * qk;
      m_ref[qb] = (m_ref[qb] == kNoMax && m != -INFINITY) ? m : m_ref[qb];
      over = over || (lmax[qb] * qk > m_ref[qb] + kSlack);
    }
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

  int* flags = reinterpret_cast<int*>(smem + S::kFlagsOff);
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      m_lane[qb] = -INFINITY;
      l_run[qb] = 0.f;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[qb][db] = f32x16{};
    }
    over = false;

    auto tile_scores = [&](int t, f32x16 (&sc)[kQB]) { score(smem + (t % kStages) * S::kStageBytes, sc); };
    // Every active wave takes every tile of the workgroup's range: tiles outside
    // its own queries' ranges are masked out (a few tiles per workgroup).
    // Iteration t issues the scores of tile t+1 before the softmax and PV of
    // tile t, so the matrix core has work while the softmax runs.
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
      tile_max(cur);
      tile_scores(t + 1, nxt);  // past the last tile this reads a stale buffer; unused
      weights(cur);
      pv(smem + (t % kStages) * S::kStageBytes);
    };
    for (int t = 0; t < n_tiles; t += 2) {
      iter(t, sa, sb);
      if (t + 1 < n_tiles) iter(t + 1, sb, sa);
    }

    lds_barrier();
    if (lane == 0) flags[wave] = __builtin_amdgcn_ballot_w64(over) != 0 ? 1 : 0;
    lds_barrier();
    int any = 0;
#pragma unroll
    for (int i = 0; i < W; ++i) any |= flags[i];
    if (any == 0) break;
    // second pass with each query's true max
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const float m = swap_max(m_lane[qb]) * qk;
      m_ref[qb] = m == -INFINITY ? kNoMax : m;
    }
    lds_barrier();  // flags read everywhere before they are rewritten
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

template <int DR, int W>
void launch_fa(const AttnShape& sh, const void* q_nope, const void* q_pe, const void* k_nope,
               const void* v, const void* cache, const int64_t* cu, int batch, int n_tokens,
               void* out, hipStream_t s) {
  using S = FShape<DR>;
  auto kern = prefill_fa_kernel<DR, W>;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                      S::kLdsBytes);
  const int n_qt = (n_tokens + kBM - 1) / kBM;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(n_qt), static_cast<unsigned>(sh.H)), dim3(64 * W),
                     S::kLdsBytes, s, static_cast<const bf16_t*>(q_nope), static_cast<const bf16_t*>(q_pe),
                     static_cast<const _Float16*>(k_nope), static_cast<const _Float16*>(v),
                     static_cast<const bf16_t*>(cache), cu, batch, n_tokens, sh.H, sh.H / sh.G, sh.row_w,
                     sh.r, sh.scale, static_cast<bf16_t*>(out));
}

}  // namespace

bool prefill_expanded_supported(const AttnShape& sh, int d_nope, int d_v) {
  return d_nope == kDN && d_v == kDV && sh.d_rope == 64 && sh.H % sh.G == 0 && sh.H <= 65535 &&
         sh.row_w % 8 == 0 && sh.r % 8 == 0;
}

void prefill_expanded(const AttnShape& sh, const void* q_nope, const void* q_pe, const void* k_nope,
                      const void* v, const void* cache, const int64_t* cu, int batch, int64_t n_tokens,
                      void* out, hipStream_t s) {
  if (n_tokens <= 0 || batch <= 0) return;
  launch_fa<64, MLA_PREFILL_FA_WAVES>(sh, q_nope, q_pe, k_nope, v, cache, cu, batch, static_cast<int>(n_tokens), out, s);
}

}  // namespace mla
