// bf16 MFMA decode over the latent cache: one query token per sequence.
//
// The heads of a sequence share every cache row (the absorbed score
// q_lat·c + q_pe·kr and the latent-space P·c both read only the cached [c ; kr]
// rows), so a workgroup takes a block of heads of one sequence and streams the
// rows of one split of its context through LDS once for all of them.  When the
// heads are split over several workgroups (NHH > 1) those workgroups are placed
// on the same XCD (workgroups are dealt to the 8 XCDs round-robin) so the
// second read of a tile is served by that XCD's L2.
//
// Workgroup = 8 wave64s.  Per 32-row tile (software-pipelined: the iteration
// that accumulates tile t also scores tile t+1, one barrier per tile):
//  1. the tile is copied HBM -> LDS with global_load_lds_dwordx4 (no register
//     staging; non-temporal when NHH = 1), STAGES-2 tiles in flight beyond
//     the two being used;
//  2. score: wave w (< 2·NHB) computes Sᵀ[16 rows x 16 heads] = C·Qᵀ for head
//     block w % NHB and row block w / NHB with v_mfma_f32_16x16x32_bf16; C (the
//     tile) is the A operand read from LDS, fetched a few k-steps ahead; Qᵀ is
//     the B operand held in registers (q_lat and the group's q_pe, zero
//     elsewhere, so one K loop covers the whole cache row);
//  3. softmax in registers against a per-split reference max (base 2): the
//     first tile's max, with 2^64 of headroom; a split whose later scores
//     exceed that finishes as a max-only scan and is redone with its true max,
//     so the accumulators are never rescaled; row sums stay per lane until the
//     end; P is written to LDS as bf16 (double-buffered);
//  4. PV: wave w owns latent columns [w·R/8, (w+1)·R/8) for all heads of the
//     workgroup; O += P·C with P (A operand) from LDS and C (B operand) read
//     transposed from the same tile with ds_read_b64_tr_b16.
// Output: normalised o_ (part_o null, one split) or the split's (m, l) and its
// normalised o_ in bf16.
#include <math.h>

#include <cmath>

#include <algorithm>

#include "lds_dma.h"
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kTL = 32;          // cache rows per tile
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kPP = 80;          // LDS bytes per head row of P (32 bf16 + pad: conflict-free reads)
constexpr int kPF = 3;           // score k-steps fetched ahead
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSlack = 64.f;   // base-2 headroom above the softmax reference (P <= 2^64)

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

// R: latent width; RW: cache row width; NHB: 16-head blocks per workgroup;
// NHH: workgroups sharing one (sequence, split); STAGES: LDS tile buffers.
template <int R, int RW, int NHB, int NHH, int STAGES>
struct Shape {
  static constexpr int kUnits = 2 * NHB;                        // (head block, row block) per tile
  static_assert(kUnits <= kWaves, "one score unit per wave at most");
  static_assert(R % (16 * kWaves) == 0, "latent width must split into 16-column blocks per wave");
  static_assert(RW % 32 == 0, "row width must be a multiple of 32");
  static constexpr int kHeads = NHB * 16;
  static constexpr int kSteps = RW / 32;                        // score k-steps
  // LDS row bytes: an odd multiple of 16, so the 16 rows one score read touches
  // start in 16 distinct 4-bank groups
  static constexpr int kPitch = ((RW * 2 / 16) | 1) * 16;
  static constexpr int kTileBytes = kTL * kPitch;
  static constexpr int kChunks = (kTileBytes + 1023) / 1024;    // 1 KB direct-load chunks per tile
  static constexpr int kCPW = (kChunks + kWaves - 1) / kWaves;  // chunks per wave (padded)
  static constexpr int kBufBytes = kChunks * 1024;
  static constexpr int kNC = R / kWaves;                        // PV columns per wave
  static constexpr int kNB = kNC / 16;
  static constexpr int kPBytes = kHeads * kPP;                  // one P buffer
  static constexpr int kRedBytes = 3 * kHeads * 4 + 2 * kWaves * 4;  // exchange array, flags, max per head
  static constexpr int kLdsBytes = STAGES * kBufBytes + 2 * kPBytes + kRedBytes;
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
  static_assert(STAGES >= 3 && STAGES <= 4, "tiles t, t+1 resident and 1-2 copies in flight");
  static_assert(2 * kCPW < 64, "vmcnt range");
};

__device__ __forceinline__ bf16x8 lds_frag(const unsigned char* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

template <int R, int RW, int NHB, int NHH, int STAGES>
__global__ __launch_bounds__(kThreads) void decode_mfma_kernel(
    const bf16_t* __restrict__ q_lat, const bf16_t* __restrict__ q_pe,
    const bf16_t* __restrict__ cache, const int64_t* __restrict__ seq_start,
    const int32_t* __restrict__ seq_len, int batch, int H, int G, int d_rope, float scale,
    int n_split, int split_len, bf16_t* __restrict__ part_o, float* __restrict__ part_ml,
    float* __restrict__ o_out, bf16_t* __restrict__ v4_out, const float* __restrict__ sink,
    double rope_base, const double* __restrict__ freqs, int tail, int ragged_items) {
  using S = Shape<R, RW, NHB, NHH, STAGES>;
  constexpr int kBufBytes = S::kBufBytes;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  unsigned char* pbuf = smem + STAGES * kBufBytes;                        // P [2][kHeads][kPP]
  float* xch = reinterpret_cast<float*>(pbuf + 2 * S::kPBytes);           // [2][kHeads]
  int* flag_lds = reinterpret_cast<int*>(xch + 2 * S::kHeads);            // [2][kWaves]
  float* m_lds = reinterpret_cast<float*>(flag_lds + 2 * kWaves);          // [kHeads] (V4 epilogue)

  // ---- which (sequence, split, head group) this workgroup computes
  int pair, hh;
  if (NHH == 1) {
    pair = blockIdx.x;
    hh = 0;
  } else {
    // the NHH workgroups of a pair are 8 apart: same XCD, dispatched together
    const int q = blockIdx.x / (8 * NHH), rem = blockIdx.x % (8 * NHH);
    hh = rem / 8;
    pair = q * 8 + rem % 8;
  }
  int split, b, len;
  int64_t slot;  // index of this (sequence, split) in the partial states
  int64_t row0;
  if (ragged_items > 0) {
    // plan made here from the lengths (NHH = 1): workgroup i takes item i;
    // every wave finds the same item, and a workgroup without one leaves.
    // Lane k loads sequence k's start beside its length, so neither waits on
    // the plan.
    const int64_t start_lane = (threadIdx.x & (kWave - 1)) < batch ? seq_start[threadIdx.x & (kWave - 1)] : 0;
    const RaggedLane rl = ragged_plan(seq_len, batch, ragged_items);
    const int item = blockIdx.x;
    const bool mine = (threadIdx.x & (kWave - 1)) < batch && item >= rl.first && item < rl.first + rl.count;
    const uint64_t owner = __ballot(mine);
    if (owner == 0) return;
    // uniform values, kept in scalar registers
    b = __builtin_amdgcn_readfirstlane(__ffsll(static_cast<unsigned long long>(owner)) - 1);
    split = __builtin_amdgcn_readfirstlane(item - __shfl(rl.first, b, kWave));
    split_len = __builtin_amdgcn_readfirstlane(rl.split_len);
    len = __builtin_amdgcn_readfirstlane(__shfl(rl.len, b, kWave));
    row0 = uniform_i64(__shfl(static_cast<long long>(start_lane), b, kWave));
    slot = item;
  } else {
    if (pair >= batch * n_split) return;
    split = pair % n_split;
    b = pair / n_split;
    slot = static_cast<int64_t>(b) * n_split + split;
    row0 = seq_start[b];
    len = seq_len[b];
  }
  const int head0 = hh * S::kHeads;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;

  const int l_begin = split * split_len;
  const int l_end = min(len, l_begin + split_len);
  const int n_tiles = l_end > l_begin ? (l_end - l_begin + kTL - 1) / kTL : 0;
  const char* cache_b = reinterpret_cast<const char*>(cache + row0 * RW);

  // ---- tile loader: chunk j of the padded tile image -> LDS [j*1 KB + lane*16]
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u8*)smem));
  auto issue_tile = [&](int t) {
    const int tile_row = l_begin + t * kTL;
    const int valid = min(kTL, l_end - tile_row);
    const char* tbase = cache_b + static_cast<int64_t>(tile_row) * (RW * 2);
    const uint32_t dst = lds0 + (t % STAGES) * kBufBytes;
#pragma unroll
    for (int i = 0; i < S::kCPW; ++i) {
      const int j = min(wave + kWaves * i, S::kChunks - 1);  // duplicates of the last chunk are benign
      const int off = j * 1024 + lane * 16;
      const int r = off / S::kPitch;          // tile row this lane's 16 bytes belong to
      int cb = off - r * S::kPitch;           // byte within the padded LDS row
      if (cb >= RW * 2) cb = 0;               // pad bytes: any valid 16 B of the row
      // rows past the sequence (last tile) or past the tile read the last valid row
      const uint32_t voff = r < valid ? static_cast<uint32_t>(r * (RW * 2) + cb)
                                      : static_cast<uint32_t>((valid - 1) * (RW * 2));
      // with one workgroup per (sequence, split) each tile is read once: non-temporal copy
      if constexpr (NHH == 1) global_to_lds16_stream(tbase, voff, __builtin_amdgcn_readfirstlane(dst + j * 1024));
      else global_to_lds16(tbase, voff, __builtin_amdgcn_readfirstlane(dst + j * 1024));
    }
  };
  // wait until tile t has landed, given that the copies of tiles up to `last_issued` were issued
  auto wait_tile = [&](int t, int last_issued) {
    const int later = last_issued - t;
    if (later >= 2) wait_vmcnt<2 * S::kCPW>();
    else if (later == 1) wait_vmcnt<S::kCPW>();
    else wait_vmcnt<0>();
  };

  // ---- score unit of this wave: head block hb, row block mb
  constexpr bool kAllUnits = S::kUnits == kWaves;
  const bool unit = kAllUnits || wave < S::kUnits;
  const int hb_s = wave % NHB, mb_s = wave / NHB;
  const int hloc = hb_s * 16 + l16;          // head (within the workgroup) of this lane's scores
  const int head = head0 + hloc;
  bf16x8 qf[S::kSteps];                      // Qᵀ B operand: lane k = 32ks + 8lg + e
  if (unit) {
    const int per_group = H / G;
#pragma unroll
    for (int ks = 0; ks < S::kSteps; ++ks) {
      const int k0 = ks * 32 + lg * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (head < H) {
        if (k0 < R) {
          v = *reinterpret_cast<const uint4*>(q_lat + (static_cast<int64_t>(b) * H + head) * R + k0);
        } else {
          const int g = (k0 - R) / d_rope, j0 = (k0 - R) - g * d_rope;
          if (g == head / per_group)
            v = *reinterpret_cast<const uint4*>(q_pe + (static_cast<int64_t>(b) * H + head) * d_rope + j0);
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

  // Scaled, masked scores Sᵀ of tile t for this unit: lane holds rows 16mb+4lg+i of head hloc.
  auto score = [&](int t) -> f32x4 {
    const unsigned char* arow = smem + (t % STAGES) * kBufBytes + (mb_s * 16 + l16) * S::kPitch + lg * 16;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    bf16x8 f[kPF];
#pragma unroll
    for (int p = 0; p < kPF; ++p) f[p] = lds_frag(arow + p * 64);
#pragma unroll
    for (int ks = 0; ks < S::kSteps; ++ks) {
      const bf16x8 x = f[ks % kPF];
      if (ks + kPF < S::kSteps) f[ks % kPF] = lds_frag(arow + (ks + kPF) * 64);
      if (ks & 1) acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, qf[ks], acc1, 0, 0, 0);
      else acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, qf[ks], acc0, 0, 0, 0);
    }
    f32x4 sv = (acc0 + acc1) * qk_scale;
    const int valid = min(kTL, l_end - (l_begin + t * kTL));  // rows past the split take no weight
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = (mb_s * 16 + lg * 4 + i < valid) ? sv[i] : -INFINITY;
    return sv;
  };

  float m_ref = -INFINITY;   // reference max of head `hloc` (same in both row blocks)
  float m_lane = -INFINITY;  // max of the scores this lane has seen in the pass
  float l_lane = 0.f;        // sum of P over the rows this lane holds
  f32x4 o[NHB][S::kNB];
  const int c0 = wave * S::kNC;  // PV column slice of this wave

  // P of tile t (relative to m_ref) -> LDS buffer t&1; returns whether a score
  // exceeds the reference by more than the slack.
  auto emit_p = [&](int t, const f32x4& sv) -> bool {
    m_lane = fmaxf(m_lane, fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
    const float lim = m_ref + kSlack;
    const bool over = (sv[0] > lim) || (sv[1] > lim) || (sv[2] > lim) || (sv[3] > lim);
    const float p0 = __builtin_amdgcn_exp2f(sv[0] - m_ref);
    const float p1 = __builtin_amdgcn_exp2f(sv[1] - m_ref);
    const float p2 = __builtin_amdgcn_exp2f(sv[2] - m_ref);
    const float p3 = __builtin_amdgcn_exp2f(sv[3] - m_ref);
    // the row sum takes the bf16 weights the PV product uses, so o_ is their exact average
    const uint32_t w01 = pack_bf16x2(p0, p1), w23 = pack_bf16x2(p2, p3);
    l_lane += bf16x2_sum(w01) + bf16x2_sum(w23);
    *reinterpret_cast<uint2*>(pbuf + (t & 1) * S::kPBytes + hloc * kPP + (mb_s * 16 + lg * 4) * 2) =
        make_uint2(w01, w23);
    return over;
  };

  // O[heads][c0 : c0+kNC] += P(t)[heads][rows] · C(t)[rows][cols]
  auto pv = [&](int t) {
    const unsigned char* tile = smem + (t % STAGES) * kBufBytes;
    const unsigned char* pb = pbuf + (t & 1) * S::kPBytes;
    bf16x8 bfrag[S::kNB];
#pragma unroll
    for (int nb = 0; nb < S::kNB; ++nb) {
      const int col = c0 + nb * 16 + 4 * (l16 & 3);
      const unsigned char* base = tile + (lg * 8 + (l16 >> 2)) * S::kPitch + col * 2;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + 4 * S::kPitch));
      bfrag[nb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    bf16x8 pf[NHB];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) pf[hb] = lds_frag(pb + (hb * 16 + l16) * kPP + lg * 16);
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int nb = 0; nb < S::kNB; ++nb)
        o[hb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[hb], bfrag[nb], o[hb][nb], 0, 0, 0);
  };

  // score(ts) and pv(tp) in one instruction stream: the operands of both are
  // fetched first, then score and PV MFMAs alternate, so the MFMA pipe has
  // independent work while LDS reads are outstanding.
  auto score_and_pv = [&](int ts, int tp) -> f32x4 {
    const unsigned char* tile = smem + (tp % STAGES) * kBufBytes;
    const unsigned char* pb = pbuf + (tp & 1) * S::kPBytes;
    bf16x8 bfrag[S::kNB];
#pragma unroll
    for (int nb = 0; nb < S::kNB; ++nb) {
      const int col = c0 + nb * 16 + 4 * (l16 & 3);
      const unsigned char* base = tile + (lg * 8 + (l16 >> 2)) * S::kPitch + col * 2;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + 4 * S::kPitch));
      bfrag[nb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    bf16x8 pf[NHB];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) pf[hb] = lds_frag(pb + (hb * 16 + l16) * kPP + lg * 16);
    const unsigned char* arow = smem + (ts % STAGES) * kBufBytes + (mb_s * 16 + l16) * S::kPitch + lg * 16;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    bf16x8 f[kPF];
#pragma unroll
    for (int p = 0; p < kPF; ++p) f[p] = lds_frag(arow + p * 64);
    constexpr int kPV = NHB * S::kNB;
#pragma unroll
    for (int ks = 0; ks < (S::kSteps > kPV ? S::kSteps : kPV); ++ks) {
      if (ks < S::kSteps) {
        const bf16x8 x = f[ks % kPF];
        if (ks + kPF < S::kSteps) f[ks % kPF] = lds_frag(arow + (ks + kPF) * 64);
        if (ks & 1) acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, qf[ks], acc1, 0, 0, 0);
        else acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, qf[ks], acc0, 0, 0, 0);
      }
      if (ks < kPV) {
        const int hb = ks / S::kNB, nb = ks % S::kNB;
        o[hb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[hb], bfrag[nb], o[hb][nb], 0, 0, 0);
      }
    }
    f32x4 sv = (acc0 + acc1) * qk_scale;
    const int valid = min(kTL, l_end - (l_begin + ts * kTL));  // rows past the split take no weight
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = (mb_s * 16 + lg * 4 + i < valid) ? sv[i] : -INFINITY;
    return sv;
  };

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int nb = 0; nb < S::kNB; ++nb) o[hb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    l_lane = 0.f;
    m_lane = -INFINITY;
    bool scan = false;  // workgroup-uniform: some score exceeded the reference's slack

#pragma unroll
    for (int t = 0; t < STAGES - 1; ++t)
      if (t < n_tiles) issue_tile(t);
    int issued = min(STAGES - 1, n_tiles) - 1;  // last tile whose copy is in flight or done

    if (n_tiles > 0) {
      // prologue: score tile 0; in the first pass its max sets the reference
      wait_tile(0, issued);
      lds_barrier();
      f32x4 sv = {0.f, 0.f, 0.f, 0.f};
      if (unit) sv = score(0);
      if (pass == 0) {
        if (unit) {
          float tmax = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
          tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
          tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
          if (lg == 0) xch[mb_s * S::kHeads + hloc] = tmax;
        }
        lds_barrier();
        if (unit) m_ref = fmaxf(xch[hloc], xch[S::kHeads + hloc]);
      }
      if (unit) {
        const bool over = __ballot(emit_p(0, sv)) != 0;  // every lane votes
        if (lane == 0) flag_lds[wave] = over ? 1 : 0;
      }
    }

    // steady state: iteration t scores tile t+1 and accumulates tile t
    for (int t = 0; t < n_tiles; ++t) {
      if (t + 1 < n_tiles) wait_tile(t + 1, issued);
      lds_barrier();  // tile t+1, P(t) and the flags of tile t are visible; tile t-1's buffer is free
      {
        int any = 0;
#pragma unroll
        for (int w = 0; w < S::kUnits; ++w) any |= flag_lds[(t & 1) * kWaves + w];
        scan = scan || (any != 0);
      }
      if (t + STAGES - 1 < n_tiles) {
        issue_tile(t + STAGES - 1);
        issued = t + STAGES - 1;
      }
      // Tile t+1 is scored even past the last tile: its rows are then all masked
      // (P = 0, no effect), which keeps this loop body free of branches.  In a
      // scan, P may be out of range; the accumulators are then discarded.
      if constexpr (kAllUnits) {
        const f32x4 sv = score_and_pv(t + 1, t);
        const bool over = __ballot(emit_p(t + 1, sv)) != 0;
        if (lane == 0) flag_lds[((t + 1) & 1) * kWaves + wave] = over ? 1 : 0;
      } else {
        if (unit) {
          const f32x4 sv = score(t + 1);
          const bool over = __ballot(emit_p(t + 1, sv)) != 0;
          if (lane == 0) flag_lds[((t + 1) & 1) * kWaves + wave] = over ? 1 : 0;
        }
        pv(t);
      }
    }
    if (!scan) break;
    // second pass with the split's true max (over all rows of both row blocks) as the reference
    float mx = m_lane;
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (unit && lg == 0) xch[mb_s * S::kHeads + hloc] = mx;
    lds_barrier();
    if (unit) m_ref = fmaxf(xch[hloc], xch[S::kHeads + hloc]);
    lds_barrier();
  }

  // ---- epilogue: l = sum over the lanes and both row blocks; O normalised or as a partial
  float l = l_lane;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (unit && lg == 0) xch[mb_s * S::kHeads + hloc] = l;
  if (v4_out != nullptr && unit && mb_s == 0 && lg == 0) m_lds[hloc] = m_ref;
  lds_barrier();
  if (v4_out != nullptr) {
    // the DeepSeek-V4 variant with one split: the head's attention sink joins
    // the denominator and the last `tail` columns are rotated back by the
    // query's position; adjacent columns (a rotary pair) sit in adjacent lanes
    const int32_t pos = seq_len[b] - 1;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hl = hb * 16 + lg * 4 + i;
        const int h = head0 + hl;
        const bool ok = h < H;
        const float lh = xch[hl] + xch[S::kHeads + hl];
        const float inv = ok ? 1.f / (lh + exp2f(sink[ok ? h : 0] * kLog2e - m_lds[hl])) : 0.f;
#pragma unroll
        for (int nb = 0; nb < S::kNB; ++nb) {
          const int col = c0 + nb * 16 + l16;
          float v = o[hb][nb][i] * inv;
          if (c0 + nb * 16 + 16 > R - tail) {  // uniform: the block holds rotary columns
            const float other = __shfl_xor(v, 1, 64);
            if (col >= R - tail) {
              float cs, sn;
              angle_cos_sin(-static_cast<double>(pos) * rope_freq((col - (R - tail)) / 2, rope_base, freqs), &cs,
                            &sn);
              v = (l16 & 1) == 0 ? v * cs - other * sn : v * cs + other * sn;
            }
          }
          if (ok) v4_out[(static_cast<int64_t>(b) * H + h) * R + col] = f32_to_bf16(v);
        }
      }
    return;
  }
  const bool partials = part_o != nullptr;
  if (unit && mb_s == 0 && lg == 0 && partials && head < H) {
    const int64_t pidx = slot * H + head;
    part_ml[pidx * 2 + 0] = m_ref;
    part_ml[pidx * 2 + 1] = xch[hloc] + xch[S::kHeads + hloc];
  }
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hl = hb * 16 + lg * 4 + i;
      const int h = head0 + hl;
      if (h >= H) continue;
      const float lh = xch[hl] + xch[S::kHeads + hl];
      const float inv = lh > 0.f ? 1.f / lh : 0.f;  // an empty split has l = 0 and o_ = 0
      if (!partials) {
        float* dst = o_out + (static_cast<int64_t>(b) * H + h) * R + c0 + l16;
#pragma unroll
        for (int nb = 0; nb < S::kNB; ++nb) dst[nb * 16] = o[hb][nb][i] * inv;
      } else {
        bf16_t* dst = part_o + (slot * H + h) * R + c0 + l16;
#pragma unroll
        for (int nb = 0; nb < S::kNB; ++nb) dst[nb * 16] = f32_to_bf16(o[hb][nb][i] * inv);
      }
    }
}

template <int R, int RW, int NHB, int NHH, int STAGES>
void launch(const AttnShape& sh, const void* q_lat, const void* q_pe, const void* cache,
            const int64_t* seq_start, const int32_t* seq_len, int batch, int n_split, int split_len,
            void* part_o, float* part_ml, float* o_out, const V4Epilogue* v4, hipStream_t s, int ragged_items) {
  using S = Shape<R, RW, NHB, NHH, STAGES>;
  auto kern = decode_mfma_kernel<R, RW, NHB, NHH, STAGES>;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                      S::kLdsBytes);
  const int pairs = batch * n_split;
  const int grid = ragged_items > 0 ? ragged_items : NHH == 1 ? pairs : (pairs + 7) / 8 * 8 * NHH;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), S::kLdsBytes, s,
                     static_cast<const bf16_t*>(q_lat), static_cast<const bf16_t*>(q_pe),
                     static_cast<const bf16_t*>(cache), seq_start, seq_len, batch, sh.H, sh.G,
                     sh.d_rope, sh.scale, n_split, split_len, static_cast<bf16_t*>(part_o), part_ml,
                     o_out, v4 ? static_cast<bf16_t*>(v4->out) : nullptr, v4 ? v4->sink : nullptr,
                     v4 ? std::pow(v4->theta, -2.0 / v4->d_rope) : 0.0, v4 ? v4->freqs : nullptr,
                     v4 ? v4->d_rope : 0, NHH == 1 ? ragged_items : 0);
}

// Compiled shapes: (latent r, row width r + G*d_rope, 16-head blocks per workgroup,
// workgroups per sequence split, LDS stages, head count range served).
#define MLA_DECODE_SHAPES(X)                                                                  \
  X(512, 576, 4, 2, 4, 113, 128) /* H = 128, G = 1, d_rope = 64 (DeepSeek-V2)          */ \
  X(512, 544, 2, 1, 4, 17, 32)   /* H = 32, G = 4, d_rope = 8 (Qwen3-30B-A3B MLA delta) */ \
  X(128, 160, 2, 1, 3, 17, 32)   /* H = 28, G = 4, d_rope = 8 (Qwen2.5-7B MLA delta)    */ \
  X(512, 512, 1, 1, 4, 1, 16)    /* one 512-wide KV head as key and value (DeepSeek-V4)  */

}  // namespace

bool decode_mfma_supported(const AttnShape& sh) {
  if (sh.d_rope % 8 != 0) return false;
#define MLA_MATCH(R_, RW_, NHB_, NHH_, ST_, HLO_, HHI_) \
  if (sh.r == R_ && sh.row_w == RW_ && sh.H >= HLO_ && sh.H <= HHI_) return true;
  MLA_DECODE_SHAPES(MLA_MATCH)
#undef MLA_MATCH
  return false;
}

int decode_mfma_head_groups(const AttnShape& sh) {
#define MLA_NHH(R_, RW_, NHB_, NHH_, ST_, HLO_, HHI_) \
  if (sh.r == R_ && sh.row_w == RW_ && sh.H >= HLO_ && sh.H <= HHI_) return NHH_;
  MLA_DECODE_SHAPES(MLA_NHH)
#undef MLA_NHH
  return 1;
}

int decode_mfma_blocks_per_cu(const AttnShape& sh) {
  int lds = 0;
#define MLA_LDS(R_, RW_, NHB_, NHH_, ST_, HLO_, HHI_)              \
  if (sh.r == R_ && sh.row_w == RW_ && sh.H >= HLO_ && sh.H <= HHI_) \
    lds = Shape<R_, RW_, NHB_, NHH_, ST_>::kLdsBytes;
  MLA_DECODE_SHAPES(MLA_LDS)
#undef MLA_LDS
  if (lds == 0) return 1;
  return std::max(1, std::min(4, (160 * 1024) / lds));
}

void decode_mfma(const AttnShape& sh, const void* q_lat, const void* q_pe, const void* cache,
                 const int64_t* seq_start, const int32_t* seq_len, int batch, int n_split,
                 int split_len, void* part_o, float* part_ml, float* o_out, hipStream_t s,
                 const V4Epilogue* v4, int ragged_items) {
  if (batch <= 0) return;
#define MLA_LAUNCH(R_, RW_, NHB_, NHH_, ST_, HLO_, HHI_)                                          \
  if (sh.r == R_ && sh.row_w == RW_ && sh.H >= HLO_ && sh.H <= HHI_) {                           \
    launch<R_, RW_, NHB_, NHH_, ST_>(sh, q_lat, q_pe, cache, seq_start, seq_len, batch, n_split, \
                                     split_len, part_o, part_ml, o_out, v4, s, ragged_items);    \
    return;                                                                                      \
  }
  MLA_DECODE_SHAPES(MLA_LAUNCH)
#undef MLA_LAUNCH
}

}  // namespace mla
