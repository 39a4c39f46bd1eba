// bf16 MFMA decode for the wide-head shape: H = 128 query heads sharing one
// latent cache row of r = 512 latent + 64 rotary dims (one rotary key).
//
// The absorbed score of every head reads the same cached row [c ; kr] and the
// latent-space PV reads the same c (MLA principle page, section on matrix
// absorption, eqs. (4)-(5)), so one workgroup takes ALL heads of one
// (sequence, context split): each cache tile crosses HBM -> LDS once per CU.
//
// Workgroup = 8 wave64s, two per SIMD, so one wave's softmax, LDS waits and
// copy issue run under the other wave's MFMAs (with one wave per SIMD those
// latencies were exposed).  Each wave has half a SIMD's register file:
//   - wave w scores heads [16w, 16w+16): their Qᵀ for the split is 72 registers
//     of bf16 MFMA operands;
//   - wave w accumulates latent columns [64w, 64w+64) of O for all 128 heads
//     (128 fp32 registers).  Splitting the PV by columns makes each wave read
//     only its eighth of the transposed C fragments; the softmax weights cross
//     between waves through a small LDS buffer.
// Tiles of 32 rows:
//   - copies HBM -> LDS by global_load_lds_dwordx4 into 4 buffers (tiles t and
//     t+1 in use, t+2 and t+3 in flight) with the non-temporal hint (each
//     tile is read once), issued by waves 0-3 only: a copy's
//     issue stalls while the CU's memory pipeline is full, and with one issuing
//     wave per SIMD the other wave keeps the SIMD's MFMAs busy meanwhile (the
//     waves w and w + 4 share a SIMD); stored without padding; the 16-byte
//     chunks of a row are XOR-swizzled by 2·((row / 2) mod 4) within groups
//     of eight, so the score's fragment reads and the transposed PV reads
//     both fall on distinct banks;
//   - score: Sᵀ[32 rows x 16 heads], two 16x16 blocks of
//     v_mfma_f32_16x16x32_bf16 over the whole row (K = 576), tile rows as the A
//     operand from LDS, Qᵀ as the B operand from registers;
//   - softmax against a per-head reference max of the split (the first tile's
//     max, base 2, with 2^64 of headroom; no running max is kept); a split
//     whose weights pass the headroom (seen in the row sums) is redone after a
//     max-only scan with its true max, so O is never rescaled;
//   - softmax weights P as bf16 MFMA A fragments into a double-buffered LDS
//     exchange [head block][lane] (8 KB a tile): a score lane holds rows
//     4lg..4lg+3 and 16+4lg..16+4lg+3 of its head, and the K order of the PV
//     product is taken to be exactly that;
//   - PV: O[128 heads x 64 columns of wave w] += P[128 x 32]·C[32 x 64], the
//     transposed C fragments (ds_read_b64_tr_b16) read at those row bases.
// Iteration t (one barrier, for the tile ring and the P exchange): score of
// tile t+1, its softmax and store to the exchange, then the PV of tile t.
// Output: normalised o_ (part_o null, one split) or the split's (m, l) and
// its normalised o_ in bf16.
#include <math.h>

#include "lds_dma.h"
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kR = 512;              // latent width
constexpr int kRW = 576;             // cache row width (r + d_rope, one rotary group)
constexpr int kHeads = 128;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTL = 32;              // rows per tile
constexpr int kStages = 4;
constexpr int kRowBytes = kRW * 2;   // 1152
constexpr int kRowChunks = kRowBytes / 16;           // 72
constexpr int kTileBytes = kTL * kRowBytes;          // 36864
constexpr int kDmaOps = kTileBytes / 1024;           // 36 one-KB copies per tile
constexpr int kDmaWaves = 4;                          // waves 0-3 issue every copy; 4-7 none
constexpr int kDmaMax = kDmaOps / kDmaWaves;          // 9
constexpr int kSteps = kRW / 32;                     // 18 score k-steps
constexpr int kHW = kHeads / kWaves;                 // 16 heads per wave in the score
constexpr int kHB = kHeads / 16;                     // 8 head blocks of the PV
constexpr int kCB = kR / 16 / kWaves;                // 4 column blocks of 16 per wave
constexpr int kPBytes = kHB * 64 * 16;               // one tile's softmax weights: 8 KB
constexpr int kPOff = kStages * kTileBytes;          // P exchange, two buffers
constexpr int kLdsBytes = kPOff + 2 * kPBytes;       // 160 KB
// after a pass's tile loop the ring is idle: its first bytes hold the row sums
// per head (xch) and the restart flags
constexpr int kFlagsOff = 1024;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kSLA = 2;                              // score k-steps of fragments in flight

static_assert(kHW == 16, "one 16-head block per wave in the score");
static_assert(kDmaOps == kDmaWaves * kDmaMax, "copies split evenly over the issuing waves");
static_assert(kRowChunks % 8 == 0, "swizzle groups of eight chunks");
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
static_assert(kHeads * 4 <= kFlagsOff && kFlagsOff + 4 * kWaves <= kTileBytes, "xch and flags inside tile slot 0");
static_assert(3 * kDmaMax < 64, "vmcnt range");
static_assert(kTL * kRowChunks <= 2304, "row-of-chunk division by multiplication is exact below 2304");

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

// wait until at most N tiles' copies of this wave are in flight (OPS copies per tile)
template <int N, int OPS>
__device__ __forceinline__ void wait_tiles_after() {
  wait_vmcnt<N * OPS>();
}

__global__ __launch_bounds__(kThreads, 1) void decode_wide_kernel(
    const bf16_t* __restrict__ q_lat, const bf16_t* __restrict__ q_pe,
    const bf16_t* __restrict__ cache, const int64_t* __restrict__ seq_start,
    const int32_t* __restrict__ seq_len, int batch, float scale, int n_split, int split_len,
    bf16_t* __restrict__ part_o, float* __restrict__ part_ml, float* __restrict__ o_out) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  float* xch = reinterpret_cast<float*>(smem);               // [kHeads], after the tile loop
  int* flags = reinterpret_cast<int*>(smem + kFlagsOff);      // [kWaves], after the tile loop

  const int pair = blockIdx.x;
  if (pair >= batch * n_split) return;
  const int split = pair % n_split;
  const int b = pair / n_split;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  const bool dma_wave = wave < kDmaWaves;

  const int64_t row0 = seq_start[b];
  const int len = seq_len[b];
  const int l_begin = split * split_len;
  const int l_end = min(len, l_begin + split_len);
  const int n_tiles = l_end > l_begin ? (l_end - l_begin + kTL - 1) / kTL : 0;
  const char* cache_b = reinterpret_cast<const char*>(cache + row0 * kRW);
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u8*)smem));

  // ---- tile copy: wave w < 4 issues 1 KB copies j = w + 4i < 36; copy j fills LDS
  // chunks [64j, 64j + 64) of the tile image.  LDS chunk L (row L / 72, slot
  // L % 72) holds global chunk swz(slot, row) of the same row, which is
  // L ^ row_key(row) since rows are whole groups of eight chunks.  Rows past
  // the split read a chunk of its last valid row instead.  The lane index is
  // made opaque so the few offset instructions are redone per tile rather than
  // held in registers.
  auto issue_op = [&](int t, int j) {
    const int tile_row = l_begin + t * kTL;
    const int valid = min(kTL, l_end - tile_row);
    const char* tbase = cache_b + static_cast<int64_t>(tile_row) * kRowBytes;
    const uint32_t dst = lds0 + (t % kStages) * kTileBytes;
    int ln = lane;
    __asm__ volatile("" : "+v"(ln));
    if (valid == kTL) {
      // whole tile: the copy's 64 chunks span rows r0 and r0 + 1 (lanes from
      // bnd on), each with a uniform swizzle key, so a lane's offset within the
      // copy's kilobyte is 16·lane ^ key (the key only touches bits 4..6)
      const int r0 = (j * 64) / kRowChunks;
      const int bnd = (r0 + 1) * kRowChunks - j * 64;
      const int k0 = row_key(r0) << 4, k1 = row_key(r0 + 1) << 4;
      const uint32_t voff = static_cast<uint32_t>((ln * 16) ^ (ln < bnd ? k0 : k1));
      global_to_lds16_stream(tbase + j * 1024, voff, __builtin_amdgcn_readfirstlane(dst + j * 1024));
    } else {
      // last tile of the split: rows past it read a chunk of its last valid row
      const int L = j * 64 + ln;
      const int r = (L * 1821) >> 17;  // L / 72 for L < 2304
      const int g = r < valid ? (L ^ row_key(r)) : (valid - 1) * kRowChunks + (L & 63);
      global_to_lds16_stream(tbase, static_cast<uint32_t>(g * 16), __builtin_amdgcn_readfirstlane(dst + j * 1024));
    }
  };
  auto issue_tile = [&](int t) {
    if (dma_wave) {
#pragma unroll
      for (int i = 0; i < kDmaMax; ++i) issue_op(t, wave + kDmaWaves * i);
    }
  };
  auto wait_tile = [&](int t, int last_issued) {
    const int n = last_issued - t;  // tiles issued after t
    if (dma_wave) {
      switch (n) {
        case 0: wait_tiles_after<0, kDmaMax>(); break;
        case 1: wait_tiles_after<1, kDmaMax>(); break;
        default: wait_tiles_after<2, kDmaMax>(); break;
      }
    }
  };

  // ---- Qᵀ of this wave's heads: B operand, lane = head 16w + l16, k = 32ks + 8lg + e
  bf16x8 qf[kSteps];
  {
    const int head = wave * kHW + l16;
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) {
      const int k0 = ks * 32 + lg * 8;
      const uint4 v = k0 < kR
          ? *reinterpret_cast<const uint4*>(q_lat + (static_cast<int64_t>(b) * kHeads + head) * kR + k0)
          : *reinterpret_cast<const uint4*>(q_pe + (static_cast<int64_t>(b) * kHeads + head) * (kRW - kR) +
                                            (k0 - kR));
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }
  const float qk_scale = scale * kLog2e;
  // the Q loads must land before any tile copy is issued: the compiler's wait at
  // their first use would otherwise also drain the copies in flight
  wait_vmcnt<0>();

  // score fragment addresses: row r = 16rb + l16, chunk 4ks + lg, whose slot in
  // its group of eight is (4(ks & 1) + lg) ^ row_key(r), the same for both rb
  const int a_off0 = l16 * kRowBytes, a_off1 = (16 + l16) * kRowBytes;
  const int x_even = (lg ^ row_key(l16)) & 7;
  const int x_odd = ((4 + lg) ^ row_key(l16)) & 7;

  float m_ref = -INFINITY;   // reference max of head 16w + l16 (base 2)
  float m_lane, l_lane;      // raw score max, bf16 weight sum of the lane
  f32x4 o[kHB][kCB];         // O[heads 16hb + 4lg + i][columns 64w + 16j + l16]

  // Raw scores q·k of tile tt (unscaled; rows past the split masked to -inf):
  // s[rb] = rows 16rb + 4lg + i, head 16w + l16.  Fragments of k-step ks + 2 are
  // read while the MFMAs of ks run; the scheduling barriers keep the compiler
  // from hoisting more reads.
  auto score = [&](int tt, f32x4 (&s)[2]) {
    const unsigned char* tb = smem + (tt % kStages) * kTileBytes;
    s[0] = s[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto frag = [&](int ks, int off) {
      const int coff = (ks >> 1) * 128 + ((ks & 1) ? x_odd : x_even) * 16;
      return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(tb + off + coff));
    };
    bf16x8 fa[kSLA][2];
#pragma unroll
    for (int p = 0; p < kSLA; ++p) {
      fa[p][0] = frag(p, a_off0);
      fa[p][1] = frag(p, a_off1);
    }
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) {
      const bf16x8 a0 = fa[ks % kSLA][0], a1 = fa[ks % kSLA][1];
      s[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[ks], s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[ks], s[1], 0, 0, 0);
      if (ks + kSLA < kSteps) {
        fa[ks % kSLA][0] = frag(ks + kSLA, a_off0);
        fa[ks % kSLA][1] = frag(ks + kSLA, a_off1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    const int valid = min(kTL, l_end - (l_begin + tt * kTL));  // < kTL only in the last tile
    if (valid < kTL) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (rb * 16 + lg * 4 + i >= valid) s[rb][i] = -INFINITY;
    }
  };

  // softmax weights P = 2^(s·scale·log2(e) - m_ref) of the wave's head block,
  // packed bf16 as the A operand of the PV product (K order [rows 4lg + i, then
  // 16 + 4lg + i]) and stored to slot [w][lane] of exchange buffer pbuf.  The
  // row sum takes the bf16 weights the PV product uses (v_dot2 with ones).
  const bf16x2_t ones = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
  auto softmax = [&](const f32x4 (&s)[2], unsigned char* pbuf) {
    uint32_t w[4];
    const float nm = -m_ref;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const f32x4 v = s[rb];
      const float p0 = __builtin_amdgcn_exp2f(fmaf(v[0], qk_scale, nm));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(v[1], qk_scale, nm));
      const float p2 = __builtin_amdgcn_exp2f(fmaf(v[2], qk_scale, nm));
      const float p3 = __builtin_amdgcn_exp2f(fmaf(v[3], qk_scale, nm));
      w[2 * rb] = pack_bf16x2(p0, p1);
      w[2 * rb + 1] = pack_bf16x2(p2, p3);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      l_lane = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[e]), ones, l_lane, false);
    *reinterpret_cast<uint4*>(pbuf + (wave * 64 + lane) * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  };

  // transposed C fragment of column block nb: lane (l16, lg) gets column
  // 16nb + l16 at rows 4lg + (0..3) (lo) and 16 + 4lg + (0..3) (hi); lane s of a
  // 16-lane group supplies the address of row base + s/4, columns 4(s % 4)..+3
  const int r_lo = lg * 4 + (l16 >> 2), r_hi = 16 + r_lo;
  const int c_sub = (l16 & 1) * 8, c_half = (l16 & 3) >> 1;
  auto cfrag = [&](const unsigned char* tb, int nb) {
    const int chunk = nb * 2 + c_half;
    const unsigned char* plo = tb + r_lo * kRowBytes + swz(chunk, r_lo) * 16 + c_sub;
    const unsigned char* phi = tb + r_hi * kRowBytes + swz(chunk, r_hi) * 16 + c_sub;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(plo));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(phi));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // PV of tile tt over this wave's 64 columns, P of all heads from exchange
  // buffer tt % 2: head block outer, the wave's four C fragments held.
  // pv_load reads the C fragments and the first P fragment (issued before the
  // softmax, whose VALU work then covers their latency); pv_mma reads each P
  // fragment one head block ahead of its MFMAs.
  auto pfrag = [&](const unsigned char* pb, int hb) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(pb + (hb * 64 + lane) * 16));
  };
  auto pv_load = [&](int tt, bf16x8 (&cf)[kCB], bf16x8 (&pf)[2]) {
    const unsigned char* tb = smem + (tt % kStages) * kTileBytes;
#pragma unroll
    for (int j = 0; j < kCB; ++j) cf[j] = cfrag(tb, wave * kCB + j);
    pf[0] = pfrag(smem + kPOff + (tt & 1) * kPBytes, 0);
  };
  auto pv_mma = [&](int tt, const bf16x8 (&cf)[kCB], bf16x8 (&pf)[2]) {
    const unsigned char* pb = smem + kPOff + (tt & 1) * kPBytes;
#pragma unroll
    for (int hb = 0; hb < kHB; ++hb) {
      if (hb + 1 < kHB) pf[(hb + 1) & 1] = pfrag(pb, hb + 1);
#pragma unroll
      for (int j = 0; j < kCB; ++j)
        o[hb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[hb & 1], cf[j], o[hb][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  auto tile_max = [&](const f32x4 (&s)[2]) {
    return fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                 fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
  };
  // One pass over the split: weights and PV against m_ref (set from tile 0 in
  // the first pass), or (kScan) the running max of the raw scores only.
  auto run_pass = [&](auto scan_c, bool set_ref) {
    constexpr bool kScan = decltype(scan_c)::value;
#pragma unroll
    for (int hb = 0; hb < kHB; ++hb)
#pragma unroll
      for (int j = 0; j < kCB; ++j) o[hb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_lane = -INFINITY;
    l_lane = 0.f;

#pragma unroll
    for (int t = 0; t < kStages - 1; ++t)
      if (t < n_tiles) issue_tile(t);
    int issued = min(kStages - 1, n_tiles) - 1;

    if (n_tiles > 0) {
      // prologue: tile 0; in the first pass its max sets the reference
      wait_tile(0, issued);
      lds_barrier();
      f32x4 s0[2];
      score(0, s0);
      if constexpr (kScan) {
        m_lane = tile_max(s0);
      } else {
        if (set_ref) {
          float mx = tile_max(s0);
          mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
          mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
          m_ref = mx * qk_scale;
        }
        softmax(s0, smem + kPOff);
      }
    }

    // iteration t: scores of tile t+1, their softmax into exchange buffer
    // (t+1) % 2, then the PV of tile t
    for (int t = 0; t < n_tiles; ++t) {
      if (t + 1 < n_tiles) wait_tile(t + 1, issued);
      // tile t+1 and the P of tile t visible; PV(t-1) done everywhere: ring
      // buffer (t-1) % 4 and P buffer (t+1) % 2 are free
      lds_barrier();
      if (t + kStages - 1 < n_tiles) {  // tile t+3 into buffer (t-1) % 4
        issue_tile(t + kStages - 1);
        issued = t + kStages - 1;
      }
      // the last iteration has no next tile: PV only
      const bool next = t + 1 < n_tiles;
      f32x4 s_next[2];
      if (next) score(t + 1, s_next);
      if constexpr (kScan) {
        if (next) m_lane = fmaxf(m_lane, tile_max(s_next));
      } else {
        bf16x8 cf[kCB], pf[2];
        pv_load(t, cf, pf);
        if (next) softmax(s_next, smem + kPOff + ((t + 1) & 1) * kPBytes);
        pv_mma(t, cf, pf);
      }
    }
    lds_barrier();  // every wave is done with the ring and the P buffers
  };

  // A pass whose weights passed the reference's 2^64 headroom (seen in the row
  // sums: above 2^64, or inf/NaN) is redone after a max-only scan with the
  // split's true max per head; every lane votes.
  for (int pass = 0;; ++pass) {
    run_pass(std::false_type{}, pass == 0);
    if (pass == 1) break;
    const bool over = __ballot(!(l_lane <= 1.8e19f)) != 0;
    if (lane == 0) flags[wave] = over ? 1 : 0;
    lds_barrier();
    int any = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) any |= flags[w];
    if (!any) break;
    // every wave has read the flags before the scan's first copies refill the
    // ring slot that holds them
    lds_barrier();
    run_pass(std::true_type{}, false);
    float mx = m_lane;
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    m_ref = mx * qk_scale;
  }

  // ---- epilogue: l per head -> LDS (the wave's own heads); O normalised or as a partial
  const bool partials = part_o != nullptr;
  {
    float l = l_lane;
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int head = wave * kHW + l16;
    if (lg == 0) {
      xch[head] = l;
      if (partials) {
        const int64_t pidx = (static_cast<int64_t>(b) * n_split + split) * kHeads + head;
        part_ml[pidx * 2 + 0] = m_ref;
        part_ml[pidx * 2 + 1] = l;
      }
    }
  }
  lds_barrier();  // the row sums of every head are in LDS
  // lane holds O[head 16hb + 4lg + i][column 64w + 16j + l16]
  const int col0 = wave * kCB * 16 + l16;
#pragma unroll
  for (int hb = 0; hb < kHB; ++hb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = hb * 16 + lg * 4 + i;
      const float lh = xch[h];
      const float inv = lh > 0.f ? 1.f / lh : 0.f;  // an empty split has l = 0 and o_ = 0
      if (!partials) {
        float* dst = o_out + (static_cast<int64_t>(b) * kHeads + h) * kR + col0;
#pragma unroll
        for (int j = 0; j < kCB; ++j) dst[j * 16] = o[hb][j][i] * inv;
      } else {
        bf16_t* dst = part_o + ((static_cast<int64_t>(b) * n_split + split) * kHeads + h) * kR + col0;
#pragma unroll
        for (int j = 0; j < kCB; ++j) dst[j * 16] = f32_to_bf16(o[hb][j][i] * inv);
      }
    }
}

}  // namespace

bool decode_wide_supported(const AttnShape& sh) {
  return sh.H == kHeads && sh.G == 1 && sh.r == kR && sh.row_w == kRW;
}

void decode_wide(const AttnShape& sh, const void* q_lat, const void* q_pe, const void* cache,
                 const int64_t* seq_start, const int32_t* seq_len, int batch, int n_split,
                 int split_len, void* part_o, float* part_ml, float* o_out, hipStream_t s) {
  if (batch <= 0) return;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(decode_wide_kernel),
                      hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  hipLaunchKernelGGL(decode_wide_kernel, dim3(batch * n_split), dim3(kThreads), kLdsBytes, s,
                     static_cast<const bf16_t*>(q_lat), static_cast<const bf16_t*>(q_pe),
                     static_cast<const bf16_t*>(cache), seq_start, seq_len, batch, sh.scale, n_split,
                     split_len, static_cast<bf16_t*>(part_o), part_ml, o_out);
}

}  // namespace mla
