// Device-side helpers shared by the MLA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef uint16_t bf16_t;  // raw bfloat16 bit pattern

// MFMA operand / accumulator vector types.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed pair of bf16 (low half = a), round to nearest even
// (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

// Sum of the two bf16 values of a packed pair, as float.
__device__ __forceinline__ float bf16x2_sum(uint32_t w) {
  return __uint_as_float(w << 16) + __uint_as_float(w & 0xFFFF0000u);
}

// float -> bfloat16, round to nearest even.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return static_cast<bf16_t>(pack_bf16x2(f, 0.f) & 0xFFFFu);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<_Float16> {
  __device__ __forceinline__ static float load(const _Float16* p, int64_t i) { return static_cast<float>(p[i]); }
  __device__ __forceinline__ static void store(_Float16* p, int64_t i, float v) { p[i] = static_cast<_Float16>(v); }
};
template <> struct Elem<bf16_t> {
  __device__ __forceinline__ static float load(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  __device__ __forceinline__ static void store(bf16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// RoPE angle p·θ^(-2j/d) and its cos/sin.  The frequency is base^j with
// base = θ^(-2/d) (computed by the host in double), raised by squaring in
// double; the angle p·base^j is formed and reduced to [-π, π] in double, since
// an fp32 angle at p ~ 1e5 is off by ~1e-2 rad.  Only the reduced angle goes
// through fp32 sin/cos (error ~1e-7 for |x| <= π).
__device__ __forceinline__ void angle_cos_sin(double ang, float* c, float* s) {
  constexpr double kTwoPi = 6.283185307179586476925;
  const double k = rint(ang * (1.0 / kTwoPi));
  const float r = static_cast<float>(fma(-k, kTwoPi, ang));
  sincosf(r, s, c);
}

// Frequency of rotary pair j: base^j (base = θ^(-2/d)), or freqs[j] from a table.
__device__ __forceinline__ double rope_freq(int j, double base, const double* freqs) {
  if (freqs != nullptr) return freqs[j];
  double f = 1.0, b = base;
  for (int e = j; e != 0; e >>= 1) {
    if (e & 1) f *= b;
    b *= b;
  }
  return f;
}

__device__ __forceinline__ void rope_cos_sin(int32_t pos, int j, double base, const double* freqs, float* c,
                                             float* s) {
  angle_cos_sin(static_cast<double>(pos) * rope_freq(j, base, freqs), c, s);
}

// ---- Split plan of a ragged decode batch (at most kWave sequences), made on the
// device from the lengths so that the work spreads over n_items workgroups
// whatever the lengths.  Every split of every sequence has split_len rows, the
// smallest multiple of 64 with sum_b ceil(len_b / split_len) <= n_items; the
// items (sequence, split) are numbered sequence after sequence.  Called by a
// whole wave; lane b holds sequence b (lanes >= batch hold nothing), and every
// lane gets the same split_len.  Requires batch < n_items.
__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// A value the same in every lane, as a scalar (both 32-bit halves read from the
// first active lane).
__device__ __forceinline__ int64_t uniform_i64(long long v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v)));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

struct RaggedLane {
  int split_len;
  int len;    // this lane's sequence length (0 for lanes >= batch)
  int first;  // first item of this lane's sequence
  int count;  // items of this lane's sequence (0 for lanes >= batch)
};

__device__ inline RaggedLane ragged_plan(const int32_t* __restrict__ seq_len, int batch, int n_items) {
  const int lane = threadIdx.x & (kWave - 1);
  const int len = lane < batch ? max(seq_len[lane], 0) : 0;
  const int total = wave_sum_int(len);
  {
    // all lengths equal: n_items / batch splits each (what a plan made on the
    // host gives), no search
    int mn = lane < batch ? len : INT_MAX, mx = len;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      mn = min(mn, __shfl_xor(mn, o, kWave));
      mx = max(mx, __shfl_xor(mx, o, kWave));
    }
    if (mn == mx) {
      const int per = n_items / batch;
      RaggedLane r;
      r.split_len = max(64, ((mx + per - 1) / per + 63) / 64 * 64);
      r.len = len;
      r.count = (len + r.split_len - 1) / r.split_len;
      r.first = lane * ((mx + r.split_len - 1) / r.split_len);
      return r;
    }
  }
  // split_len = 64k: k_lo cannot fit fewer items than total / n_items; k_hi
  // always fits (at most one partial split per sequence beyond total / 64k)
  int k_lo = max(1, (total + 64 * n_items - 1) / (64 * n_items));
  int k_hi = max(k_lo, (total + 64 * (n_items - batch) - 1) / (64 * (n_items - batch)));
  while (k_lo < k_hi) {
    const int mid = (k_lo + k_hi) >> 1;
    const int items = wave_sum_int((len + 64 * mid - 1) / (64 * mid));
    if (items <= n_items) k_hi = mid;
    else k_lo = mid + 1;
  }
  RaggedLane r;
  r.split_len = 64 * k_hi;
  r.len = len;
  r.count = (len + r.split_len - 1) / r.split_len;
  int incl = r.count;  // inclusive prefix sum over the lanes
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int v = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += v;
  }
  r.first = incl - r.count;
  return r;
}

}  // namespace mla
