// Internal launcher interface between the C ABI (mla_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;

// C[z][m][n] = Σ_k A[z][m][k] · B[z][k][n]; strides in elements.
struct GemmArgs {
  const void* A;
  int64_t sAz, sAm;  // A[z][m][k]: k contiguous
  const void* B;
  int64_t sBz, sBo;  // b_kn: B[z][k][n] (sBo = k stride); else B[z][n][k] (sBo = n stride)
  void* C;
  int64_t sCz, sCm;  // C[z][m][n]: n contiguous
  int M, N, K, Z;
  // fp32 path with B[z][n][k] only: columns n >= N0 come from row n - N0 of B1
  // (two projections of one input in one launch); B1 null: every column from B
  const void* B1;
  int N0;
};

// dtype == kF32: fp32 in/out VALU path.  dtype == kBF16: A bf16 (or fp32 if a_f32),
// B bf16, fp32 accumulate, C fp32 or bf16 (out_bf16).
void gemm(const GemmArgs& g, int dtype, bool a_f32, bool b_kn, bool out_bf16, hipStream_t s);
// bf16 A [z][m][k], bf16 B [z][n][k] -> fp16 C (fp32 accumulate).
void gemm_f16_out(const GemmArgs& g, hipStream_t s);

// Weight-streaming GEMM for M <= 64 rows: C[z][m][n] = Σ_k A[z][m][k]·W[z][n][k]
// with W rows n < N0 from B0 and n >= N0 from B1 (row n - N0), bf16 weights.
// splits > 1: K pieces write fp32 slices C + s*sPs that the consumer sums.
struct SkinnyArgs {
  const void* A;
  int64_t sAz, sAm;          // A[z][m][k]: bf16, or fp32 (split hi/lo)
  const uint16_t* B0;  // bf16 bit patterns
  const uint16_t* B1;
  int N0;
  int64_t sBz, sBo;          // W[z][n][k]
  void* C;
  int64_t sCz, sCm, sPs;     // C[s][z][m][n]
  int M, N, K, Z, splits, k_per_split;
  // merged A (gemm_skinny_merged): A[z][m][k] = Σ_j w_j · A[z][m][k + j*sAs] over
  // bf16 split partials (each normalised) with softmax-merge weights
  // w_j ∝ 2^(max_j) sum_j from ml[(m*n_merge + j)*ml_heads + z] = (max, sum)
  int64_t sAs;
  const float* ml;
  int ml_heads, n_merge;
  // token rows split over m_groups workgroups per column tile (0 or 1: one)
  int m_groups;
  // weights in the tiled streaming layout (gemm_skinny_tiled; B0/B1 unused)
  const uint16_t* Bt;
};
int skinny_splits(int M, int N, int Z, int K);
void gemm_skinny(SkinnyArgs sa, bool a_f32, bool out_bf16, hipStream_t s);
// Tiled streaming layout of a weight [W0 (n0 rows) ; W1 (n1 rows)] of row length
// k: blocks of kTileRows rows x kTileK k (24 KB), tile-major then k-block, each
// row's 16-byte chunks XOR-swizzled by (row & 15); rows past n0 + n1 and k past
// k are zero.  gemm_skinny_tiled reads it with one contiguous 1 KB copy per
// kilobyte of a block.
constexpr int kTileRows = 96;
constexpr int kTileK = 128;
int64_t tiled_weight_bytes(int64_t n_rows, int64_t k);
void tile_weights(const uint16_t* w0, int64_t n0, const uint16_t* w1, int64_t n1, int64_t k, uint16_t* out,
                  hipStream_t s);
// bf16 A (M <= 64) times weights in the tiled layout (sa.Bt; N = n0 + n1 rows,
// K = k), fp32 or bf16 out with sa.splits K slices as gemm_skinny
void gemm_skinny_tiled(SkinnyArgs sa, bool out_bf16, hipStream_t s);
void sum_split_slices(float* c, int splits, int64_t sps, int M, int N, int64_t ldc, hipStream_t s);
// out[m, n] (dense [M, N], dtype) = Σ_p c[p*sps + m*ldc + n]
void sum_cast_slices(int dtype, const float* c, int splits, int64_t sps, int M, int N, int64_t ldc, void* out,
                     hipStream_t s);
// fp32 A merged from n_merge <= skinny_max_merge() split-softmax partials, one K piece
int skinny_max_merge();
void gemm_skinny_merged(SkinnyArgs sa, int n_merge, bool out_bf16, hipStream_t s);

// Cache rows from the fp32 projections in `proj` ([T, r + G*d_rope], row stride ld):
// optional RMSNorm over the latent, RoPE on each rotary-key group, cast, scatter to slots.
// `proj` holds `splits` partial slices (slice stride `sps` floats) that are summed first.
// `freqs` (device, d_rope/2 doubles) replaces theta^(-2j/d_rope) when not null.
void finalize_cache_rows(int dtype, const float* proj, int64_t ld, int splits, int64_t sps,
                         void* cache, const int64_t* slots, const int32_t* positions,
                         int64_t n_tokens, int r, int n_groups, int d_rope, int latent_rmsnorm,
                         float eps, double theta, const double* freqs, hipStream_t s);

// q_pe[t,h,:] = RoPE(proj[t*ld + h*hstride : +d_rope], positions[t]), cast to dtype.
void finalize_query_rope(int dtype, const float* proj, int64_t ld, int hstride, void* q_pe,
                         const int32_t* positions, int64_t n_tokens, int n_heads, int d_rope,
                         double theta, const double* freqs, hipStream_t s);
// The query projection's rows q [splits][T, ld] (n_cols columns; head h's rotary
// part at rope_off + h*hstride): the splits summed into slice 0 (every column
// but the rotary ones) and q_pe = RoPE of the summed rotary part, in one launch;
// with one slice, finalize_query_rope alone.  Same results as sum_split_slices
// followed by finalize_query_rope.
void finalize_query(int dtype, float* q, int64_t ld, int splits, int64_t sps, int n_cols, int rope_off,
                    int hstride, void* q_pe, const int32_t* positions, int64_t n_tokens, int n_heads,
                    int d_rope, double theta, const double* freqs, hipStream_t s);

// dst[t, h, 0:n] = src[t*ld + h*hstride : +n] (fp32 -> dtype), dst dense [n_rows, n_heads, n].
void cast_heads(int dtype, const float* src, int64_t ld, int hstride, int n_heads, int n, void* dst,
                int64_t n_rows, hipStream_t s);

// out[t, :n] = RMSNorm(Σ_p proj[p*sps + t*ld + :n]) * gain (gain may be null: unit), in dtype.
bool norm_rows_supported(int n);
void norm_rows(int dtype, const float* proj, int64_t ld, int splits, int64_t sps, int n, const void* gain,
               float eps, void* out, int64_t ld_out, int64_t n_rows, hipStream_t s);

// Shape of one attention call, as the kernels see it.
struct AttnShape {
  int H, G, r, d_rope, row_w;  // row_w = r + G*d_rope
  float scale;
};

// Generic split-K attention over cache rows (any dtype/shape within limits).
// Query q (0..n_q-1) attends rows: decode (cu == nullptr): seq_start[q] + [0, seq_len[q]);
// prefill: rows cu[b] .. q, where cu[b] <= q < cu[b+1].
// n_split == 1: writes normalised o_ (fp32 [n_q, H, r]) to o_out.
// n_split > 1: writes partials part_o [n_q, n_split, H, r] and part_ml [n_q, n_split, H, 2].
void attend_generic(int dtype, const AttnShape& sh, const void* q_lat, const void* q_pe,
                    const void* cache, const int64_t* seq_start, const int32_t* seq_len,
                    const int64_t* cu, int batch, int64_t n_q, int n_split, int split_len,
                    void* part_o, float* part_ml, float* o_out, hipStream_t s);
int generic_head_block();

// Range checks of the device index arrays on host copies (checks.cpp): no-ops
// unless the library is built with MLA_DEBUG_CHECKS, where they copy the
// arrays to the host (synchronising) and return MLA_EINVAL for a bad one.
#ifdef MLA_DEBUG_CHECKS
constexpr bool kDebugChecks = true;
#else
constexpr bool kDebugChecks = false;
#endif
int debug_check_decode(const int64_t* seq_start, const int32_t* seq_len, int32_t batch, int32_t max_len);
int debug_check_prefill(const int64_t* cu_seqlens, int32_t batch, int64_t n_tokens, int32_t max_len);
int debug_check_write(const int64_t* slots, int64_t n_tokens, int64_t cache_rows);
// whether the generic kernel's LDS tile for this shape and element type fits a CU
bool attend_generic_fits(int dtype, const AttnShape& sh);

// Log-sum-exp merge of split partials into normalised o_ (fp32 [n_q, H, r]).
// part_o holds each split's normalised o_ in the layer's element type, query q's
// splits at items q·n_split ..; with ragged_items > 0 the items of the device
// plan over seq_len (ragged_plan in mla_device.h) instead.
void merge_splits(int dtype, const AttnShape& sh, int64_t n_q, int n_split, const void* part_o,
                  const float* part_ml, float* o_out, hipStream_t s, const int32_t* seq_len = nullptr,
                  int ragged_items = 0);

// bf16 MFMA decode kernel for the shapes it supports (see decode_mfma.hip).
// All 128 heads of a (sequence, split) per workgroup, for H = 128, G = 1,
// r = 512, d_rope = 64 (decode_wide.hip).
bool decode_wide_supported(const AttnShape& sh);
void decode_wide(const AttnShape& sh, const void* q_lat, const void* q_pe, const void* cache,
                 const int64_t* seq_start, const int32_t* seq_len, int batch, int n_split,
                 int split_len, void* part_o, float* part_ml, float* o_out, hipStream_t s);

bool decode_mfma_supported(const AttnShape& sh);
int decode_mfma_blocks_per_cu(const AttnShape& sh);  // workgroups one CU holds (LDS-limited)
int decode_mfma_head_groups(const AttnShape& sh);    // workgroups that share one sequence split
struct V4Epilogue;
// v4 (non-null: one split, a 16-head instance) writes the DeepSeek-V4 output
// directly (sink in the denominator, inverse rotation of the tail).
// ragged_items > 0 (shapes with one workgroup per split; at most 64 sequences,
// fewer than ragged_items): the grid is ragged_items workgroups and the split
// plan is made on the device from seq_len (ragged_plan); n_split and split_len
// are then unused and the partials are indexed by item.
void decode_mfma(const AttnShape& sh, const void* q_lat, const void* q_pe, const void* cache,
                 const int64_t* seq_start, const int32_t* seq_len, int batch, int n_split,
                 int split_len, void* part_o, float* part_ml, float* o_out, hipStream_t s,
                 const V4Epilogue* v4 = nullptr, int ragged_items = 0);
// The V4 variant's epilogue: the sink [H] (fp32 logits) joins each softmax's
// denominator and the last d_rope dims of the output are rotated back by the
// query's position (inverse frequencies from freqs, or theta).
struct V4Epilogue {
  void* out;  // bf16 [batch, H, r]
  const float* sink;
  double theta;
  const double* freqs;
  int d_rope;
};

// bf16 MFMA causal prefill kernel for the shapes it supports (see prefill_mfma.hip).
bool prefill_mfma_supported(const AttnShape& sh);
// Output: normalised o_ fp32 [T, H, r] in o_out, or (part_o non-null) bf16 o_ in
// part_o [T, H, r] with (reference max, row sum) per (token, head) in part_ml
// [T, H, 2] (base 2), a one-split state for the merge that adds a sink.
void prefill_mfma(const AttnShape& sh, const void* q_lat, const void* q_pe, const void* cache,
                  const int64_t* cu, int batch, int64_t n_tokens, int max_len, float* o_out,
                  void* part_o, float* part_ml, hipStream_t s);

// bf16 MFMA causal prefill in the original order (see prefill_expanded.hip):
// k_nope [H, T, d_nope] and v [H, T, d_v] already expanded (fp16), rotary keys
// from the cache rows, output [T, H, d_v] bf16.
// Columns of the transposed value rows vᵀ [H, d_v, cols]: n_tokens rounded up to 32.
int64_t prefill_expanded_vt_cols(int64_t n_tokens);
// Largest n_tokens the kernel addresses (128 vᵀ rows of one head within 32-bit offsets).
constexpr int64_t kPrefillExpandedMaxTokens = 16 * 1024 * 1024 - 32;
// Zero the pad columns [n_tokens, cols) of `rows` vᵀ rows (fp16).
void prefill_expanded_vt_pad(void* vt, int64_t rows, int64_t n_tokens, hipStream_t s);
bool prefill_expanded_supported(const AttnShape& sh, int d_nope, int d_v);
void prefill_expanded(const AttnShape& sh, const void* q_nope, const void* q_pe, const void* k_nope,
                      const void* v, const void* cache, const int64_t* cu, int batch, int64_t n_tokens,
                      void* out, hipStream_t s);

// DeepSeek-V4 variant (v4.hip).  Rows of width D from fp32 projections (K-slice
// sum): optional RMSNorm (norm != 0) with gain (null: unit), complex-form RoPE of the last
// d_rope dims at positions[t]; row r = (t = r / heads, h = r % heads) reads
// proj[t*ld + h*D], writes out[(slots ? slots[t] : r) * D].
bool v4_rows_supported(int D, int d_rope);
void v4_rows(int dtype, const float* proj, int64_t ld, int splits, int64_t sps, int heads, int D, int d_rope,
             int norm, const void* gain, float eps, const int32_t* positions, const int64_t* slots, double theta,
             const double* freqs, void* out, int64_t n_tokens, hipStream_t s);
// Split merge with the attention sink, then the inverse rotation of the last
// d_rope dims by the query position (decode: seq_len[q] - 1; prefill: offset in cu).
void v4_merge(int dtype, const void* part_o, const float* part_ml, int64_t n_q, int n_split, int H, int D,
              int d_rope, const float* sink, const int32_t* seq_len, const int64_t* cu, int batch, double theta,
              const double* freqs, void* out, hipStream_t s);

}  // namespace mla
