// C ABI of the MLA latent-cache hot path: argument validation, workspace
// planning and kernel launches.  The declarations and their contracts are in
// include/mla.h.  Nothing here allocates, frees or synchronises.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/mla.h"
#include "mla_internal.h"

namespace {

using mla::AttnShape;
using mla::GemmArgs;

constexpr size_t kAlign = 256;
constexpr int kMaxRank = 512;
constexpr int kCUs = 256;  // compute units of an MI355X (sizes the split of decode contexts)

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool ptr_ok(const void* p) { return p != nullptr && aligned16(p); }

AttnShape shape_of(const mla_dims* d);

int check_dims(const mla_dims* d) {
  if (!d) return MLA_EINVAL;
  if (d->d_model <= 0 || d->n_heads <= 0 || d->n_groups <= 0 || d->rank <= 0 || d->d_rope <= 0 ||
      d->d_nope <= 0 || d->d_v <= 0)
    return MLA_EINVAL;
  if (d->n_heads % d->n_groups != 0) return MLA_EINVAL;
  if (d->d_rope % 2 != 0) return MLA_EINVAL;
  if (d->dtype != MLA_F32 && d->dtype != MLA_BF16) return MLA_EINVAL;
  if (d->latent_rmsnorm != 0 && d->latent_rmsnorm != 1) return MLA_EINVAL;
  if (!(d->rms_eps >= 0.f) || !isfinite(d->rms_eps)) return MLA_EINVAL;
  if (isnan(d->softmax_scale) || isinf(d->softmax_scale)) return MLA_EINVAL;
  if (!(d->rope_theta > 0.0) || !isfinite(d->rope_theta)) return MLA_EINVAL;
  if (d->rope_freqs != nullptr && !aligned16(d->rope_freqs)) return MLA_EINVAL;
  // limits of the compiled kernels
  if (d->rank > kMaxRank || d->rank % 16 != 0) return MLA_ENOTSUP;
  if (d->dtype == MLA_BF16 && (d->d_model % 8 != 0 || d->d_nope % 8 != 0)) return MLA_ENOTSUP;
  // the cache-row epilogue holds one projected row (<= 1024 floats) and one
  // cos/sin table (<= 256 pairs) in LDS
  if (d->rank + static_cast<int64_t>(d->n_groups) * d->d_rope > 1024 || d->d_rope > 512) return MLA_ENOTSUP;
  // fp32 layers attend in the generic kernel, whose staged tile of 32 fp32 rows
  // must fit the 160 KB of LDS (cache rows up to 1017 values)
  if (d->dtype == MLA_F32 && !mla::attend_generic_fits(mla::kF32, shape_of(d))) return MLA_ENOTSUP;
  return MLA_OK;
}

float eff_scale(const mla_dims* d) {
  if (d->softmax_scale > 0.f) return d->softmax_scale;
  return 1.0f / sqrtf(static_cast<float>(d->d_nope + d->d_rope));
}

AttnShape shape_of(const mla_dims* d) {
  AttnShape s;
  s.H = d->n_heads;
  s.G = d->n_groups;
  s.r = d->rank;
  s.d_rope = d->d_rope;
  s.row_w = d->rank + d->n_groups * d->d_rope;
  s.scale = eff_scale(d);
  return s;
}

// How a decode call is split.  Shared by mla_workspace_size and mla_decode so the
// two always agree.
struct DecodePlan {
  bool wide;  // all heads per workgroup (decode_wide)
  bool mfma;
  int n_split;
  int split_len;
  // > 0: the MFMA kernel makes the split plan on the device from the lengths,
  // over this many workgroups (partial states indexed by item); 0: the plan above
  int ragged_items;
  size_t part_o_bytes, part_ml_bytes, o_bytes;
  size_t total() const { return part_o_bytes + part_ml_bytes + o_bytes; }
};

int split_rows(int L, int64_t ns, int unit = 64) {
  int split_len = static_cast<int>((L + ns - 1) / ns);
  return (split_len + unit - 1) / unit * unit;
}

DecodePlan decode_plan(const mla_dims* d, int32_t batch, int32_t max_len, int32_t force_splits = 0,
                       bool allow_ragged = true) {
  DecodePlan p{};
  AttnShape sh = shape_of(d);
  p.wide = d->dtype == MLA_BF16 && mla::decode_wide_supported(sh);
  p.mfma = !p.wide && d->dtype == MLA_BF16 && mla::decode_mfma_supported(sh);
  const int64_t B = std::max<int32_t>(batch, 0);
  const int L = std::max<int32_t>(max_len, 1);
  if (force_splits > 0) {
    p.split_len = split_rows(L, force_splits);
    p.n_split = force_splits;
    return p;
  }
  // Workgroups per split: the MFMA kernel splits the heads of a sequence over
  // decode_mfma_head_groups() workgroups; the generic kernel into 8-head blocks.
  const int64_t per_split =
      p.wide ? B
      : p.mfma ? B * mla::decode_mfma_head_groups(sh)
               : B * ((sh.H + mla::generic_head_block() - 1) / mla::generic_head_block());
  // Fill the 256 compute units of an MI355X once (the MFMA kernel's LDS
  // footprint allows one workgroup per CU at the large shapes), keeping
  // splits >= 256 rows (multiples of 64) for the MFMA kernels and >= 32 rows
  // (one tile) for the generic one, whose workgroups walk their rows serially:
  // a short context with few head blocks (the fp32 layer) would otherwise run
  // as a single workgroup.
  const bool generic = !p.wide && !p.mfma;
  const int64_t target =
      p.wide ? kCUs : p.mfma ? mla::decode_mfma_blocks_per_cu(sh) * kCUs : 2 * kCUs;
  int64_t ns = per_split > 0 ? (target + per_split - 1) / per_split : 1;
  const int64_t max_ns = std::max<int64_t>(1, L / (generic ? 32 : 256));
  ns = std::max<int64_t>(1, std::min<int64_t>(ns, max_ns));
  const int split_len = split_rows(L, ns, generic ? 32 : 64);
  ns = (L + split_len - 1) / split_len;
  p.n_split = static_cast<int>(ns);
  p.split_len = split_len;
  // A plan made here knows only the longest length, so a ragged batch leaves
  // most of the shorter sequences' splits empty.  Where the MFMA kernel takes a
  // whole split per workgroup and the merge is a separate kernel anyway (more
  // splits than the merge folded into W_UV takes), let the kernel plan over the
  // same number of workgroups from the lengths themselves (at most 64 of them).
  if (allow_ragged && p.mfma && mla::decode_mfma_head_groups(sh) == 1 && B <= 64 &&
      p.n_split > mla::skinny_max_merge())
    p.ragged_items = static_cast<int>(B) * p.n_split;
  p.o_bytes = align_up(static_cast<size_t>(B) * sh.H * sh.r * sizeof(float));
  const int64_t items = p.ragged_items > 0 ? p.ragged_items : (p.n_split > 1 ? B * p.n_split : 0);
  if (items > 0) {
    const size_t elem = d->dtype == MLA_F32 ? sizeof(float) : 2;  // partials in the layer's type
    p.part_o_bytes = align_up(static_cast<size_t>(items) * sh.H * sh.r * elem);
    p.part_ml_bytes = align_up(static_cast<size_t>(items) * sh.H * 2 * sizeof(float));
  }
  return p;
}

// Few-token bf16 projections stream their weights with the skinny kernel.
bool skinny_ok(const mla_dims* d, int64_t m) { return d->dtype == MLA_BF16 && m > 0 && m <= 64; }

// x [T, d_model] · [W0; W1]ᵀ -> fp32 C (row stride ldc), W0 giving columns [0, n0)
// and W1 columns [n0, n0 + n1).  The skinny kernel runs both weights in one
// launch and leaves `splits` K-slices (slice stride sps floats) for the consumer
// to sum; the tiled kernel runs once per weight and leaves one slice.
struct Proj {
  int splits;
  int64_t sps;
};

Proj proj_plan_k(const mla_dims* d, int n, int k, int64_t n_tokens, int64_t ldc) {
  Proj p{1, 0};
  if (skinny_ok(d, n_tokens)) {
    p.splits = mla::skinny_splits(static_cast<int>(n_tokens), n, 1, k);
    p.sps = static_cast<int64_t>(align_up(static_cast<size_t>(n_tokens) * ldc * sizeof(float)) / sizeof(float));
  }
  return p;
}

Proj proj_plan(const mla_dims* d, int n, int64_t n_tokens, int64_t ldc) {
  return proj_plan_k(d, n, d->d_model, n_tokens, ldc);
}

size_t proj_bytes_k(const mla_dims* d, int n, int k, int64_t n_tokens, int64_t ldc) {
  const Proj p = proj_plan_k(d, n, k, n_tokens, ldc);
  return static_cast<size_t>(p.splits) * align_up(static_cast<size_t>(n_tokens) * ldc * sizeof(float));
}

size_t proj_bytes(const mla_dims* d, int n, int64_t n_tokens, int64_t ldc) {
  return proj_bytes_k(d, n, d->d_model, n_tokens, ldc);
}

GemmArgs proj_args(const mla_dims* d, const void* x, const void* w, int n, float* c, int64_t ldc,
                   int64_t n_tokens) {
  GemmArgs g{};
  g.A = x;
  g.sAm = d->d_model;
  g.B = w;
  g.sBo = d->d_model;
  g.C = c;
  g.sCm = ldc;
  g.M = static_cast<int>(n_tokens);
  g.N = n;
  g.K = d->d_model;
  g.Z = 1;
  return g;
}

// C (fp32, row stride ldc) = A [T, k] (row stride lda, layer dtype) · Wᵀ, W [n, k].
// Few bf16 tokens: the weight-streaming kernel, leaving `splits` K slices.
Proj proj_one(const mla_dims* d, const void* a, int64_t lda, int k, const void* w, int n, float* c,
              int64_t ldc, int64_t n_tokens, hipStream_t s) {
  const Proj p = proj_plan_k(d, n, k, n_tokens, ldc);
  if (skinny_ok(d, n_tokens)) {
    mla::SkinnyArgs sa{};
    sa.A = a;
    sa.sAm = lda;
    sa.B0 = sa.B1 = static_cast<const uint16_t*>(w);
    sa.N0 = n;
    sa.sBo = k;
    sa.C = c;
    sa.sCm = ldc;
    sa.sPs = p.sps;
    sa.M = static_cast<int>(n_tokens);
    sa.N = n;
    sa.K = k;
    sa.Z = 1;
    sa.splits = p.splits;
    mla::gemm_skinny(sa, /*a_f32=*/false, /*out_bf16=*/false, s);
  } else {
    GemmArgs g{};
    g.A = a;
    g.sAm = lda;
    g.B = w;
    g.sBo = k;
    g.C = c;
    g.sCm = ldc;
    g.M = static_cast<int>(n_tokens);
    g.N = n;
    g.K = k;
    g.Z = 1;
    mla::gemm(g, d->dtype, false, false, false, s);
  }
  return p;
}

Proj proj_two(const mla_dims* d, const void* x, const void* w0, int n0, const void* w1, int n1,
              float* c, int64_t ldc, int64_t n_tokens, hipStream_t s) {
  const Proj p = proj_plan(d, n0 + n1, n_tokens, ldc);
  if (skinny_ok(d, n_tokens)) {
    mla::SkinnyArgs sa{};
    sa.A = x;
    sa.sAm = d->d_model;
    sa.B0 = static_cast<const uint16_t*>(w0);
    sa.B1 = static_cast<const uint16_t*>(w1);
    sa.N0 = n0;
    sa.sBo = d->d_model;
    sa.C = c;
    sa.sCm = ldc;
    sa.sPs = p.sps;
    sa.M = static_cast<int>(n_tokens);
    sa.N = n0 + n1;
    sa.K = d->d_model;
    sa.Z = 1;
    sa.splits = p.splits;
    mla::gemm_skinny(sa, /*a_f32=*/false, /*out_bf16=*/false, s);
  } else if (d->dtype == MLA_F32) {
    // the fp32 GEMM takes both weights in one launch
    GemmArgs g = proj_args(d, x, w0, n0 + n1, c, ldc, n_tokens);
    g.B1 = w1;
    g.N0 = n0;
    mla::gemm(g, d->dtype, false, false, false, s);
  } else {
    mla::gemm(proj_args(d, x, w0, n0, c, ldc, n_tokens), d->dtype, false, false, false, s);
    mla::gemm(proj_args(d, x, w1, n1, c + n0, ldc, n_tokens), d->dtype, false, false, false, s);
  }
  return p;
}

size_t prefill_ws(const mla_dims* d, int64_t n_tokens) {
  return align_up(static_cast<size_t>(std::max<int64_t>(n_tokens, 0)) * d->n_heads * d->rank *
                  sizeof(float));
}

int row_width(const mla_dims* d) { return d->rank + d->n_groups * d->d_rope; }
// fp32 query projection row: [q_nope (H x d_nope) | q_rope (H x d_rope)], padded to
// 8 floats so every row starts 32-byte aligned for the W_UK GEMM's vector loads.
int q_cols(const mla_dims* d) { return d->n_heads * (d->d_nope + d->d_rope); }
int64_t q_width(const mla_dims* d) { return (static_cast<int64_t>(q_cols(d)) + 7) / 8 * 8; }

size_t write_ws(const mla_dims* d, int64_t n_tokens) {
  const int64_t T = std::max<int64_t>(n_tokens, 0);
  return proj_bytes(d, row_width(d), T, row_width(d));
}

size_t absorb_ws(const mla_dims* d, int64_t n_tokens) {
  const int64_t T = std::max<int64_t>(n_tokens, 0);
  return proj_bytes(d, q_cols(d), T, q_width(d));
}

// Expanded keys and values of the original-order prefill: k_nope [H, T, d_nope]
// then v [H, T, d_v], fp16.
size_t expanded_k_bytes(const mla_dims* d, int64_t n_tokens) {
  return align_up(static_cast<size_t>(std::max<int64_t>(n_tokens, 0)) * d->n_heads * d->d_nope * 2);
}
size_t expanded_ws(const mla_dims* d, int64_t n_tokens) {
  return expanded_k_bytes(d, n_tokens) +
         align_up(static_cast<size_t>(mla::prefill_expanded_vt_cols(std::max<int64_t>(n_tokens, 0))) *
                  d->n_heads * d->d_v * 2);
}

// Low-rank query path: [x·W_QAᵀ fp32 slices][normalised rows, layer dtype][q fp32 slices]
int64_t lowrank_ld(int32_t q_rank) { return (static_cast<int64_t>(q_rank) + 7) / 8 * 8; }
struct LowrankWs {
  size_t cq, cqn, q;
  size_t total() const { return cq + cqn + q; }
};
LowrankWs lowrank_ws(const mla_dims* d, int32_t q_rank, int64_t n_tokens) {
  const int64_t T = std::max<int64_t>(n_tokens, 0);
  LowrankWs w{};
  w.cq = proj_bytes_k(d, q_rank, d->d_model, T, lowrank_ld(q_rank));
  w.cqn = align_up(static_cast<size_t>(T) * q_rank * (d->dtype == MLA_F32 ? 4 : 2));
  w.q = proj_bytes_k(d, q_cols(d), q_rank, T, q_width(d));
  return w;
}

// Output projection: fp32 slices of the few-token weight-streaming product
int64_t out_width(const mla_dims* d) { return (static_cast<int64_t>(d->d_model) + 7) / 8 * 8; }
size_t output_ws(const mla_dims* d, int64_t n_tokens) {
  const int64_t T = std::max<int64_t>(n_tokens, 0);
  if (!skinny_ok(d, T)) return 0;
  return proj_bytes_k(d, d->d_model, d->n_heads * d->d_v, T, out_width(d));
}

int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? MLA_OK : MLA_EHIP;
}

// out[q, h, :] = W_UV[h] · o_[q, h, :]   (o_ fp32 [n_q, H, r]; W_UV [H, d_v, r])
void apply_w_uv(const mla_dims* d, const float* o_lat, int64_t n_q, const void* w_uv, void* out,
                hipStream_t s) {
  if (skinny_ok(d, n_q)) {
    mla::SkinnyArgs sa{};
    sa.A = o_lat;
    sa.sAz = d->rank;
    sa.sAm = static_cast<int64_t>(d->n_heads) * d->rank;
    sa.B0 = sa.B1 = static_cast<const uint16_t*>(w_uv);
    sa.N0 = d->d_v;
    sa.sBz = static_cast<int64_t>(d->d_v) * d->rank;
    sa.sBo = d->rank;
    sa.C = out;
    sa.sCz = d->d_v;
    sa.sCm = static_cast<int64_t>(d->n_heads) * d->d_v;
    sa.M = static_cast<int>(n_q);
    sa.N = d->d_v;
    sa.K = d->rank;
    sa.Z = d->n_heads;
    sa.splits = 1;
    mla::gemm_skinny(sa, /*a_f32=*/true, /*out_bf16=*/true, s);
    return;
  }
  GemmArgs g{};
  g.A = o_lat;
  g.sAz = d->rank;
  g.sAm = static_cast<int64_t>(d->n_heads) * d->rank;
  g.B = w_uv;
  g.sBz = static_cast<int64_t>(d->d_v) * d->rank;
  g.sBo = d->rank;
  g.C = out;
  g.sCz = d->d_v;
  g.sCm = static_cast<int64_t>(d->n_heads) * d->d_v;
  g.M = static_cast<int>(n_q);
  g.N = d->d_v;
  g.K = d->rank;
  g.Z = d->n_heads;
  mla::gemm(g, d->dtype, /*a_f32=*/true, /*b_kn=*/false, /*out_bf16=*/d->dtype == MLA_BF16, s);
}

}  // namespace

extern "C" {

int mla_version(void) { return 101; }

const char* mla_strerror(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_EINVAL: return "invalid argument";
    case MLA_ENOTSUP: return "unsupported dimensions";
    case MLA_EWORKSPACE: return "workspace too small";
    case MLA_EHIP: return "HIP runtime error";
    case MLA_ESCRATCH: return "the call needs more than the static scratch array (MLA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int mla_check_dims(const mla_dims* dims) { return check_dims(dims); }

int mla_rope_yarn_table(int32_t d_rope, double theta, double factor, double original_window, double alpha,
                        double beta, double* out) {
  if (out == nullptr || d_rope <= 0 || d_rope % 2 != 0) return MLA_EINVAL;
  if (!(theta > 0.0) || !(factor > 0.0) || !(original_window > 0.0) || !(beta > alpha) ||
      !std::isfinite(theta) || !std::isfinite(factor) || !std::isfinite(original_window) || !std::isfinite(alpha) ||
      !std::isfinite(beta))
    return MLA_EINVAL;
  constexpr double kTwoPi = 6.283185307179586476925;
  for (int j = 0; j < d_rope / 2; ++j) {
    const double f = std::pow(theta, -2.0 * j / d_rope);
    const double turns = original_window * f / kTwoPi;  // turns of the pair over the original window
    const double g = std::min(1.0, std::max(0.0, (turns - alpha) / (beta - alpha)));
    out[j] = (1.0 - g) * f / factor + g * f;
  }
  return MLA_OK;
}

size_t mla_workspace_size(const mla_dims* dims, int op, int32_t batch, int64_t n_tokens,
                          int32_t max_len) {
  if (check_dims(dims) != MLA_OK) return 0;
  switch (op) {
    case MLA_OP_WRITE_CACHE: return write_ws(dims, n_tokens);
    case MLA_OP_ABSORB: return absorb_ws(dims, n_tokens);
    case MLA_OP_DECODE: return decode_plan(dims, batch, max_len).total();
    case MLA_OP_PREFILL: return prefill_ws(dims, n_tokens);
    case MLA_OP_QUERY: return absorb_ws(dims, n_tokens);
    case MLA_OP_PREFILL_EXPANDED: return expanded_ws(dims, n_tokens);
    case MLA_OP_OUTPUT: return output_ws(dims, n_tokens);
    default: return 0;
  }
}

int mla_write_cache(const mla_dims* dims, const void* x, const void* w_dkv, const void* w_kr,
                    const int32_t* positions, const int64_t* slots, int64_t n_tokens, void* cache,
                    int64_t cache_rows, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (n_tokens < 0 || cache_rows < 0) return MLA_EINVAL;
  if (n_tokens == 0) return MLA_OK;
  if (n_tokens > INT32_MAX) return MLA_ENOTSUP;
  if (!ptr_ok(x) || !ptr_ok(w_dkv) || !ptr_ok(w_kr) || !ptr_ok(positions) || !ptr_ok(slots) ||
      !ptr_ok(cache) || !ptr_ok(workspace))
    return MLA_EINVAL;
  if (workspace_bytes < write_ws(dims, n_tokens)) return MLA_EWORKSPACE;
  if (mla::kDebugChecks) {
    const int dc = mla::debug_check_write(slots, n_tokens, cache_rows);
    if (dc != MLA_OK) return dc;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int row_w = row_width(dims);
  float* proj = static_cast<float*>(workspace);
  const Proj p = proj_two(dims, x, w_dkv, dims->rank, w_kr, dims->n_groups * dims->d_rope, proj,
                          row_w, n_tokens, s);
  mla::finalize_cache_rows(dims->dtype, proj, row_w, p.splits, p.sps, cache, slots, positions,
                           n_tokens, dims->rank, dims->n_groups, dims->d_rope, dims->latent_rmsnorm,
                           dims->rms_eps, dims->rope_theta, dims->rope_freqs, s);
  return launch_status();
}

}  // extern "C"

namespace {
// The absorption after the query projection: q (fp32 rows [q_nope | q_rope],
// p.splits K slices) -> q_pe = RoPE(q_rope) and q_lat = q_nope·W_UK per head.
void absorb_finish(const mla_dims* dims, float* q, const Proj& p, const void* w_uk,
                   const int32_t* positions, int64_t n_tokens, void* q_lat, void* q_pe, hipStream_t s) {
  const int H = dims->n_heads;
  const int64_t ld = q_width(dims);
  mla::finalize_query(dims->dtype, q, ld, p.splits, p.sps, q_cols(dims), H * dims->d_nope, dims->d_rope, q_pe,
                      positions, n_tokens, H, dims->d_rope, dims->rope_theta, dims->rope_freqs, s);
  // q_lat[t,h,:] = Σ_d q_nope[t,h,d] W_UK[h,d,:]   (batched over heads)
  GemmArgs a{};
  a.A = q;
  a.sAz = dims->d_nope;
  a.sAm = ld;
  a.B = w_uk;
  a.sBz = static_cast<int64_t>(dims->d_nope) * dims->rank;
  a.sBo = dims->rank;
  a.C = q_lat;
  a.sCz = dims->rank;
  a.sCm = static_cast<int64_t>(H) * dims->rank;
  a.M = static_cast<int>(n_tokens);
  a.N = dims->rank;
  a.K = dims->d_nope;
  a.Z = H;
  mla::gemm(a, dims->dtype, /*a_f32=*/true, /*b_kn=*/true, dims->dtype == MLA_BF16, s);
}

// C (fp32, row stride ldc) = A [T, k] (bf16, row stride lda) · Wᵀ with W [n, k] in
// the tiled layout; the same K-slice plan as proj_one / proj_two (few tokens)
Proj proj_tiled(const mla_dims* d, const void* a, int64_t lda, int k, const void* w_tiled, int n, float* c,
                int64_t ldc, int64_t n_tokens, hipStream_t s) {
  const Proj p = proj_plan_k(d, n, k, n_tokens, ldc);
  mla::SkinnyArgs sa{};
  sa.A = a;
  sa.sAm = lda;
  sa.Bt = static_cast<const uint16_t*>(w_tiled);
  sa.N0 = n;
  sa.C = c;
  sa.sCm = ldc;
  sa.sPs = p.sps;
  sa.M = static_cast<int>(n_tokens);
  sa.N = n;
  sa.K = k;
  sa.Z = 1;
  sa.splits = p.splits;
  mla::gemm_skinny_tiled(sa, /*out_bf16=*/false, s);
  return p;
}
}  // namespace

extern "C" {

int mla_absorb(const mla_dims* dims, const void* x, const void* w_qc, const void* w_qr,
               const void* w_uk, const int32_t* positions, int64_t n_tokens, void* q_lat,
               void* q_pe, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (n_tokens < 0) return MLA_EINVAL;
  if (n_tokens == 0) return MLA_OK;
  if (n_tokens > INT32_MAX) return MLA_ENOTSUP;
  if (!ptr_ok(x) || !ptr_ok(w_qc) || !ptr_ok(w_qr) || !ptr_ok(w_uk) || !ptr_ok(positions) ||
      !ptr_ok(q_lat) || !ptr_ok(q_pe) || !ptr_ok(workspace))
    return MLA_EINVAL;
  if (workspace_bytes < absorb_ws(dims, n_tokens)) return MLA_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int H = dims->n_heads;
  const int64_t ld = q_width(dims);
  // one fp32 row per token: [q_nope (H x d_nope) | q_rope (H x d_rope)]
  float* q = static_cast<float*>(workspace);
  const Proj p = proj_two(dims, x, w_qc, H * dims->d_nope, w_qr, H * dims->d_rope, q, ld, n_tokens, s);
  absorb_finish(dims, q, p, w_uk, positions, n_tokens, q_lat, q_pe, s);
  return launch_status();
}

size_t mla_tiled_weight_bytes(int64_t n_rows, int64_t k) {
  if (n_rows <= 0 || k <= 0) return 0;
  return static_cast<size_t>(mla::tiled_weight_bytes(n_rows, k));
}

int mla_tile_weights(const void* w0, int64_t n0, const void* w1, int64_t n1, int64_t k, void* out,
                     size_t out_bytes, void* stream) {
  if (n0 < 0 || n1 < 0 || n0 + n1 <= 0 || k <= 0 || k % 8 != 0) return MLA_EINVAL;
  if (n0 + n1 > INT32_MAX || k > INT32_MAX) return MLA_ENOTSUP;
  if ((n0 > 0 && !ptr_ok(w0)) || (n1 > 0 && !ptr_ok(w1)) || !ptr_ok(out)) return MLA_EINVAL;
  if (out_bytes < mla_tiled_weight_bytes(n0 + n1, k)) return MLA_EINVAL;
  mla::tile_weights(static_cast<const uint16_t*>(w0), n0, static_cast<const uint16_t*>(w1), n1, k,
                    static_cast<uint16_t*>(out), static_cast<hipStream_t>(stream));
  return launch_status();
}

int mla_absorb_tiled(const mla_dims* dims, const void* x, const void* w_q_tiled, const void* w_uk,
                     const int32_t* positions, int64_t n_tokens, void* q_lat, void* q_pe, void* workspace,
                     size_t workspace_bytes, void* stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (n_tokens < 0) return MLA_EINVAL;
  if (n_tokens == 0) return MLA_OK;
  if (dims->dtype != MLA_BF16 || n_tokens > 64) return MLA_ENOTSUP;
  if (!ptr_ok(x) || !ptr_ok(w_q_tiled) || !ptr_ok(w_uk) || !ptr_ok(positions) || !ptr_ok(q_lat) ||
      !ptr_ok(q_pe) || !ptr_ok(workspace))
    return MLA_EINVAL;
  if (workspace_bytes < absorb_ws(dims, n_tokens)) return MLA_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* q = static_cast<float*>(workspace);
  const Proj p = proj_tiled(dims, x, dims->d_model, dims->d_model, w_q_tiled, q_cols(dims), q, q_width(dims),
                            n_tokens, s);
  absorb_finish(dims, q, p, w_uk, positions, n_tokens, q_lat, q_pe, s);
  return launch_status();
}

int mla_decode(const mla_dims* dims, const void* q_lat, const void* q_pe, const void* cache,
               const int64_t* seq_start, const int32_t* seq_len, int32_t batch, int32_t max_len,
               const void* w_uv, void* out, void* workspace, size_t workspace_bytes,
               void* stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 0) return MLA_EINVAL;
  if (batch == 0) return MLA_OK;
  if (max_len <= 0) return MLA_EINVAL;
  if (!ptr_ok(q_lat) || !ptr_ok(q_pe) || !ptr_ok(cache) || !ptr_ok(seq_start) ||
      !ptr_ok(seq_len) || !ptr_ok(w_uv) || !ptr_ok(out) || !ptr_ok(workspace))
    return MLA_EINVAL;
  DecodePlan p = decode_plan(dims, batch, max_len);
  if (workspace_bytes < p.total()) return MLA_EWORKSPACE;
  if (mla::kDebugChecks) {
    const int dc = mla::debug_check_decode(seq_start, seq_len, batch, max_len);
    if (dc != MLA_OK) return dc;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  AttnShape sh = shape_of(dims);
  char* ws = static_cast<char*>(workspace);
  float* o_lat = reinterpret_cast<float*>(ws);
  const bool parts = p.ragged_items > 0 || p.n_split > 1;
  void* part_o = parts ? static_cast<void*>(ws + p.o_bytes) : nullptr;
  float* part_ml = parts ? reinterpret_cast<float*>(ws + p.o_bytes + p.part_o_bytes) : nullptr;
  if (p.wide)
    mla::decode_wide(sh, q_lat, q_pe, cache, seq_start, seq_len, batch, p.n_split, p.split_len,
                     part_o, part_ml, o_lat, s);
  else if (p.mfma)
    mla::decode_mfma(sh, q_lat, q_pe, cache, seq_start, seq_len, batch, p.n_split, p.split_len,
                     part_o, part_ml, o_lat, s, nullptr, p.ragged_items);
  else
    mla::attend_generic(dims->dtype, sh, q_lat, q_pe, cache, seq_start, seq_len, nullptr, batch,
                        batch, p.n_split, p.split_len, part_o, part_ml, o_lat, s);
  if (p.ragged_items > 0) {
    mla::merge_splits(dims->dtype, sh, batch, p.n_split, part_o, part_ml, o_lat, s, seq_len, p.ragged_items);
    apply_w_uv(dims, o_lat, batch, w_uv, out, s);
    return launch_status();
  }
  if (p.n_split > 1 && skinny_ok(dims, batch) && p.n_split <= mla::skinny_max_merge()) {
    // split merge folded into the W_UV operand load:
    //   out[b,h,:] = W_UV[h] · Σ_j w_j(b,h) part_o[b,j,h,:]
    mla::SkinnyArgs sa{};
    sa.A = part_o;
    sa.sAz = dims->rank;
    sa.sAm = static_cast<int64_t>(p.n_split) * dims->n_heads * dims->rank;
    sa.sAs = static_cast<int64_t>(dims->n_heads) * dims->rank;
    sa.ml = part_ml;
    sa.ml_heads = dims->n_heads;
    sa.B0 = sa.B1 = static_cast<const uint16_t*>(w_uv);
    sa.N0 = dims->d_v;
    sa.sBz = static_cast<int64_t>(dims->d_v) * dims->rank;
    sa.sBo = dims->rank;
    sa.C = out;
    sa.sCz = dims->d_v;
    sa.sCm = static_cast<int64_t>(dims->n_heads) * dims->d_v;
    sa.M = batch;
    sa.N = dims->d_v;
    sa.K = dims->rank;
    sa.Z = dims->n_heads;
    mla::gemm_skinny_merged(sa, p.n_split, /*out_bf16=*/true, s);
    return launch_status();
  }
  if (p.n_split > 1) mla::merge_splits(dims->dtype, sh, batch, p.n_split, part_o, part_ml, o_lat, s);
  apply_w_uv(dims, o_lat, batch, w_uv, out, s);
  return launch_status();
}

int32_t mla_decode_splits(const mla_dims* dims, int32_t batch, int32_t max_len) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 0 || max_len <= 0) return MLA_EINVAL;
  return decode_plan(dims, batch, max_len, 0, /*allow_ragged=*/false).n_split;
}

int32_t mla_decode_split_rows(const mla_dims* dims, int32_t batch, int32_t max_len) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 0 || max_len <= 0) return MLA_EINVAL;
  return decode_plan(dims, batch, max_len, 0, /*allow_ragged=*/false).split_len;
}

int mla_decode_partials(const mla_dims* dims, const void* q_lat, const void* q_pe,
                        const void* cache, const int64_t* seq_start, const int32_t* seq_len,
                        int32_t batch, int32_t max_len, int32_t n_split, void* part_o,
                        float* part_ml, void* stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 0 || n_split < 1) return MLA_EINVAL;
  if (batch == 0) return MLA_OK;
  if (max_len <= 0) return MLA_EINVAL;
  if (!ptr_ok(q_lat) || !ptr_ok(q_pe) || !ptr_ok(cache) || !ptr_ok(seq_start) ||
      !ptr_ok(seq_len) || !ptr_ok(part_o) || !ptr_ok(part_ml))
    return MLA_EINVAL;
  const DecodePlan p = decode_plan(dims, batch, max_len, n_split);
  if (mla::kDebugChecks) {
    const int dc = mla::debug_check_decode(seq_start, seq_len, batch, max_len);
    if (dc != MLA_OK) return dc;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  AttnShape sh = shape_of(dims);
  if (p.wide)
    mla::decode_wide(sh, q_lat, q_pe, cache, seq_start, seq_len, batch, p.n_split, p.split_len,
                     part_o, part_ml, nullptr, s);
  else if (p.mfma)
    mla::decode_mfma(sh, q_lat, q_pe, cache, seq_start, seq_len, batch, p.n_split, p.split_len,
                     part_o, part_ml, nullptr, s);
  else
    mla::attend_generic(dims->dtype, sh, q_lat, q_pe, cache, seq_start, seq_len, nullptr, batch,
                        batch, p.n_split, p.split_len, part_o, part_ml, nullptr, s);
  return launch_status();
}

int mla_prefill(const mla_dims* dims, const void* q_lat, const void* q_pe, const void* cache,
                const int64_t* cu_seqlens, int32_t batch, int64_t n_tokens, int32_t max_len,
                const void* w_uv, void* out, void* workspace, size_t workspace_bytes,
                void* stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 0 || n_tokens < 0) return MLA_EINVAL;
  if (batch == 0 || n_tokens == 0) return MLA_OK;
  if (max_len <= 0) return MLA_EINVAL;
  if (n_tokens > INT32_MAX) return MLA_ENOTSUP;
  if (!ptr_ok(q_lat) || !ptr_ok(q_pe) || !ptr_ok(cache) || !ptr_ok(cu_seqlens) || !ptr_ok(w_uv) ||
      !ptr_ok(out) || !ptr_ok(workspace))
    return MLA_EINVAL;
  if (workspace_bytes < prefill_ws(dims, n_tokens)) return MLA_EWORKSPACE;
  if (mla::kDebugChecks) {
    const int dc = mla::debug_check_prefill(cu_seqlens, batch, n_tokens, max_len);
    if (dc != MLA_OK) return dc;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  AttnShape sh = shape_of(dims);
  float* o_lat = static_cast<float*>(workspace);
  if (dims->dtype == MLA_BF16 && mla::prefill_mfma_supported(sh))
    mla::prefill_mfma(sh, q_lat, q_pe, cache, cu_seqlens, batch, n_tokens, max_len, o_lat, nullptr, nullptr, s);
  else
    mla::attend_generic(dims->dtype, sh, q_lat, q_pe, cache, nullptr, nullptr, cu_seqlens, batch,
                        n_tokens, 1, max_len, nullptr, nullptr, o_lat, s);
  apply_w_uv(dims, o_lat, n_tokens, w_uv, out, s);
  return launch_status();
}

int mla_query(const mla_dims* dims, const void* x, const void* w_qc, const void* w_qr,
              const int32_t* positions, int64_t n_tokens, void* q_nope, void* q_pe, void* workspace,
              size_t workspace_bytes, void* stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (n_tokens < 0) return MLA_EINVAL;
  if (n_tokens == 0) return MLA_OK;
  if (n_tokens > INT32_MAX) return MLA_ENOTSUP;
  if (!ptr_ok(x) || !ptr_ok(w_qc) || !ptr_ok(w_qr) || !ptr_ok(positions) || !ptr_ok(q_nope) ||
      !ptr_ok(q_pe) || !ptr_ok(workspace))
    return MLA_EINVAL;
  if (workspace_bytes < absorb_ws(dims, n_tokens)) return MLA_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int H = dims->n_heads;
  const int64_t ld = q_width(dims);
  float* q = static_cast<float*>(workspace);
  const Proj p = proj_two(dims, x, w_qc, H * dims->d_nope, w_qr, H * dims->d_rope, q, ld, n_tokens, s);
  mla::finalize_query(dims->dtype, q, ld, p.splits, p.sps, q_cols(dims), H * dims->d_nope, dims->d_rope, q_pe,
                      positions, n_tokens, H, dims->d_rope, dims->rope_theta, dims->rope_freqs, s);
  mla::cast_heads(dims->dtype, q, ld, dims->d_nope, H, dims->d_nope, q_nope, n_tokens, s);
  return launch_status();
}

int mla_prefill_expanded(const mla_dims* dims, const void* q_nope, const void* q_pe, const void* cache,
                         const int64_t* cu_seqlens, int32_t batch, int64_t n_tokens, int32_t max_len,
                         const void* w_uk, const void* w_uv, void* out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 0 || n_tokens < 0) return MLA_EINVAL;
  if (batch == 0 || n_tokens == 0) return MLA_OK;
  if (max_len <= 0) return MLA_EINVAL;
  if (n_tokens > mla::kPrefillExpandedMaxTokens) return MLA_ENOTSUP;
  const AttnShape sh = shape_of(dims);
  if (dims->dtype != MLA_BF16 || !mla::prefill_expanded_supported(sh, dims->d_nope, dims->d_v))
    return MLA_ENOTSUP;
  if (!ptr_ok(q_nope) || !ptr_ok(q_pe) || !ptr_ok(cache) || !ptr_ok(cu_seqlens) || !ptr_ok(w_uk) ||
      !ptr_ok(w_uv) || !ptr_ok(out) || !ptr_ok(workspace))
    return MLA_EINVAL;
  if (workspace_bytes < expanded_ws(dims, n_tokens)) return MLA_EWORKSPACE;
  if (mla::kDebugChecks) {
    const int dc = mla::debug_check_prefill(cu_seqlens, batch, n_tokens, max_len);
    if (dc != MLA_OK) return dc;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int H = dims->n_heads;
  const int T = static_cast<int>(n_tokens);
  char* ws = static_cast<char*>(workspace);
  void* k_nope = ws;
  void* v = ws + expanded_k_bytes(dims, n_tokens);
  // k_nope[h, t, :] = W_UK[h] · c[t]  and  vᵀ[h, :, t] = W_UV[h] · c[t]  (c = cache row t, cols 0..r),
  // stored in fp16: three more significant bits than bf16 for the two operands
  // this order rounds and the absorbed one does not.  v is kept transposed
  // (rows of T_pad keys, the pad zero) for the attention kernel's PV operand.
  GemmArgs g{};
  g.A = cache;
  g.sAz = 0;
  g.sAm = sh.row_w;
  g.B = w_uk;
  g.sBz = static_cast<int64_t>(dims->d_nope) * dims->rank;
  g.sBo = dims->rank;
  g.C = k_nope;
  g.sCz = static_cast<int64_t>(T) * dims->d_nope;
  g.sCm = dims->d_nope;
  g.M = T;
  g.N = dims->d_nope;
  g.K = dims->rank;
  g.Z = H;
  mla::gemm_f16_out(g, s);
  const int64_t t_pad = mla::prefill_expanded_vt_cols(T);
  GemmArgs gv{};
  gv.A = w_uv;
  gv.sAz = static_cast<int64_t>(dims->d_v) * dims->rank;
  gv.sAm = dims->rank;
  gv.B = cache;
  gv.sBz = 0;
  gv.sBo = sh.row_w;
  gv.C = v;
  gv.sCz = static_cast<int64_t>(dims->d_v) * t_pad;
  gv.sCm = t_pad;
  gv.M = dims->d_v;
  gv.N = T;
  gv.K = dims->rank;
  gv.Z = H;
  mla::gemm_f16_out(gv, s);
  mla::prefill_expanded_vt_pad(v, static_cast<int64_t>(H) * dims->d_v, T, s);
  mla::prefill_expanded(sh, q_nope, q_pe, k_nope, v, cache, cu_seqlens, batch, n_tokens, out, s);
  return launch_status();
}

size_t mla_lowrank_workspace_size(const mla_dims* dims, int32_t q_rank, int64_t n_tokens) {
  if (check_dims(dims) != MLA_OK || q_rank <= 0) return 0;
  return lowrank_ws(dims, q_rank, n_tokens).total();
}

namespace {

// Shared front of the low-rank query calls: q = RMSNorm(x·W_QAᵀ)·gain · W_QBᵀ into
// the fp32 rows of the workspace ([H, d_nope + d_rope] per token), q_pe rotated.
// Returns the fp32 rows (row stride q_width) or nullptr after an argument error in *st.
// tiled: W_QA and W_QB in the tiled layout (bf16, at most 64 tokens)
float* lowrank_front(const mla_dims* dims, int32_t q_rank, const void* x, const void* w_qa,
                     const void* q_gain, const void* w_qb, const int32_t* positions, int64_t n_tokens,
                     void* q_pe, void* workspace, size_t workspace_bytes, hipStream_t s, int* st,
                     bool tiled = false) {
  *st = check_dims(dims);
  if (*st != MLA_OK) return nullptr;
  if (q_rank <= 0 || n_tokens < 0) {
    *st = MLA_EINVAL;
    return nullptr;
  }
  if (q_rank % 8 != 0 || !mla::norm_rows_supported(q_rank) || n_tokens > INT32_MAX ||
      (tiled && n_tokens > 0 && (dims->dtype != MLA_BF16 || n_tokens > 64))) {
    *st = MLA_ENOTSUP;
    return nullptr;
  }
  if (n_tokens == 0) return nullptr;
  if (!ptr_ok(x) || !ptr_ok(w_qa) || (q_gain != nullptr && !ptr_ok(q_gain)) || !ptr_ok(w_qb) ||
      !ptr_ok(positions) || !ptr_ok(q_pe) || !ptr_ok(workspace)) {
    *st = MLA_EINVAL;
    return nullptr;
  }
  const LowrankWs w = lowrank_ws(dims, q_rank, n_tokens);
  if (workspace_bytes < w.total()) {
    *st = MLA_EWORKSPACE;
    return nullptr;
  }
  char* base = static_cast<char*>(workspace);
  float* cq = reinterpret_cast<float*>(base);
  void* cqn = base + w.cq;
  float* q = reinterpret_cast<float*>(base + w.cq + w.cqn);
  const int64_t ldq = lowrank_ld(q_rank);
  const Proj p1 = tiled ? proj_tiled(dims, x, dims->d_model, dims->d_model, w_qa, q_rank, cq, ldq, n_tokens, s)
                        : proj_one(dims, x, dims->d_model, dims->d_model, w_qa, q_rank, cq, ldq, n_tokens, s);
  mla::norm_rows(dims->dtype, cq, ldq, p1.splits, p1.sps, q_rank, q_gain, dims->rms_eps, cqn, q_rank,
                 n_tokens, s);
  const int64_t ld = q_width(dims);
  const Proj p2 = tiled ? proj_tiled(dims, cqn, q_rank, q_rank, w_qb, q_cols(dims), q, ld, n_tokens, s)
                        : proj_one(dims, cqn, q_rank, q_rank, w_qb, q_cols(dims), q, ld, n_tokens, s);
  const int hw = dims->d_nope + dims->d_rope;
  mla::finalize_query(dims->dtype, q, ld, p2.splits, p2.sps, q_cols(dims), dims->d_nope, hw, q_pe, positions,
                      n_tokens, dims->n_heads, dims->d_rope, dims->rope_theta, dims->rope_freqs, s);
  return q;
}

int absorb_lowrank(const mla_dims* dims, int32_t q_rank, const void* x, const void* w_qa, const void* q_gain,
                   const void* w_qb, const void* w_uk, const int32_t* positions, int64_t n_tokens, void* q_lat,
                   void* q_pe, void* workspace, size_t workspace_bytes, void* stream, bool tiled) {
  const int st0 = check_dims(dims);
  if (st0 != MLA_OK) return st0;
  if (n_tokens > 0 && (!ptr_ok(w_uk) || !ptr_ok(q_lat))) return MLA_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int st = MLA_OK;
  float* q = lowrank_front(dims, q_rank, x, w_qa, q_gain, w_qb, positions, n_tokens, q_pe, workspace,
                           workspace_bytes, s, &st, tiled);
  if (q == nullptr) return st;
  const int H = dims->n_heads;
  GemmArgs a{};
  a.A = q;
  a.sAz = dims->d_nope + dims->d_rope;
  a.sAm = q_width(dims);
  a.B = w_uk;
  a.sBz = static_cast<int64_t>(dims->d_nope) * dims->rank;
  a.sBo = dims->rank;
  a.C = q_lat;
  a.sCz = dims->rank;
  a.sCm = static_cast<int64_t>(H) * dims->rank;
  a.M = static_cast<int>(n_tokens);
  a.N = dims->rank;
  a.K = dims->d_nope;
  a.Z = H;
  mla::gemm(a, dims->dtype, /*a_f32=*/true, /*b_kn=*/true, dims->dtype == MLA_BF16, s);
  return launch_status();
}

}  // namespace

int mla_absorb_lowrank(const mla_dims* dims, int32_t q_rank, const void* x, const void* w_qa,
                       const void* q_gain, const void* w_qb, const void* w_uk, const int32_t* positions,
                       int64_t n_tokens, void* q_lat, void* q_pe, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return absorb_lowrank(dims, q_rank, x, w_qa, q_gain, w_qb, w_uk, positions, n_tokens, q_lat, q_pe, workspace,
                        workspace_bytes, stream, false);
}

int mla_absorb_lowrank_tiled(const mla_dims* dims, int32_t q_rank, const void* x, const void* w_qa_tiled,
                             const void* q_gain, const void* w_qb_tiled, const void* w_uk,
                             const int32_t* positions, int64_t n_tokens, void* q_lat, void* q_pe,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return absorb_lowrank(dims, q_rank, x, w_qa_tiled, q_gain, w_qb_tiled, w_uk, positions, n_tokens, q_lat, q_pe,
                        workspace, workspace_bytes, stream, true);
}

int mla_query_lowrank(const mla_dims* dims, int32_t q_rank, const void* x, const void* w_qa,
                      const void* q_gain, const void* w_qb, const int32_t* positions, int64_t n_tokens,
                      void* q_nope, void* q_pe, void* workspace, size_t workspace_bytes, void* stream) {
  const int st0 = check_dims(dims);
  if (st0 != MLA_OK) return st0;
  if (n_tokens > 0 && !ptr_ok(q_nope)) return MLA_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int st = MLA_OK;
  float* q = lowrank_front(dims, q_rank, x, w_qa, q_gain, w_qb, positions, n_tokens, q_pe, workspace,
                           workspace_bytes, s, &st);
  if (q == nullptr) return st;
  mla::cast_heads(dims->dtype, q, q_width(dims), dims->d_nope + dims->d_rope, dims->n_heads, dims->d_nope,
                  q_nope, n_tokens, s);
  return launch_status();
}

int mla_output(const mla_dims* dims, const void* attn, const void* w_o, int64_t n_tokens, void* out,
               void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (n_tokens < 0) return MLA_EINVAL;
  if (n_tokens == 0) return MLA_OK;
  if (n_tokens > INT32_MAX) return MLA_ENOTSUP;
  const int K = dims->n_heads * dims->d_v;
  if (dims->dtype == MLA_BF16 && K % 8 != 0) return MLA_ENOTSUP;
  const size_t need = output_ws(dims, n_tokens);
  if (!ptr_ok(attn) || !ptr_ok(w_o) || !ptr_ok(out) || (need > 0 && !ptr_ok(workspace))) return MLA_EINVAL;
  if (workspace_bytes < need) return MLA_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (need > 0) {
    // few tokens: stream W_o once, K slices in fp32, then sum and cast
    float* c = static_cast<float*>(workspace);
    const int64_t ld = out_width(dims);
    const Proj p = proj_one(dims, attn, K, K, w_o, dims->d_model, c, ld, n_tokens, s);
    mla::sum_cast_slices(dims->dtype, c, p.splits, p.sps, static_cast<int>(n_tokens), dims->d_model, ld, out, s);
  } else {
    GemmArgs g{};
    g.A = attn;
    g.sAm = K;
    g.B = w_o;
    g.sBo = K;
    g.C = out;
    g.sCm = dims->d_model;
    g.M = static_cast<int>(n_tokens);
    g.N = dims->d_model;
    g.K = K;
    g.Z = 1;
    mla::gemm(g, dims->dtype, /*a_f32=*/false, /*b_kn=*/false, /*out_bf16=*/dims->dtype == MLA_BF16, s);
  }
  return launch_status();
}

int mla_output_tiled(const mla_dims* dims, const void* attn, const void* w_o_tiled, int64_t n_tokens,
                     void* out, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (n_tokens < 0) return MLA_EINVAL;
  if (n_tokens == 0) return MLA_OK;
  const int K = dims->n_heads * dims->d_v;
  if (dims->dtype != MLA_BF16 || n_tokens > 64 || K % 8 != 0) return MLA_ENOTSUP;
  const size_t need = output_ws(dims, n_tokens);
  if (!ptr_ok(attn) || !ptr_ok(w_o_tiled) || !ptr_ok(out) || !ptr_ok(workspace)) return MLA_EINVAL;
  if (workspace_bytes < need) return MLA_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* c = static_cast<float*>(workspace);
  const int64_t ld = out_width(dims);
  const Proj p = proj_tiled(dims, attn, K, K, w_o_tiled, dims->d_model, c, ld, n_tokens, s);
  mla::sum_cast_slices(dims->dtype, c, p.splits, p.sps, static_cast<int>(n_tokens), dims->d_model, ld, out, s);
  return launch_status();
}

}  // extern "C"

// ---------------------------------------------------------------------------
// DeepSeek-V4 variant
// ---------------------------------------------------------------------------
namespace {

int v4_check(const mla_v4_dims* d) {
  if (!d) return MLA_EINVAL;
  if (d->d_model <= 0 || d->n_heads <= 0 || d->head_dim <= 0 || d->d_rope < 0 || d->q_rank <= 0 ||
      d->o_groups <= 0 || d->o_rank <= 0)
    return MLA_EINVAL;
  if (d->d_rope % 2 != 0 || d->d_rope > d->head_dim) return MLA_EINVAL;
  if ((static_cast<int64_t>(d->n_heads) * d->head_dim) % d->o_groups != 0) return MLA_EINVAL;
  if (d->dtype != MLA_F32 && d->dtype != MLA_BF16) return MLA_EINVAL;
  if (!(d->rms_eps >= 0.f) || !isfinite(d->rms_eps)) return MLA_EINVAL;
  if (isnan(d->softmax_scale) || isinf(d->softmax_scale)) return MLA_EINVAL;
  if (!(d->rope_theta > 0.0) || !isfinite(d->rope_theta)) return MLA_EINVAL;
  const int64_t gdim = static_cast<int64_t>(d->n_heads) * d->head_dim / d->o_groups;
  if (d->dtype != MLA_BF16 || d->head_dim > 512 || d->head_dim % 16 != 0 || d->d_model % 8 != 0 ||
      d->q_rank % 8 != 0 || !mla::norm_rows_supported(d->q_rank) || d->o_rank % 8 != 0 || gdim % 8 != 0 ||
      !mla::v4_rows_supported(d->head_dim, d->d_rope))
    return MLA_ENOTSUP;
  return MLA_OK;
}

// The projection helpers above only look at the element type.
mla_dims v4_shadow(const mla_v4_dims* d) {
  mla_dims s{};
  s.d_model = d->d_model;
  s.dtype = d->dtype;
  return s;
}

AttnShape v4_shape(const mla_v4_dims* d) {
  AttnShape s;
  s.H = d->n_heads;
  s.G = 1;
  s.r = d->head_dim;
  s.d_rope = 0;  // the rotary dims are inside the row
  s.row_w = d->head_dim;
  s.scale = d->softmax_scale > 0.f ? d->softmax_scale : 1.0f / sqrtf(static_cast<float>(d->head_dim));
  return s;
}

struct V4Decode {
  bool mfma;
  int n_split, split_len;
  size_t part_o, part_ml;
};

V4Decode v4_decode_plan(const mla_v4_dims* d, int32_t batch, int32_t max_len) {
  V4Decode p{};
  const AttnShape sh = v4_shape(d);
  p.mfma = mla::decode_mfma_supported(sh);
  const int64_t B = std::max<int32_t>(batch, 0);
  const int L = std::max<int32_t>(max_len, 1);
  const int64_t per = p.mfma ? B : B * ((sh.H + mla::generic_head_block() - 1) / mla::generic_head_block());
  const int64_t target = p.mfma ? mla::decode_mfma_blocks_per_cu(sh) * kCUs : 2 * kCUs;
  int64_t ns = per > 0 ? (target + per - 1) / per : 1;
  ns = std::max<int64_t>(1, std::min<int64_t>(ns, std::max<int64_t>(1, L / 256)));
  p.split_len = split_rows(L, ns);
  p.n_split = (L + p.split_len - 1) / p.split_len;
  p.part_o = align_up(static_cast<size_t>(B) * p.n_split * sh.H * d->head_dim * 2);
  p.part_ml = align_up(static_cast<size_t>(B) * p.n_split * sh.H * 2 * sizeof(float));
  return p;
}

struct V4Query {
  size_t cq, cqn, q;
  size_t total() const { return cq + cqn + q; }
};
V4Query v4_query_ws(const mla_v4_dims* d, int64_t T) {
  const mla_dims sh = v4_shadow(d);
  V4Query w{};
  w.cq = proj_bytes_k(&sh, d->q_rank, d->d_model, T, lowrank_ld(d->q_rank));
  w.cqn = align_up(static_cast<size_t>(T) * d->q_rank * 2);
  w.q = proj_bytes_k(&sh, d->n_heads * d->head_dim, d->q_rank, T, static_cast<int64_t>(d->n_heads) * d->head_dim);
  return w;
}

struct V4Out {
  int splits_a;
  int64_t sps_a;
  int u_splits;   // K pieces of the W_OB product run as one batched GEMM (few output tiles)
  int64_t u_sps;
  size_t a_slices, a, u;
  size_t total() const { return a_slices + a + u; }
};
V4Out v4_out_ws(const mla_v4_dims* d, int64_t T) {
  const mla_dims sh = v4_shadow(d);
  V4Out w{};
  const int gr = d->o_groups * d->o_rank;
  w.a = align_up(static_cast<size_t>(T) * gr * 2);
  if (skinny_ok(&sh, T)) {
    const int gdim = d->n_heads * d->head_dim / d->o_groups;
    w.splits_a = mla::skinny_splits(static_cast<int>(T), d->o_rank, d->o_groups, gdim);
    w.sps_a = static_cast<int64_t>(align_up(static_cast<size_t>(T) * gr * sizeof(float)) / sizeof(float));
    w.a_slices = static_cast<size_t>(w.splits_a) * w.sps_a * sizeof(float);
  }
  // W_OB: d_model outputs over K = o_groups·o_rank.  With few 64x64 output tiles
  // the K range is cut into pieces that run as the batch index of one GEMM
  // (fp32 slices, summed after), so the grid fills the chip.
  const int64_t tiles = (T + 63) / 64 * ((d->d_model + 63) / 64);
  int sp = 1;
  while (sp < 16 && tiles * sp < 256 && gr % (2 * sp * 32) == 0) sp *= 2;
  w.u_splits = sp;
  if (sp > 1) {
    w.u_sps = static_cast<int64_t>(align_up(static_cast<size_t>(T) * d->d_model * sizeof(float)) / sizeof(float));
    w.u = static_cast<size_t>(sp) * w.u_sps * sizeof(float);
  }
  return w;
}

size_t v4_ws(const mla_v4_dims* d, int op, int32_t batch, int64_t n_tokens, int32_t max_len) {
  const mla_dims sh = v4_shadow(d);
  const int64_t T = std::max<int64_t>(n_tokens, 0);
  switch (op) {
    case MLA_V4_OP_WRITE_CACHE: return proj_bytes_k(&sh, d->head_dim, d->d_model, T, d->head_dim);
    case MLA_V4_OP_QUERY: return v4_query_ws(d, T).total();
    case MLA_V4_OP_DECODE: {
      const V4Decode p = v4_decode_plan(d, batch, max_len);
      return p.part_o + p.part_ml;
    }
    case MLA_V4_OP_PREFILL:
      return align_up(static_cast<size_t>(T) * d->n_heads * d->head_dim * 2) +
             align_up(static_cast<size_t>(T) * d->n_heads * 2 * sizeof(float));
    case MLA_V4_OP_OUTPUT: return v4_out_ws(d, T).total();
    default: return 0;
  }
}

}  // namespace

extern "C" {

int mla_v4_check_dims(const mla_v4_dims* dims) { return v4_check(dims); }

size_t mla_v4_workspace_size(const mla_v4_dims* dims, int op, int32_t batch, int64_t n_tokens,
                             int32_t max_len) {
  if (v4_check(dims) != MLA_OK) return 0;
  return v4_ws(dims, op, batch, n_tokens, max_len);
}

int mla_v4_write_cache(const mla_v4_dims* dims, const void* x, const void* w_kv, const void* kv_gain,
                       const int32_t* positions, const int64_t* slots, int64_t n_tokens, void* cache,
                       int64_t cache_rows, const double* rope_freqs, void* workspace,
                       size_t workspace_bytes, void* stream) {
  int st = v4_check(dims);
  if (st != MLA_OK) return st;
  if (n_tokens < 0 || cache_rows < 0) return MLA_EINVAL;
  if (n_tokens == 0) return MLA_OK;
  if (n_tokens > INT32_MAX) return MLA_ENOTSUP;
  if (!ptr_ok(x) || !ptr_ok(w_kv) || !ptr_ok(kv_gain) || !ptr_ok(positions) || !ptr_ok(slots) ||
      !ptr_ok(cache) || !ptr_ok(workspace) || (rope_freqs != nullptr && !ptr_ok(rope_freqs)))
    return MLA_EINVAL;
  if (workspace_bytes < v4_ws(dims, MLA_V4_OP_WRITE_CACHE, 0, n_tokens, 0)) return MLA_EWORKSPACE;
  if (mla::kDebugChecks) {
    const int dc = mla::debug_check_write(slots, n_tokens, cache_rows);
    if (dc != MLA_OK) return dc;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const mla_dims sh = v4_shadow(dims);
  float* proj = static_cast<float*>(workspace);
  const int D = dims->head_dim;
  const Proj p = proj_one(&sh, x, dims->d_model, dims->d_model, w_kv, D, proj, D, n_tokens, s);
  mla::v4_rows(dims->dtype, proj, D, p.splits, p.sps, 1, D, dims->d_rope, /*norm=*/1, kv_gain, dims->rms_eps,
               positions, slots, dims->rope_theta, rope_freqs, cache, n_tokens, s);
  return launch_status();
}

int mla_v4_query(const mla_v4_dims* dims, const void* x, const void* w_qa, const void* q_gain,
                 const void* w_qb, const int32_t* positions, int64_t n_tokens, const double* rope_freqs,
                 void* q, void* workspace, size_t workspace_bytes, void* stream) {
  int st = v4_check(dims);
  if (st != MLA_OK) return st;
  if (n_tokens < 0) return MLA_EINVAL;
  if (n_tokens == 0) return MLA_OK;
  if (n_tokens > INT32_MAX) return MLA_ENOTSUP;
  if (!ptr_ok(x) || !ptr_ok(w_qa) || !ptr_ok(q_gain) || !ptr_ok(w_qb) || !ptr_ok(positions) || !ptr_ok(q) ||
      !ptr_ok(workspace) || (rope_freqs != nullptr && !ptr_ok(rope_freqs)))
    return MLA_EINVAL;
  const V4Query w = v4_query_ws(dims, n_tokens);
  if (workspace_bytes < w.total()) return MLA_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const mla_dims sh = v4_shadow(dims);
  char* base = static_cast<char*>(workspace);
  float* cq = reinterpret_cast<float*>(base);
  void* cqn = base + w.cq;
  float* qp = reinterpret_cast<float*>(base + w.cq + w.cqn);
  const int64_t ldq = lowrank_ld(dims->q_rank);
  const Proj p1 = proj_one(&sh, x, dims->d_model, dims->d_model, w_qa, dims->q_rank, cq, ldq, n_tokens, s);
  mla::norm_rows(dims->dtype, cq, ldq, p1.splits, p1.sps, dims->q_rank, q_gain, dims->rms_eps, cqn,
                 dims->q_rank, n_tokens, s);
  const int HD = dims->n_heads * dims->head_dim;
  const Proj p2 = proj_one(&sh, cqn, dims->q_rank, dims->q_rank, w_qb, HD, qp, HD, n_tokens, s);
  mla::v4_rows(dims->dtype, qp, HD, p2.splits, p2.sps, dims->n_heads, dims->head_dim, dims->d_rope, /*norm=*/0,
               nullptr, 0.f, positions, nullptr, dims->rope_theta, rope_freqs, q, n_tokens, s);
  return launch_status();
}

int mla_v4_decode(const mla_v4_dims* dims, const void* q, const void* cache, const int64_t* seq_start,
                  const int32_t* seq_len, int32_t batch, int32_t max_len, const float* sink,
                  const double* rope_freqs, void* out, void* workspace, size_t workspace_bytes,
                  void* stream) {
  int st = v4_check(dims);
  if (st != MLA_OK) return st;
  if (batch < 0) return MLA_EINVAL;
  if (batch == 0) return MLA_OK;
  if (max_len <= 0) return MLA_EINVAL;
  if (!ptr_ok(q) || !ptr_ok(cache) || !ptr_ok(seq_start) || !ptr_ok(seq_len) || !ptr_ok(sink) || !ptr_ok(out) ||
      !ptr_ok(workspace) || (rope_freqs != nullptr && !ptr_ok(rope_freqs)))
    return MLA_EINVAL;
  const V4Decode p = v4_decode_plan(dims, batch, max_len);
  if (workspace_bytes < p.part_o + p.part_ml) return MLA_EWORKSPACE;
  if (mla::kDebugChecks) {
    const int dc = mla::debug_check_decode(seq_start, seq_len, batch, max_len);
    if (dc != MLA_OK) return dc;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const AttnShape sh = v4_shape(dims);
  char* base = static_cast<char*>(workspace);
  void* part_o = base;
  float* part_ml = reinterpret_cast<float*>(base + p.part_o);
  if (p.mfma && p.n_split == 1) {
    // one split: the kernel applies the sink and the inverse rotation itself
    const mla::V4Epilogue epi{out, sink, dims->rope_theta, rope_freqs, dims->d_rope};
    mla::decode_mfma(sh, q, nullptr, cache, seq_start, seq_len, batch, 1, p.split_len, nullptr, nullptr, nullptr,
                     s, &epi);
    return launch_status();
  }
  if (p.mfma)
    mla::decode_mfma(sh, q, nullptr, cache, seq_start, seq_len, batch, p.n_split, p.split_len, part_o, part_ml,
                     nullptr, s);
  else
    mla::attend_generic(dims->dtype, sh, q, nullptr, cache, seq_start, seq_len, nullptr, batch, batch,
                        p.n_split, p.split_len, part_o, part_ml, nullptr, s);
  mla::v4_merge(dims->dtype, part_o, part_ml, batch, p.n_split, sh.H, dims->head_dim, dims->d_rope, sink,
                seq_len, nullptr, batch, dims->rope_theta, rope_freqs, out, s);
  return launch_status();
}

int mla_v4_prefill(const mla_v4_dims* dims, const void* q, const void* cache, const int64_t* cu_seqlens,
                   int32_t batch, int64_t n_tokens, int32_t max_len, const float* sink,
                   const double* rope_freqs, void* out, void* workspace, size_t workspace_bytes,
                   void* stream) {
  int st = v4_check(dims);
  if (st != MLA_OK) return st;
  if (batch < 0 || n_tokens < 0) return MLA_EINVAL;
  if (batch == 0 || n_tokens == 0) return MLA_OK;
  if (max_len <= 0) return MLA_EINVAL;
  if (n_tokens > INT32_MAX) return MLA_ENOTSUP;
  if (!ptr_ok(q) || !ptr_ok(cache) || !ptr_ok(cu_seqlens) || !ptr_ok(sink) || !ptr_ok(out) ||
      !ptr_ok(workspace) || (rope_freqs != nullptr && !ptr_ok(rope_freqs)))
    return MLA_EINVAL;
  if (workspace_bytes < v4_ws(dims, MLA_V4_OP_PREFILL, batch, n_tokens, max_len)) return MLA_EWORKSPACE;
  if (mla::kDebugChecks) {
    const int dc = mla::debug_check_prefill(cu_seqlens, batch, n_tokens, max_len);
    if (dc != MLA_OK) return dc;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const AttnShape sh = v4_shape(dims);
  char* base = static_cast<char*>(workspace);
  void* part_o = base;
  float* part_ml = reinterpret_cast<float*>(
      base + align_up(static_cast<size_t>(n_tokens) * dims->n_heads * dims->head_dim * 2));
  if (dims->dtype == MLA_BF16 && mla::prefill_mfma_supported(sh))
    mla::prefill_mfma(sh, q, nullptr, cache, cu_seqlens, batch, n_tokens, max_len, nullptr, part_o, part_ml, s);
  else
    mla::attend_generic(dims->dtype, sh, q, nullptr, cache, nullptr, nullptr, cu_seqlens, batch, n_tokens, 1,
                        max_len, part_o, part_ml, nullptr, s);
  mla::v4_merge(dims->dtype, part_o, part_ml, n_tokens, 1, sh.H, dims->head_dim, dims->d_rope, sink, nullptr,
                cu_seqlens, batch, dims->rope_theta, rope_freqs, out, s);
  return launch_status();
}

int mla_v4_output(const mla_v4_dims* dims, const void* attn, const void* w_oa, const void* w_ob,
                  int64_t n_tokens, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  int st = v4_check(dims);
  if (st != MLA_OK) return st;
  if (n_tokens < 0) return MLA_EINVAL;
  if (n_tokens == 0) return MLA_OK;
  if (n_tokens > INT32_MAX) return MLA_ENOTSUP;
  if (!ptr_ok(attn) || !ptr_ok(w_oa) || !ptr_ok(w_ob) || !ptr_ok(out) || !ptr_ok(workspace)) return MLA_EINVAL;
  const V4Out w = v4_out_ws(dims, n_tokens);
  if (workspace_bytes < w.total()) return MLA_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int G = dims->o_groups, R = dims->o_rank, HD = dims->n_heads * dims->head_dim, gdim = HD / G;
  const int T = static_cast<int>(n_tokens);
  char* base = static_cast<char*>(workspace);
  float* a_sl = reinterpret_cast<float*>(base);
  void* a = base + w.a_slices;
  float* u_sl = reinterpret_cast<float*>(base + w.a_slices + w.a);
  if (w.a_slices > 0) {
    // few tokens: each group's W_OA block streamed once, K slices in fp32
    mla::SkinnyArgs sa{};
    sa.A = attn;
    sa.sAz = gdim;
    sa.sAm = HD;
    sa.B0 = sa.B1 = static_cast<const uint16_t*>(w_oa);
    sa.N0 = R;
    sa.sBz = static_cast<int64_t>(R) * gdim;
    sa.sBo = gdim;
    sa.C = a_sl;
    sa.sCz = R;
    sa.sCm = static_cast<int64_t>(G) * R;
    sa.sPs = w.sps_a;
    sa.M = T;
    sa.N = R;
    sa.K = gdim;
    sa.Z = G;
    sa.splits = w.splits_a;
    mla::gemm_skinny(sa, /*a_f32=*/false, /*out_bf16=*/false, s);
    mla::sum_cast_slices(dims->dtype, a_sl, w.splits_a, w.sps_a, T, G * R, static_cast<int64_t>(G) * R, a, s);
  } else {
    GemmArgs g{};
    g.A = attn;
    g.sAz = gdim;
    g.sAm = HD;
    g.B = w_oa;
    g.sBz = static_cast<int64_t>(R) * gdim;
    g.sBo = gdim;
    g.C = a;
    g.sCz = R;
    g.sCm = static_cast<int64_t>(G) * R;
    g.M = T;
    g.N = R;
    g.K = gdim;
    g.Z = G;
    mla::gemm(g, dims->dtype, false, false, /*out_bf16=*/true, s);
  }
  if (w.u_splits > 1) {
    const int kc = G * R / w.u_splits;
    GemmArgs g2{};
    g2.A = a;
    g2.sAz = kc;  // piece z reads columns [z·kc, (z+1)·kc) of a and of W_OB
    g2.sAm = static_cast<int64_t>(G) * R;
    g2.B = w_ob;
    g2.sBz = kc;
    g2.sBo = static_cast<int64_t>(G) * R;
    g2.C = u_sl;
    g2.sCz = w.u_sps;
    g2.sCm = dims->d_model;
    g2.M = T;
    g2.N = dims->d_model;
    g2.K = kc;
    g2.Z = w.u_splits;
    mla::gemm(g2, dims->dtype, false, false, /*out_bf16=*/false, s);
    mla::sum_cast_slices(dims->dtype, u_sl, w.u_splits, w.u_sps, T, dims->d_model, dims->d_model, out, s);
  } else {
    GemmArgs g2{};
    g2.A = a;
    g2.sAm = static_cast<int64_t>(G) * R;
    g2.B = w_ob;
    g2.sBo = static_cast<int64_t>(G) * R;
    g2.C = out;
    g2.sCm = dims->d_model;
    g2.M = T;
    g2.N = dims->d_model;
    g2.K = G * R;
    g2.Z = 1;
    mla::gemm(g2, dims->dtype, false, false, /*out_bf16=*/true, s);
  }
  return launch_status();
}

}  // extern "C"
