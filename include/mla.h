/*
 * mla.h — C ABI of the MLA latent-cache hot path for AMD Instinct MI355X (gfx950).
 *
 * Multi-head Latent Attention keeps one row per token in the KV cache:
 *   row = [ c (r values) ; kr_0 (d_rope) ; ... ; kr_{G-1} (d_rope) ]
 * where c = x·W_DKVᵀ is the low-rank latent and kr_g the rotary key of group g,
 * already rotated by the token's position.  Attention is computed in the
 * "absorbed" order: W_UK is folded into the query (q_lat = q_nope·W_UK), scores
 * are taken against the latent directly, P·c is formed in latent space and W_UV
 * is applied last.
 *
 * Sources (pages on MLA; equations are the pages' own numbers):
 *  - MLA principle page (dtcms.com, DeepSeek-V2 walkthrough), section on the
 *    KV down-projection and up-projection (kv_a_proj_with_mqa / kv_b_proj), the
 *    section on rotating q_pe and k_pe, and section "矩阵吸收" with the absorbed
 *    score q_pe·k_peᵀ + q_lat·cᵀ and eqs. (4)-(5) (o_ = P·c, o = o_·W_UV).
 *  - Qwen2.5-7B MLAfication page (wzjinhao.cn), section on how MLAfication
 *    rewrites attention: only the latent is cached, RoPE only on a small
 *    rotary subspace per KV head, the query split into content and rotary parts.
 *  - nanowhale-100m MLA page (cnnetsun.cn), section on attention: causal
 *    scaled-dot-product attention with an explicit scale.
 *
 * Conventions for every entry point
 *  - Pointers named "device" are device (HBM) addresses on the current HIP
 *    device; the caller allocates and owns every buffer, including workspaces.
 *    The library allocates nothing, frees nothing and never synchronises: all
 *    work is enqueued on `stream` (a hipStream_t; NULL = the default stream).
 *    (A library built with MLA_DEBUG_CHECKS synchronises to copy index arrays
 *    to the host; mla_decode_noalloc's static scratch array is the one piece of
 *    device memory the library itself holds.)
 *  - Tensors are dense row-major.  Element type of x, weights, cache, q_lat,
 *    q_pe and out is dims->dtype (MLA_F32 or MLA_BF16); positions are int32,
 *    cache slots / sequence starts are int64, lengths are int32.
 *    Base pointers must be 16-byte aligned.
 *  - Projection weights use the [out_features, in_features] layout:
 *      W_DKV [r, d_model]   W_KR [G*d_rope, d_model]
 *      W_QC  [H*d_nope, d_model]   W_QR [H*d_rope, d_model]
 *    and the up-projection is split per head: W_UK [H, d_nope, r], W_UV [H, d_v, r].
 *  - Return value: MLA_OK or a negative mla_status.  Argument errors are
 *    detected on the host before anything is enqueued, and outputs are then
 *    untouched.  Contents of device index arrays (positions, slots, lengths)
 *    are trusted: out-of-range values are undefined behaviour.
 *  - Calls on one stream are ordered; calls on different streams that share a
 *    workspace or an output race.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mla_status {
  MLA_OK = 0,
  MLA_EINVAL = -1,     /* null/misaligned pointer, bad dimension, H % G != 0, ... */
  MLA_ENOTSUP = -2,    /* a dimension combination the compiled kernels do not cover */
  MLA_EWORKSPACE = -3, /* workspace smaller than mla_workspace_size() */
  MLA_EHIP = -4,       /* the HIP runtime reported an error at launch */
  MLA_ESCRATCH = -5    /* the call needs more than the library's static scratch array */
} mla_status;

typedef enum mla_dtype { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype;

typedef enum mla_op {
  MLA_OP_WRITE_CACHE = 0,
  MLA_OP_ABSORB = 1,
  MLA_OP_DECODE = 2,
  MLA_OP_PREFILL = 3,
  MLA_OP_QUERY = 4,
  MLA_OP_PREFILL_EXPANDED = 5,
  MLA_OP_OUTPUT = 6
} mla_op;

/* Layer dimensions and hyper-parameters shared by all calls. */
typedef struct mla_dims {
  int32_t d_model;        /* hidden size of x */
  int32_t n_heads;        /* H, query heads */
  int32_t n_groups;       /* G, rotary-key groups; head h uses group h / (H/G) */
  int32_t rank;           /* r, latent width (multiple of 16, at most 512) */
  int32_t d_rope;         /* rotary dims per query head and per key group (even, at most
                             512; r + G*d_rope at most 1024 for bf16 and at most 1017
                             for fp32, whose 32-row attention tile must fit 160 KB of
                             LDS) */
  int32_t d_nope;         /* non-rotary query/key dims per head */
  int32_t d_v;            /* value dims per head */
  int32_t dtype;          /* mla_dtype */
  int32_t latent_rmsnorm; /* 1: c <- c / sqrt(mean(c^2) + rms_eps) before storage */
  float rms_eps;          /* RMSNorm epsilon (unit gain) */
  float softmax_scale;    /* applied to the whole score; <= 0 selects 1/sqrt(d_nope + d_rope) */
  double rope_theta;      /* RoPE base; pair (j, j + d_rope/2) turns by p * theta^(-2j/d_rope) */
  /* Device float64 [d_rope/2]: the inverse frequency of each rotary pair, used in
   * place of theta^(-2j/d_rope) by every call that rotates (cache write, absorb,
   * query and their low-rank forms); NULL selects theta.  A context extension
   * such as YaRN (Zebra hybrid page: factor 32 over a 32K window) changes only
   * this table; mla_rope_yarn_table() fills one.  Borrowed: it must stay valid
   * until the calls that read it have run on their stream.  Key and query rows
   * must be rotated with the same table. */
  const double* rope_freqs;
} mla_dims;

/* YaRN's rescaled inverse frequencies (Peng et al., YaRN: Efficient Context
 * Window Extension of Large Language Models, the per-pair interpolation it keeps),
 * written to host memory out[0 .. d_rope/2):
 *   f_j = theta^(-2j/d_rope); r_j = original_window * f_j / (2 pi) (turns of pair j
 *   over the pretraining window); g = clamp((r_j - alpha) / (beta - alpha), 0, 1);
 *   out[j] = (1 - g) * f_j / factor + g * f_j.
 * The paper uses alpha = 1, beta = 32.  Its attention temperature, logits times
 * (0.1 ln(factor) + 1)^2, belongs in softmax_scale.  Host only, no HIP call.
 * MLA_EINVAL for an odd or non-positive d_rope, factor or window <= 0,
 * beta <= alpha, or a null out. */
int mla_rope_yarn_table(int32_t d_rope, double theta, double factor, double original_window, double alpha,
                        double beta, double* out);

/* Range checks of the index arrays the device calls read, on HOST copies the
 * caller provides (the calls themselves never read device contents: a bad
 * length or slot is undefined behaviour there).  For debugging, and used by a
 * library built with MLA_DEBUG_CHECKS, whose decode, prefill and cache-write
 * calls copy these arrays to the host (a synchronising copy) and refuse them
 * with MLA_EINVAL before any launch.  Pass cache_rows = INT64_MAX when the
 * cache's size is not known.  Return MLA_OK or MLA_EINVAL; no HIP call.
 *   mla_check_decode_rows:  for every b: 1 <= seq_len[b] <= max_len, seq_start[b] >= 0,
 *                           seq_start[b] + seq_len[b] <= cache_rows
 *   mla_check_prefill_rows: cu_seqlens[0] = 0, non-decreasing, cu_seqlens[batch] = n_tokens,
 *                           every segment at most max_len rows, n_tokens <= cache_rows
 *   mla_check_write_rows:   every slot in [0, cache_rows), no slot twice */
int mla_check_decode_rows(const int64_t* seq_start, const int32_t* seq_len, int32_t batch, int32_t max_len,
                          int64_t cache_rows);
int mla_check_prefill_rows(const int64_t* cu_seqlens, int32_t batch, int64_t n_tokens, int32_t max_len,
                           int64_t cache_rows);
int mla_check_write_rows(const int64_t* slots, int64_t n_tokens, int64_t cache_rows);

/* Bytes of scratch an operation needs for the given sizes (0 if none).
 * op: mla_op.  batch: sequences (decode/prefill).  n_tokens: tokens in the call.
 * max_len: the largest per-sequence context in the call (decode/prefill).
 * Returns 0 also for invalid dims; mla_check_dims() tells them apart. */
size_t mla_workspace_size(const mla_dims* dims, int op, int32_t batch, int64_t n_tokens,
                          int32_t max_len);

/* Validate dims on the host only (no HIP call).  MLA_OK, MLA_EINVAL or MLA_ENOTSUP. */
int mla_check_dims(const mla_dims* dims);

/* Cache write (latent down-projection + partial RoPE key), for n_tokens tokens.
 *   cache[slots[t], 0:r]                = c[t] = x[t]·W_DKVᵀ   (RMSNorm'd if latent_rmsnorm)
 *   cache[slots[t], r+g*d_rope : +d_rope] = RoPE(x[t]·W_KR[g*d_rope : +d_rope]ᵀ, positions[t])
 * Source: MLA principle page, KV down-projection section (kv_a_proj_with_mqa) and
 * the q_pe/k_pe rotation section; MLAfication page, "X → down_kv → c_kv, only it is
 * cached"; Qwen3-30B delta page, variant "disrms" (read as RMSNorm on c).
 *   x         device [n_tokens, d_model]
 *   w_dkv     device [r, d_model];  w_kr device [G*d_rope, d_model]
 *   positions device int32 [n_tokens] (>= 0)
 *   slots     device int64 [n_tokens], each in [0, cache_rows); distinct
 *   cache     device [cache_rows, r + G*d_rope] (written rows only)
 *   workspace device, >= mla_workspace_size(dims, MLA_OP_WRITE_CACHE, 0, n_tokens, 0) bytes
 * n_tokens == 0 is a no-op. */
int mla_write_cache(const mla_dims* dims, const void* x, const void* w_dkv, const void* w_kr,
                    const int32_t* positions, const int64_t* slots, int64_t n_tokens,
                    void* cache, int64_t cache_rows, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Query side with W_UK absorption, for n_tokens query tokens.
 *   q_nope[t,h] = x[t]·W_QC[h*d_nope : +d_nope]ᵀ
 *   q_pe[t,h]   = RoPE(x[t]·W_QR[h*d_rope : +d_rope]ᵀ, positions[t])
 *   q_lat[t,h,:] = Σ_d q_nope[t,h,d]·W_UK[h,d,:]
 * Source: MLA principle page, split of q into q_nope/q_pe and section "矩阵吸收"
 * (einsum 'hdc,bhqd->bhqc' of W_UK with q_nope); MLAfication page, q_c_proj / q_r_proj.
 *   x device [n_tokens, d_model]; w_qc device [H*d_nope, d_model];
 *   w_qr device [H*d_rope, d_model]; w_uk device [H, d_nope, r]
 *   positions device int32 [n_tokens]
 *   q_lat device out [n_tokens, H, r];  q_pe device out [n_tokens, H, d_rope]
 *   workspace device, >= mla_workspace_size(dims, MLA_OP_ABSORB, 0, n_tokens, 0) bytes */
int mla_absorb(const mla_dims* dims, const void* x, const void* w_qc, const void* w_qr,
               const void* w_uk, const int32_t* positions, int64_t n_tokens, void* q_lat,
               void* q_pe, void* workspace, size_t workspace_bytes, void* stream);

/* Batched decode: one query token per sequence, attending to all of its cached rows.
 * For sequence b with n = seq_len[b] >= 1 rows starting at cache row seq_start[b]
 * (the query's own row, at position n-1, is the last one):
 *   s[h,l] = scale·(q_lat[b,h]·c[l] + q_pe[b,h]·kr[l, g(h)])
 *   P = softmax_l(s);  o_[h,:] = Σ_l P[h,l]·c[l,:];  out[b,h,:] = W_UV[h]·o_[h,:]
 * Source: MLA principle page, section "矩阵吸收" (absorbed score on compressed_kv,
 * softmax_scale on the sum) and eqs. (4)-(5) (P·c first, then W_UV).
 *   q_lat device [batch, H, r]; q_pe device [batch, H, d_rope]
 *   cache device [*, r + G*d_rope]; seq_start device int64 [batch]; seq_len device int32 [batch]
 *   max_len: host upper bound on seq_len (sizes the split of each context)
 *   w_uv device [H, d_v, r];  out device out [batch, H, d_v]
 *   workspace device, >= mla_workspace_size(dims, MLA_OP_DECODE, batch, 0, max_len) bytes
 * batch == 0 is a no-op; seq_len[b] must be in [1, max_len]. */
int mla_decode(const mla_dims* dims, const void* q_lat, const void* q_pe, const void* cache,
               const int64_t* seq_start, const int32_t* seq_len, int32_t batch, int32_t max_len,
               const void* w_uv, void* out, void* workspace, size_t workspace_bytes,
               void* stream);

/* mla_decode without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The split partials live in a static device array of
 * MLA_NOALLOC_SCRATCH_BYTES inside the library; every GPU the library runs on
 * holds its own copy from the first call on that device until the process ends.
 * The call allocates nothing.  Arguments and results are those of mla_decode;
 * the current device must be the stream's device.
 *   MLA_ESCRATCH (before any HIP call) when mla_workspace_size(dims,
 *   MLA_OP_DECODE, batch, 0, max_len) exceeds MLA_NOALLOC_SCRATCH_BYTES
 *   (64 MiB covers 64 sequences of 8192 rows at H = 128, r = 512);
 *   MLA_EHIP if the array's device address cannot be taken.
 * Every call on a GPU uses that GPU's one array, and the array keeps the last
 * call's contents: calls that overlap on one GPU (two streams, two threads)
 * race.  Serialise them. */
#define MLA_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
int mla_decode_noalloc(const mla_dims* dims, const void* q_lat, const void* q_pe, const void* cache,
                       const int64_t* seq_start, const int32_t* seq_len, int32_t batch, int32_t max_len,
                       const void* w_uv, void* out, void* stream);

/* The split plan made from the batch and the longest length: the number of
 * context splits per sequence (>= 1), or a negative mla_status.  Split j of a
 * sequence covers its rows [j*L, min(n, (j+1)*L)) with
 * L = mla_decode_split_rows(dims, batch, max_len); trailing splits may be empty.
 * mla_decode uses this plan, except where the MFMA kernel takes whole splits of
 * at most 64 sequences and this plan has more splits than the merge folded into
 * W_UV takes: there the kernel re-plans on the device from the actual lengths
 * (equal-sized splits spread over the same number of workgroups), so a ragged
 * batch does not leave most of the shorter sequences' workgroups empty.  The
 * workspace mla_workspace_size reports covers either plan. */
int32_t mla_decode_splits(const mla_dims* dims, int32_t batch, int32_t max_len);
int32_t mla_decode_split_rows(const mla_dims* dims, int32_t batch, int32_t max_len);

/* The attention of mla_decode without its merge and W_UV: per (sequence, split,
 * head) the softmax state of the split's rows, for callers that combine partial
 * results themselves (one sequence's rows spread over several devices, or a
 * projection fused downstream).  With s_l the score of row l (as in mla_decode)
 * and u_l = s_l·log2(e):
 *   part_ml[b,j,h] = (m, l = Σ_l 2^(u_l - m))   m: a per-split reference, base 2
 *   part_o[b,j,h,:] = Σ_l 2^(u_l - m)·c[l,:] / l  (the split's own o_)
 * so o_ = Σ_j 2^(m_j - M)·l_j·part_o_j / Σ_j 2^(m_j - M)·l_j for any M.  An empty
 * split gives m = -inf, l = 0, part_o = 0.  m need not be the true max: the
 * kernels may use any reference that keeps 2^(u_l - m) finite.
 * Source: split softmax merge of the MLA principle page's attention (eq. (4)
 * computed per split of the context), the exchange a multi-device split needs.
 *   q_lat, q_pe, cache, seq_start, seq_len, max_len: as mla_decode
 *   n_split: >= 1; splits of L = ceil(max_len / n_split) rounded up to 64 rows
 *   part_o device out [batch, n_split, H, r] in the layer's element type (dims->dtype)
 *   part_ml device fp32 out [batch, n_split, H, 2]
 * Needs no workspace; batch == 0 is a no-op. */
int mla_decode_partials(const mla_dims* dims, const void* q_lat, const void* q_pe,
                        const void* cache, const int64_t* seq_start, const int32_t* seq_len,
                        int32_t batch, int32_t max_len, int32_t n_split, void* part_o,
                        float* part_ml, void* stream);

/* Causal prefill over packed sequences.  Tokens cu_seqlens[b] .. cu_seqlens[b+1]-1
 * form sequence b at positions 0..n_b-1; token t's own cache row is row t, and it
 * attends to rows cu_seqlens[b] .. t (same formula as mla_decode per token).
 * Source: as mla_decode, plus the causal SDPA of the nanowhale MLA page.
 *   q_lat device [n_tokens, H, r]; q_pe device [n_tokens, H, d_rope]
 *   cache device [>= n_tokens, r + G*d_rope]
 *   cu_seqlens device int64 [batch+1], cu_seqlens[0] = 0, cu_seqlens[batch] = n_tokens
 *   max_len: host upper bound on n_b
 *   w_uv device [H, d_v, r];  out device out [n_tokens, H, d_v]
 *   workspace device, >= mla_workspace_size(dims, MLA_OP_PREFILL, batch, n_tokens, max_len) */
int mla_prefill(const mla_dims* dims, const void* q_lat, const void* q_pe, const void* cache,
                const int64_t* cu_seqlens, int32_t batch, int64_t n_tokens, int32_t max_len,
                const void* w_uv, void* out, void* workspace, size_t workspace_bytes,
                void* stream);

/* Query side without absorption (the input of the original-order prefill).
 *   q_nope[t,h] = x[t]·W_QC[h*d_nope : +d_nope]ᵀ
 *   q_pe[t,h]   = RoPE(x[t]·W_QR[h*d_rope : +d_rope]ᵀ, positions[t])
 * Source: MLA principle page, split of the query into q_nope / q_pe and the
 * rotation of q_pe; MLAfication page, q_c_proj / q_r_proj.
 *   x device [n_tokens, d_model]; w_qc device [H*d_nope, d_model];
 *   w_qr device [H*d_rope, d_model]; positions device int32 [n_tokens]
 *   q_nope device out [n_tokens, H, d_nope]; q_pe device out [n_tokens, H, d_rope]
 *   workspace device, >= mla_workspace_size(dims, MLA_OP_QUERY, 0, n_tokens, 0) bytes
 * n_tokens == 0 is a no-op. */
int mla_query(const mla_dims* dims, const void* x, const void* w_qc, const void* w_qr,
              const int32_t* positions, int64_t n_tokens, void* q_nope, void* q_pe, void* workspace,
              size_t workspace_bytes, void* stream);

/* Causal prefill in the original (non-absorbed) order, same sequences and
 * result as mla_prefill.  The cached latents are first up-projected per head,
 *   k_nope[h,l] = W_UK[h]·c[l],   v[h,l] = W_UV[h]·c[l],
 * and token t then attends to rows cu_seqlens[b] .. t with
 *   s[h,l] = scale·(q_nope[t,h]·k_nope[h,l] + q_pe[t,h]·kr[l, g(h)])
 *   out[t,h,:] = Σ_l softmax_l(s)[h,l]·v[h,l]
 * For a long prompt this order costs 2(d_nope + d_rope) + 2 d_v flops per
 * (query, key, head) against 2(r + d_rope) + 2r for the absorbed one.
 * Source: MLA principle page, section "原始顺序" eqs. (1)-(2) (v = W_UV·c, then
 * o = P·v) and the up-projection kv_b_proj split into W_UK / W_UV; causal SDPA
 * of the nanowhale MLA page.
 *   q_nope device [n_tokens, H, d_nope]; q_pe device [n_tokens, H, d_rope] (mla_query)
 *   cache, cu_seqlens, batch, n_tokens, max_len: as mla_prefill
 *   w_uk device [H, d_nope, r]; w_uv device [H, d_v, r]; out device out [n_tokens, H, d_v]
 *   workspace device, >= mla_workspace_size(dims, MLA_OP_PREFILL_EXPANDED, batch, n_tokens,
 *   max_len) bytes.  After the call it holds the expanded keys and values in fp16
 *   (11 significant bits, where bf16 would push the result past 1e-2):
 *   k_nope [H, n_tokens, d_nope] from byte 0, then, from the next multiple of 256
 *   bytes, vᵀ [H, d_v, T_pad] with T_pad = n_tokens rounded up to 32 and the pad
 *   columns zero: 2·H·(n_tokens·d_nope + d_v·T_pad) bytes plus alignment.
 *   Range: fp16 holds |k_nope|, |v| and |q_nope| up to 65504.  Nothing checks
 *   this; larger values become inf and the output is then not finite.
 * Compiled for bf16 with d_nope = d_v = 128 and d_rope = 64; other layers get
 * MLA_ENOTSUP (mla_prefill covers them).  batch == 0 or n_tokens == 0 is a no-op. */
int mla_prefill_expanded(const mla_dims* dims, const void* q_nope, const void* q_pe, const void* cache,
                         const int64_t* cu_seqlens, int32_t batch, int64_t n_tokens, int32_t max_len,
                         const void* w_uk, const void* w_uv, void* out, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Low-rank query path (DeepSeek-V2's query factorisation), with or without the
 * W_UK absorption:
 *   c_q        = RMSNorm(x[t]·W_QAᵀ) * q_gain      (eps = dims->rms_eps; over q_rank values)
 *   q[t,h,:]   = c_q·W_QB[h*(d_nope+d_rope) : +(d_nope+d_rope)]ᵀ = [q_nope ; q_pe_raw]
 *   q_pe[t,h]  = RoPE(q_pe_raw, positions[t])
 *   q_lat[t,h,:] = Σ_d q_nope[t,h,d]·W_UK[h,d,:]    (mla_absorb_lowrank)
 * c_q is rounded to the layer's element type between the two projections.
 * Source: MLA principle page, section "步骤": q = q_b_proj(q_a_layernorm(q_a_proj(x)))
 * (5120 -> 1536 -> 24576 = 128 heads x 192), viewed per head and split into q_nope /
 * q_pe; the nanowhale MLA page's wq_a / q_norm / wq_b.
 *   q_rank: width of the middle (multiple of 8, at most 4096)
 *   x device [n_tokens, d_model]; w_qa device [q_rank, d_model]
 *   q_gain device [q_rank] or NULL (unit gain); w_qb device [H*(d_nope+d_rope), q_rank],
 *     rows head-major with each head's d_nope rows before its d_rope rows
 *   w_uk device [H, d_nope, r]; positions device int32 [n_tokens]
 *   q_lat device out [n_tokens, H, r] or q_nope device out [n_tokens, H, d_nope];
 *   q_pe device out [n_tokens, H, d_rope]
 *   workspace device, >= mla_lowrank_workspace_size(dims, q_rank, n_tokens) bytes
 * n_tokens == 0 is a no-op. */
size_t mla_lowrank_workspace_size(const mla_dims* dims, int32_t q_rank, int64_t n_tokens);
int mla_absorb_lowrank(const mla_dims* dims, int32_t q_rank, const void* x, const void* w_qa,
                       const void* q_gain, const void* w_qb, const void* w_uk, const int32_t* positions,
                       int64_t n_tokens, void* q_lat, void* q_pe, void* workspace, size_t workspace_bytes,
                       void* stream);
int mla_query_lowrank(const mla_dims* dims, int32_t q_rank, const void* x, const void* w_qa,
                      const void* q_gain, const void* w_qb, const int32_t* positions, int64_t n_tokens,
                      void* q_nope, void* q_pe, void* workspace, size_t workspace_bytes, void* stream);

/* Output projection after W_UV:  u[t,:] = Σ_h Σ_e attn[t,h,e]·W_o[:, h*d_v + e].
 * Source: MLA principle page, eqs. (3)/(6) (einsum 'hdD,bhqd->bqD' of W_o with the
 * per-head outputs) and o_proj of size [num_heads * v_head_dim -> hidden].
 *   attn device [n_tokens, H, d_v] (the output of mla_decode / mla_prefill)
 *   w_o device [d_model, H*d_v];  out device out [n_tokens, d_model]
 *   workspace device, >= mla_workspace_size(dims, MLA_OP_OUTPUT, 0, n_tokens, 0) bytes
 *   (0 for many tokens: then workspace may be NULL)
 * n_tokens == 0 is a no-op. */
int mla_output(const mla_dims* dims, const void* attn, const void* w_o, int64_t n_tokens, void* out,
               void* workspace, size_t workspace_bytes, void* stream);

/* Tiled weights for few-token steps.  With n_tokens <= 64 a projection is a
 * stream of its whole weight.  Read in place, 96 rows at a time, the weight
 * arrives as 256-byte runs of 96 rows that lie 2*in_features bytes apart, which
 * leaves HBM pages mostly unused.  mla_tile_weights re-lays a weight [W0 ; W1]
 * once (at load time) so that each block of 96 rows x 128 input features is one
 * contiguous 24 KB piece: block t*ceil(k/128) + j holds rows [96t, 96t + 96) and
 * features [128j, 128j + 128), row after row, with the 16-byte chunks of block
 * row i in the order (chunk ^ (i & 15)); rows past n0 + n1 and features past k
 * are zero.  Only the *_tiled calls read the result.
 *   w0 device bf16 [n0, k]; w1 device bf16 [n1, k] (may be NULL when n1 == 0)
 *   out device, >= mla_tiled_weight_bytes(n0 + n1, k) bytes
 *   k: multiple of 8.  Sizes or pointers out of range return MLA_EINVAL.
 * mla_absorb_tiled and mla_output_tiled compute what mla_absorb and mla_output
 * compute, from
 *   w_q_tiled = [W_QC ; W_QR] tiled: mla_tile_weights(w_qc, H*d_nope, w_qr, H*d_rope, d_model, ...)
 *   w_o_tiled = W_o tiled:           mla_tile_weights(w_o, d_model, NULL, 0, H*d_v, ...)
 * with the workspace of MLA_OP_ABSORB / MLA_OP_OUTPUT, for dims->dtype == MLA_BF16
 * and 1 <= n_tokens <= 64 (MLA_ENOTSUP otherwise; n_tokens == 0 is a no-op).
 * Where mla_absorb / mla_output stream the weight with the same kernel (96
 * output columns per workgroup, as at H = 128 and d_model = 5120) the results
 * are bit-identical; elsewhere they agree to rounding.
 * Source: the passages cited at mla_absorb and mla_output; the layout is a
 * storage choice of this library. */
size_t mla_tiled_weight_bytes(int64_t n_rows, int64_t k);
int mla_tile_weights(const void* w0, int64_t n0, const void* w1, int64_t n1, int64_t k, void* out,
                     size_t out_bytes, void* stream);
int mla_absorb_tiled(const mla_dims* dims, const void* x, const void* w_q_tiled, const void* w_uk,
                     const int32_t* positions, int64_t n_tokens, void* q_lat, void* q_pe, void* workspace,
                     size_t workspace_bytes, void* stream);
int mla_output_tiled(const mla_dims* dims, const void* attn, const void* w_o_tiled, int64_t n_tokens,
                     void* out, void* workspace, size_t workspace_bytes, void* stream);
/* mla_absorb_lowrank with both low-rank weights tiled:
 *   w_qa_tiled = mla_tile_weights(w_qa, q_rank, NULL, 0, d_model, ...)
 *   w_qb_tiled = mla_tile_weights(w_qb, H*(d_nope+d_rope), NULL, 0, q_rank, ...)
 * workspace as mla_absorb_lowrank (mla_lowrank_workspace_size); bf16, 1 <= n_tokens <= 64
 * (MLA_ENOTSUP otherwise; n_tokens == 0 is a no-op). */
int mla_absorb_lowrank_tiled(const mla_dims* dims, int32_t q_rank, const void* x, const void* w_qa_tiled,
                             const void* q_gain, const void* w_qb_tiled, const void* w_uk,
                             const int32_t* positions, int64_t n_tokens, void* q_lat, void* q_pe,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------
 * DeepSeek-V4 / nanowhale variant (nanowhale MLA page).  One KV head of head_dim
 * values, kv = kv_norm(x·W_KVᵀ) (RMSNorm with gain), its last d_rope dims rotated
 * in the page's complex form (apply_rotary_emb: pairs (2i, 2i+1) turned by
 * p·f_i, f_i = theta^(-2i/d_rope) or a caller's table), is cached per token and
 * used by every query head as both key and value:
 *   q[t,h]   = (RMSNorm(x[t]·W_QAᵀ)·q_gain)·W_QB[h*D : +D]ᵀ, last d_rope dims rotated
 *   s[h,l]   = scale·q[t,h]·kv[l]                  (scale <= 0: 1/sqrt(head_dim))
 *   o[t,h,:] = Σ_l e^(s_l) kv[l] / (Σ_l e^(s_l) + e^(sink[h])),
 *              then its last d_rope dims rotated back by the query's position
 *   u[t]     = W_OB · concat_g(W_OA[g]·o_g[t])      (o_g: group g of the H·D outputs)
 * Sources: nanowhale MLA page, sections on the single KV head (wkv, kv_norm), the
 * low-rank query (wq_a, q_norm, wq_b), the partial RoPE with rotation before and
 * after attention, the SDPA over kv for keys and values with attn_sink, and the
 * grouped low-rank output (wo_a, wo_b).
 * rope_freqs: device float64 [d_rope/2] inverse frequencies, or NULL for
 * theta^(-2i/d_rope); a context-extension rescaling passes its own table.
 * Compiled for bf16 with head_dim <= 512 (multiple of 16).  head_dim 512 runs
 * on MFMA kernels: decode with up to 16 heads, prefill with a head count that
 * divides 16; other shapes run the generic kernel.
 * ------------------------------------------------------------------------------ */
typedef struct mla_v4_dims {
  int32_t d_model;      /* hidden size */
  int32_t n_heads;      /* H query heads, all reading the one KV head */
  int32_t head_dim;     /* D: KV row width and per-head query width */
  int32_t d_rope;       /* rotary dims at the end of the row (even, <= D) */
  int32_t q_rank;       /* low-rank query width (multiple of 8, <= 4096) */
  int32_t o_groups;     /* output groups; (H*D) % o_groups == 0 */
  int32_t o_rank;       /* per-group output rank */
  int32_t dtype;        /* MLA_BF16 */
  float rms_eps;        /* eps of kv_norm and q_norm */
  float softmax_scale;  /* <= 0: 1/sqrt(head_dim) */
  double rope_theta;
} mla_v4_dims;

typedef enum mla_v4_op {
  MLA_V4_OP_WRITE_CACHE = 0,
  MLA_V4_OP_QUERY = 1,
  MLA_V4_OP_DECODE = 2,
  MLA_V4_OP_PREFILL = 3,
  MLA_V4_OP_OUTPUT = 4
} mla_v4_op;

int mla_v4_check_dims(const mla_v4_dims* dims);
size_t mla_v4_workspace_size(const mla_v4_dims* dims, int op, int32_t batch, int64_t n_tokens,
                             int32_t max_len);

/* cache[slots[t], :] = rotated kv_norm(x[t]·W_KVᵀ)·kv_gain.
 *   x device [n_tokens, d_model]; w_kv device [D, d_model]; kv_gain device [D]
 *   positions device int32 [n_tokens]; slots device int64 [n_tokens], distinct, < cache_rows
 *   cache device [cache_rows, D] */
int mla_v4_write_cache(const mla_v4_dims* dims, const void* x, const void* w_kv, const void* kv_gain,
                       const int32_t* positions, const int64_t* slots, int64_t n_tokens, void* cache,
                       int64_t cache_rows, const double* rope_freqs, void* workspace,
                       size_t workspace_bytes, void* stream);

/* q[t,h,:] as above.  w_qa device [q_rank, d_model]; q_gain device [q_rank];
 * w_qb device [H*D, q_rank]; q device out [n_tokens, H, D]. */
int mla_v4_query(const mla_v4_dims* dims, const void* x, const void* w_qa, const void* q_gain,
                 const void* w_qb, const int32_t* positions, int64_t n_tokens, const double* rope_freqs,
                 void* q, void* workspace, size_t workspace_bytes, void* stream);

/* Decode: one query per sequence (at position seq_len[b]-1, its own row already
 * cached) over rows seq_start[b] .. seq_start[b]+seq_len[b]-1.
 *   q device [batch, H, D]; sink device fp32 [H]; out device out [batch, H, D] */
int mla_v4_decode(const mla_v4_dims* dims, const void* q, const void* cache, const int64_t* seq_start,
                  const int32_t* seq_len, int32_t batch, int32_t max_len, const float* sink,
                  const double* rope_freqs, void* out, void* workspace, size_t workspace_bytes,
                  void* stream);

/* Causal prefill over packed sequences (as mla_prefill: token t's row is cache row t,
 * it attends rows cu_seqlens[b] .. t, its position is t - cu_seqlens[b]).
 *   q device [n_tokens, H, D]; out device out [n_tokens, H, D] */
int mla_v4_prefill(const mla_v4_dims* dims, const void* q, const void* cache, const int64_t* cu_seqlens,
                   int32_t batch, int64_t n_tokens, int32_t max_len, const float* sink,
                   const double* rope_freqs, void* out, void* workspace, size_t workspace_bytes,
                   void* stream);

/* u = grouped low-rank output projection of attn [n_tokens, H, D].
 *   w_oa device [o_groups*o_rank, H*D/o_groups] (group g: rows g*o_rank ..)
 *   w_ob device [d_model, o_groups*o_rank]; out device out [n_tokens, d_model]
 * The o_groups*o_rank intermediate is rounded to the layer's element type. */
int mla_v4_output(const mla_v4_dims* dims, const void* attn, const void* w_oa, const void* w_ob,
                  int64_t n_tokens, void* out, void* workspace, size_t workspace_bytes, void* stream);

/* Human-readable text for a status code (static storage). */
const char* mla_strerror(int status);

/* Library ABI version (major * 100 + minor). */
int mla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
