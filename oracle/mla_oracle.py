"""Plain float64 CPU oracle for MLA over a latent KV cache (non-absorbed form).

TEST INFRASTRUCTURE ONLY. Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module. The product path (the HIP
library and its Python binding) never calls it, and it shares no code with it.

What it computes, step by step, and the passage each step follows.  Pages are
named by their title / subject; equation numbers are the pages' own.

* Page "MLA 原理 / 关于矩阵吸收十倍提速" (dtcms.com, the DeepSeek-V2 MLA walkthrough):
  - §"对KV张量的降维、分裂K、拆分KV且升维": the latent c = x·W_DKV is what the
    cache holds (kv_a_proj_with_mqa, the report's eq. (41)); the up-projection
    kv_b_proj (eq. (42)) is viewed as [H, d_nope + d_v, r] and split into
    W_UK = [:, :d_nope, :] and W_UV = [:, d_nope:, :].
  - §"将查询和键张量 q_pe 和 k_pe 进行旋转": only q_pe / k_pe are rotated
    (apply_rotary_pos_emb with cos/sin and position ids); the query is
    [q_nope ; q_pe] with the no-position part first.
  - §"升维之后计算注意力": after the up-projection, standard attention.
  - "原始顺序" eq. (1)-(2): v = einsum('hdc,blc->blhd', W_UV, c),
    o = attn_weights · v.  This oracle follows that original order: it EXPANDS
    k_nope = W_UK·c and v = W_UV·c for every cached row, and never uses the
    absorbed rewrite except in ``absorbed_query`` (the per-token W_UK absorption
    the page writes as einsum('hdc,bhqd->bhqc'), kept to localise errors in a GPU
    intermediate, never used to produce the attention output).
* Page "Qwen2.5-7B-base-mla-topk8-rank128 MLAfication" (wzjinhao.cn),
  §"MLAfication 如何改写注意力结构": X → down_kv → c_kv (the only thing cached);
  c_kv → up_kc / up_v; RoPE only on a small rotary subspace per KV head
  (k_r_proj, q_r_proj); the query is split into a content part (q_c_proj) and a
  rotary part (q_r_proj).  With several KV groups, each query head uses its
  group's rotary key.
* Page "Qwen3-30B-A3B-base-mla-topk8-rank512" (kwkr.cn): config field
  ``variant: disrms``; read here as RMSNorm over the latent before it is stored
  (unit gain), matching the nanowhale page's kv_norm (DeepseekV4RMSNorm on the
  KV projection).
* Page "MLA 在 nanowhale-100m 中的实现原理", §"高效注意力计算实现": causal
  scaled-dot-product attention with an explicit scale (SDPA with is_causal).
* Beyond the attention itself (``lowrank_query``, ``output_projection``): the
  MLA principle page's low-rank query q_b_proj(q_a_layernorm(q_a_proj(x))) of its
  §"步骤", and its output projection o_proj, eqs. (3)/(6).
* Page "zebra_qwen3_7MLA21GDN": the context window extended 32 times with YaRN
  (factor 32.0 over a 32K pretraining window); YaRN changes only the rotary
  frequencies (``yarn_inv_freq``, from the YaRN paper), which every rotating
  function here accepts as ``inv_freq``.
* The nanowhale page's DeepSeek-V4 variant (``v4_*``): one normalised KV head
  used as both key and value, the complex-form RoPE on its last dims with the
  inverse rotation of the output, an attention sink, and the grouped low-rank
  output projection.

Readings taken where the pages are silent (each is listed in the design doc):
rotate-half RoPE pairing (j, j + d_r/2) with θ_j = θ^(-2j/d_r) and the angle
p·θ_j formed in float64; softmax over keys after the causal mask; causal rule
p[key] <= p[query] within one sequence; head h uses rotary-key group
h // (H/G); no biases; unit-gain RMSNorm with eps inside the square root.

Parity pins: see tests/test_oracle_pins.py (brute force, associativity, torch
SDPA in float64, RoPE invariants, closed forms, consistency, page facts).
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=F64)


# ----------------------------------------------------------------------------
# rotary embedding on the rotary sub-dims only
# ----------------------------------------------------------------------------


def rope_angles(pos, d_rope: int, theta: float, inv_freq=None) -> np.ndarray:
    """Angles p·θ_j, θ_j = θ^(-2j/d_rope), j < d_rope/2, in float64; shape [..., d_rope/2].
    ``inv_freq`` [d_rope/2], when given, replaces θ_j (a rescaled table such as YaRN's)."""
    if d_rope % 2:
        raise ValueError("rotary width must be even")
    half = d_rope // 2
    if inv_freq is None:
        j = np.arange(half, dtype=F64)
        inv_freq = float(theta) ** (-2.0 * j / d_rope)
    inv_freq = _f64(inv_freq)
    if inv_freq.shape != (half,):
        raise ValueError("inverse-frequency table must hold d_rope/2 values")
    return _f64(pos)[..., None] * inv_freq


def yarn_inv_freq(d_rope: int, theta: float, factor: float, original_window: float,
                  alpha: float = 1.0, beta: float = 32.0) -> np.ndarray:
    """YaRN's rescaled inverse frequencies (Peng et al., "YaRN: Efficient Context
    Window Extension of Large Language Models", the "NTK-by-parts" interpolation
    that YaRN keeps).  Pair j turns at θ_j = θ^(-2j/d_rope), i.e. with wavelength
    λ_j = 2π/θ_j; r_j = original_window/λ_j counts its turns over the pretraining
    window.  A ramp γ(r) is 0 below α, 1 above β and linear between; the new
    frequency is (1 − γ)·θ_j/factor + γ·θ_j: slow pairs are interpolated by the
    factor, fast pairs keep their frequency.  The Zebra hybrid page extends a
    32K window 32 times this way; α = 1 and β = 32 are the paper's values."""
    if d_rope % 2 or factor <= 0 or original_window <= 0 or not beta > alpha:
        raise ValueError("bad YaRN parameters")
    j = np.arange(d_rope // 2, dtype=F64)
    base = float(theta) ** (-2.0 * j / d_rope)
    r = float(original_window) * base / (2.0 * np.pi)
    gamma = np.clip((r - alpha) / (beta - alpha), 0.0, 1.0)
    return (1.0 - gamma) * base / float(factor) + gamma * base


def yarn_logit_scale(factor: float) -> float:
    """YaRN's attention temperature: logits are multiplied by (0.1·ln(factor) + 1)²
    (the paper applies √(1/t) = 0.1·ln s + 1 to both q and k); a caller folds it
    into the softmax scale."""
    m = 0.1 * np.log(float(factor)) + 1.0 if factor > 1 else 1.0
    return float(m * m)


def rope(y, pos, theta: float, inv_freq=None) -> np.ndarray:
    """Rotate-half RoPE of the last axis of ``y`` (width d_r) by position ``pos``.

    Dims j and j + d_r/2 form a pair rotated by angle p·θ_j:
      y'[j]        = y[j]·cos − y[j+half]·sin
      y'[j+half]   = y[j+half]·cos + y[j]·sin
    ``pos`` broadcasts against y's leading axes.  ``inv_freq`` replaces θ_j.
    """
    y = _f64(y)
    d = y.shape[-1]
    half = d // 2
    ang = rope_angles(pos, d, theta, inv_freq)
    # broadcast angles over any middle axes (e.g. heads) of y
    while ang.ndim < y.ndim:
        ang = np.expand_dims(ang, axis=-2)
    cos, sin = np.cos(ang), np.sin(ang)
    a, b = y[..., :half], y[..., half:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=-1)


# ----------------------------------------------------------------------------
# cache side: latent + rotary key
# ----------------------------------------------------------------------------


def rmsnorm(v, eps: float) -> np.ndarray:
    """Unit-gain RMSNorm over the last axis: v / sqrt(mean(v^2) + eps)."""
    v = _f64(v)
    return v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)


def latent(x, w_dkv, latent_rmsnorm: bool = False, eps: float = 1e-6) -> np.ndarray:
    """c = x · W_DKVᵀ  (W_DKV stored [r, d_model]); optional RMSNorm. Shape [T, r]."""
    c = _f64(x) @ _f64(w_dkv).T
    return rmsnorm(c, eps) if latent_rmsnorm else c


def rotary_key(x, w_kr, pos, n_groups: int, d_rope: int, theta: float, inv_freq=None) -> np.ndarray:
    """kr[t, g] = RoPE(x[t] · W_KR[g·d_r:(g+1)·d_r]ᵀ, p[t]). Shape [T, G, d_r]."""
    raw = (_f64(x) @ _f64(w_kr).T).reshape(-1, n_groups, d_rope)
    return rope(raw, pos, theta, inv_freq)


def cache_rows(x, w_dkv, w_kr, pos, *, n_groups, d_rope, theta, latent_rmsnorm=False,
               eps=1e-6, inv_freq=None) -> np.ndarray:
    """One cache row per token: [c (r) ; kr_0 ; ... ; kr_{G-1}] (width r + G·d_r)."""
    c = latent(x, w_dkv, latent_rmsnorm, eps)
    kr = rotary_key(x, w_kr, pos, n_groups, d_rope, theta, inv_freq)
    return np.concatenate([c, kr.reshape(kr.shape[0], -1)], axis=1)


def split_rows(rows, rank: int, n_groups: int, d_rope: int):
    """Split cache rows into (c [S, r], kr [S, G, d_r])."""
    rows = _f64(rows)
    return rows[:, :rank], rows[:, rank:rank + n_groups * d_rope].reshape(-1, n_groups, d_rope)


# ----------------------------------------------------------------------------
# query side
# ----------------------------------------------------------------------------


def query(x, w_qc, w_qr, pos, *, n_heads, d_nope, d_rope, theta, inv_freq=None):
    """qn[t,h] = x[t]·W_QC[h·d_nope:(h+1)·d_nope]ᵀ; qr[t,h] = RoPE(x[t]·W_QR[h·d_r:…]ᵀ, p[t])."""
    x = _f64(x)
    qn = (x @ _f64(w_qc).T).reshape(-1, n_heads, d_nope)
    qr = rope((x @ _f64(w_qr).T).reshape(-1, n_heads, d_rope), pos, theta, inv_freq)
    return qn, qr


def absorbed_query(qn, w_uk) -> np.ndarray:
    """q_lat[t,h,:] = Σ_d qn[t,h,d]·W_UK[h,d,:] — W_UK folded into the query (A6).

    Used only to check a GPU intermediate; the attention output of this oracle
    never goes through it.
    """
    return np.einsum("hdc,thd->thc", _f64(w_uk), _f64(qn))


def lowrank_query(x, w_qa, q_gain, w_qb, pos, *, n_heads, d_nope, d_rope, theta, eps, inv_freq=None):
    """The low-rank query path, page "MLA 原理" §"步骤" (the report's eqs. (37)-(40)):
    q = q_b_proj(q_a_layernorm(q_a_proj(x))), viewed as [H, d_nope + d_rope] per
    token and split into q_nope (first d_nope) and q_pe (last d_rope); q_pe is then
    rotated like the full-rank q_pe.  Same structure on the nanowhale page
    (wq_a, q_norm = RMSNorm over the q rank, wq_b).
    W_QA [q_rank, d_model]; q_gain [q_rank] (None: unit gain); W_QB [H·(d_nope+d_rope), q_rank].
    Returns (qn [T, H, d_nope], qr [T, H, d_rope])."""
    cq = rmsnorm(_f64(x) @ _f64(w_qa).T, eps)
    if q_gain is not None:
        cq = cq * _f64(q_gain)
    q = (cq @ _f64(w_qb).T).reshape(-1, n_heads, d_nope + d_rope)
    return q[..., :d_nope], rope(q[..., d_nope:], pos, theta, inv_freq)


# ----------------------------------------------------------------------------
# non-absorbed attention
# ----------------------------------------------------------------------------


def expand_kv(c, w_uk, w_uv):
    """Decompress every cached latent: kn[s,h,:] = W_UK[h]·c[s], v[s,h,:] = W_UV[h]·c[s]."""
    c = _f64(c)
    kn = np.einsum("hdc,sc->shd", _f64(w_uk), c)
    v = np.einsum("hdc,sc->shd", _f64(w_uv), c)
    return kn, v


def head_groups(n_heads: int, n_groups: int) -> np.ndarray:
    """g(h) = h // (H/G): contiguous blocks of query heads share a rotary key."""
    if n_heads % n_groups:
        raise ValueError("heads must divide evenly into rotary-key groups")
    return np.arange(n_heads) // (n_heads // n_groups)


def softmax_attention(q, k, v, allowed, scale: float) -> np.ndarray:
    """Standard attention for one query set: q [Tq, H, d], k [S, H, d], v [S, H, e],
    ``allowed`` [Tq, S] bool.  a = scale·q·k; P = softmax over allowed keys
    (max subtracted); out = P·v.  Every query must allow at least one key."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    # a[h,t,s] = scale·Σ_d q[t,h,d]·k[s,h,d]  (a matrix product per head)
    a = scale * np.matmul(q.transpose(1, 0, 2), k.transpose(1, 2, 0))
    a = np.where(allowed[None, :, :], a, -np.inf)
    m = a.max(axis=-1, keepdims=True)
    e = np.exp(a - m)
    p = e / e.sum(axis=-1, keepdims=True)
    # out[t,h,e] = Σ_s p[h,t,s]·v[s,h,e]
    return np.matmul(p, v.transpose(1, 0, 2)).transpose(1, 0, 2)


def mla_attention(qn, qr, c, kr, w_uk, w_uv, q_pos, k_pos, q_seg, k_seg, scale, *,
                  head_chunk: int | None = None, query_chunk: int = 64) -> np.ndarray:
    """Non-absorbed MLA attention output [Tq, H, d_v] (before W_o).

    K[s,h] = [kn[s,h] ; kr[s, g(h)]], Q[t,h] = [qn[t,h] ; qr[t,h]]; query t may
    attend key s iff they are in the same sequence and p[s] <= p[t].
    """
    qn, qr = _f64(qn), _f64(qr)
    c, kr = _f64(c), _f64(kr)
    q_pos, k_pos = np.asarray(q_pos), np.asarray(k_pos)
    q_seg, k_seg = np.asarray(q_seg), np.asarray(k_seg)
    Tq, H, _ = qn.shape
    G = kr.shape[1]
    d_v = w_uv.shape[1]
    g_of_h = head_groups(H, G)
    out = np.zeros((Tq, H, d_v), F64)
    hc = head_chunk or H
    for h0 in range(0, H, hc):
        h1 = min(H, h0 + hc)
        kn, v = expand_kv(c, w_uk[h0:h1], w_uv[h0:h1])
        K = np.concatenate([kn, kr[:, g_of_h[h0:h1], :]], axis=-1)
        Q = np.concatenate([qn[:, h0:h1], qr[:, h0:h1]], axis=-1)
        for t0 in range(0, Tq, query_chunk):
            t1 = min(Tq, t0 + query_chunk)
            allowed = (q_seg[t0:t1, None] == k_seg[None, :]) & (k_pos[None, :] <= q_pos[t0:t1, None])
            keys = np.nonzero(allowed.any(axis=0))[0]
            if keys.size == 0:
                raise ValueError("a query has no key to attend")
            out[t0:t1, h0:h1] = softmax_attention(Q[t0:t1], K[keys], v[keys],
                                                  allowed[:, keys], scale)
    return out


def mla_layer(x_keys, x_queries, w, *, k_pos, q_pos, k_seg, q_seg, n_heads, n_groups,
              d_nope, d_rope, theta, scale, latent_rmsnorm=False, eps=1e-6,
              head_chunk=None, inv_freq=None) -> np.ndarray:
    """End-to-end chain: cache rows from x_keys, queries from x_queries, attention output.

    ``w`` holds w_dkv, w_kr, w_qc, w_qr, w_uk, w_uv (float arrays)."""
    r = w["w_dkv"].shape[0]
    rows = cache_rows(x_keys, w["w_dkv"], w["w_kr"], k_pos, n_groups=n_groups, d_rope=d_rope,
                      theta=theta, latent_rmsnorm=latent_rmsnorm, eps=eps, inv_freq=inv_freq)
    c, kr = split_rows(rows, r, n_groups, d_rope)
    qn, qr = query(x_queries, w["w_qc"], w["w_qr"], q_pos, n_heads=n_heads, d_nope=d_nope,
                   d_rope=d_rope, theta=theta, inv_freq=inv_freq)
    return mla_attention(qn, qr, c, kr, w["w_uk"], w["w_uv"], q_pos, k_pos, q_seg, k_seg,
                         scale, head_chunk=head_chunk)


def output_projection(o, w_o) -> np.ndarray:
    """u[t,:] = Σ_h Σ_e o[t,h,e]·W_o[:, h·d_v + e]: page "MLA 原理", eqs. (3)/(6)
    (einsum 'hdD,bhqd->bqD' of W_o with the per-head outputs), after W_UV.
    o [T, H, d_v]; W_o stored [d_model, H·d_v] (o_proj, [H·d_v -> hidden])."""
    o = _f64(o)
    return o.reshape(o.shape[0], -1) @ _f64(w_o).T


# ----------------------------------------------------------------------------
# DeepSeek-V4 / nanowhale variant: one latent head serves as both K and V
# (page "MLA 在 nanowhale-100m 中的实现原理")
# ----------------------------------------------------------------------------


def rope_interleaved(y, pos, theta: float = 10000.0, inv_freq=None) -> np.ndarray:
    """The nanowhale page's apply_rotary_emb(x, freqs_cis) (§"RoPE位置编码的优化应用"):
    dims (2j, 2j+1) are the complex number y[2j] + i·y[2j+1], multiplied by
    e^{i·p·f_j} with f_j = θ^(-2j/d) or a given inverse-frequency table (a
    context-extension rescaling such as YaRN supplies its own table).  A negative
    position rotates back (the page's inverse rotation of the output)."""
    y = _f64(y)
    d = y.shape[-1]
    f = _f64(inv_freq) if inv_freq is not None else float(theta) ** (-2.0 * np.arange(d // 2, dtype=F64) / d)
    ang = _f64(pos)[..., None] * f
    while ang.ndim < y.ndim:
        ang = np.expand_dims(ang, axis=-2)
    c, s = np.cos(ang), np.sin(ang)
    a, b = y[..., 0::2], y[..., 1::2]
    out = np.empty_like(y)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = b * c + a * s
    return out


def v4_cache_rows(x, w_kv, kv_gain, pos, *, d_rope, eps, theta=10000.0, inv_freq=None) -> np.ndarray:
    """kv = kv_norm(x·W_KVᵀ) (RMSNorm with gain over head_dim, §"单KV头多查询头设计"),
    then the last d_rope dims rotated by the token's position (§"RoPE位置编码的优化应用").
    W_KV [head_dim, d_model]; returns the cached rows [T, head_dim]."""
    kv = rmsnorm(_f64(x) @ _f64(w_kv).T, eps) * _f64(kv_gain)
    kv[:, -d_rope:] = rope_interleaved(kv[:, -d_rope:], pos, theta, inv_freq)
    return kv


def v4_query(x, w_qa, q_gain, w_qb, pos, *, n_heads, head_dim, d_rope, eps, theta=10000.0,
             inv_freq=None) -> np.ndarray:
    """q = wq_b(q_norm(wq_a(x))) viewed [H, head_dim] (§"低秩查询投影机制"), its last
    d_rope dims rotated by the token's position.  Returns [T, H, head_dim]."""
    c = rmsnorm(_f64(x) @ _f64(w_qa).T, eps) * _f64(q_gain)
    q = (c @ _f64(w_qb).T).reshape(-1, n_heads, head_dim)
    q[..., -d_rope:] = rope_interleaved(q[..., -d_rope:], pos, theta, inv_freq)
    return q


def v4_attention(q, kv, sink, q_pos, k_pos, q_seg, k_seg, scale, *, d_rope, theta=10000.0,
                 inv_freq=None) -> np.ndarray:
    """Multi-query attention with K = V = the cached row (§"高效注意力计算实现": SDPA of
    q against kv_expanded for both keys and values, causal), a per-head attention
    sink (a learned logit that joins each softmax's normalisation and carries no
    value), and the inverse rotation of the output's last d_rope dims by the
    query's position (§"RoPE位置编码的优化应用": rotation before and after attention).
    q [T, H, D]; kv [S, D]; sink [H]; returns [T, H, D]."""
    q, kv, sink = _f64(q), _f64(kv), _f64(sink)
    allowed = (_f64(q_seg)[:, None] == _f64(k_seg)[None, :]) & (_f64(k_pos)[None, :] <= _f64(q_pos)[:, None])
    a = scale * np.einsum("thd,sd->hts", q, kv)
    a = np.where(allowed[None], a, -np.inf)
    m = np.maximum(a.max(axis=-1), sink[:, None])                  # [H, T]
    e = np.exp(a - m[..., None])
    den = e.sum(axis=-1) + np.exp(sink[:, None] - m)
    o = np.einsum("hts,sd->thd", e, kv) / den.T[..., None]
    o[..., -d_rope:] = rope_interleaved(o[..., -d_rope:], -_f64(q_pos)[:, None], theta, inv_freq)
    return o


def v4_output(o, w_oa, w_ob, o_groups: int) -> np.ndarray:
    """Grouped low-rank output projection (§"分组低秩输出投影"): the H·D outputs are cut
    into o_groups groups, group g is projected by its own [o_rank, H·D/o_groups] block
    of W_OA (rows g·o_rank ...), and the concatenated o_groups·o_rank values by W_OB
    [d_model, o_groups·o_rank]."""
    o = _f64(o)
    T = o.shape[0]
    og = o.reshape(T, o_groups, -1)
    w = _f64(w_oa).reshape(o_groups, -1, og.shape[-1])
    a = np.einsum("tgd,grd->tgr", og, w).reshape(T, -1)
    return a @ _f64(w_ob).T


def max_rel_err(got, ref) -> float:
    """max over (token, head) of ‖got − ref‖∞ / ‖ref‖∞ over the last axis.

    The parity metric (per output vector, not per element: an attention output is
    a weighted mean that crosses zero).  A vector whose reference is all zero is
    measured by its absolute error; a NaN or inf in ``got`` makes the result NaN
    or inf, which no bar accepts.  Empty inputs give 0."""
    got, ref = _f64(got), _f64(ref)
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max()) if num.size else 0.0
