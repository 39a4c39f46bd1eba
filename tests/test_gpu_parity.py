"""GPU parity: the HIP path through the C ABI against the float64 oracle on the same
seeded inputs.  Tolerance: max over (token, head) of ‖gpu − oracle‖∞ / ‖oracle‖∞
over the d_v outputs <= 1e-2 for bf16 workloads and 1e-4 for the fp32 one.

Three levels for decode workloads: (i) cache rows written by mla_write_cache vs
the oracle's rows; (ii) attention on the GPU-written cache (oracle reads the same
rows); (iii) the whole chain from x."""
import numpy as np
import pytest

import mla_inputs as I
from tests import harness as Hh

pytestmark = pytest.mark.gpu


def _print_case(name, **kw):
    print(f"[case] {name} {kw}", flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch
    import head_latent_attention_kv_amd as M
    M.load()
    assert torch.cuda.is_available()
    return torch


# ----------------------------------------------------------------------------
# fp32 tiny layer: prefill 256 then 16 decode steps, full size
# ----------------------------------------------------------------------------


def test_tiny_f32_prefill_then_decode(torch):
    import head_latent_attention_kv_amd as M
    from oracle import mla_oracle as O
    cfg = I.CONFIGS["tiny_f32"]
    _print_case("tiny_f32", L=cfg.prefill_len, steps=cfg.decode_steps)
    layer = Hh.make_layer(cfg)
    n_all = cfg.prefill_len + cfg.decode_steps
    x = I.x_rows(cfg, 0, 0, n_all)
    cache = torch.zeros((n_all, cfg.row_width), dtype=torch.float32, device="cuda")
    # prefill
    L = cfg.prefill_len
    xd = Hh.to_dev(x[:L], cfg.dtype)
    Hh.write_cache(layer, xd, np.arange(L), np.arange(L), cache)
    q_lat, q_pe = Hh.absorb(layer, xd, np.arange(L))
    out_pre = torch.empty((L, cfg.n_heads, cfg.d_v), dtype=torch.float32, device="cuda")
    cu = torch.tensor([0, L], dtype=torch.int64, device="cuda")
    M.mla_prefill(layer.dims, q_lat, q_pe, cache, cu, L, layer.w_dev["w_uv"], out_pre)
    # decode steps: write the new row, then attend over all rows so far
    outs = []
    for i in range(cfg.decode_steps):
        p = L + i
        xi = Hh.to_dev(x[p:p + 1], cfg.dtype)
        Hh.write_cache(layer, xi, np.array([p]), np.array([p]), cache)
        ql, qp = Hh.absorb(layer, xi, np.array([p]))
        o = torch.empty((1, cfg.n_heads, cfg.d_v), dtype=torch.float32, device="cuda")
        M.mla_decode(layer.dims, ql, qp, cache, torch.zeros(1, dtype=torch.int64, device="cuda"),
                     torch.tensor([p + 1], dtype=torch.int32, device="cuda"), p + 1,
                     layer.w_dev["w_uv"], o)
        outs.append(o)
    torch.cuda.synchronize()
    got = np.concatenate([Hh.to_host(out_pre)] + [Hh.to_host(o) for o in outs])
    pos = np.arange(n_all)
    ref = O.mla_layer(x, x, layer.w_host, k_pos=pos, q_pos=pos, k_seg=np.zeros(n_all, int),
                      q_seg=np.zeros(n_all, int), n_heads=cfg.n_heads, n_groups=cfg.n_groups,
                      d_nope=cfg.d_nope, d_rope=cfg.d_rope, theta=cfg.rope_theta,
                      scale=cfg.softmax_scale)
    err = Hh.rel_err_rows(got, ref)
    print(f"tiny_f32 chain max rel err {err:.3e}")
    assert err <= Hh.TOL["f32"]
    # cache rows (i)
    rows_ref = O.cache_rows(x, layer.w_host["w_dkv"], layer.w_host["w_kr"], pos, n_groups=cfg.n_groups,
                            d_rope=cfg.d_rope, theta=cfg.rope_theta)
    assert Hh.rel_err_rows(Hh.to_host(cache), rows_ref) <= 1e-5


# ----------------------------------------------------------------------------
# bf16 decode workloads at their full layer dims, reduced batch / lengths
# ----------------------------------------------------------------------------

DECODE_CASES = [
    ("qwen25_7b_decode", [1, 65, 511, 1000]),
    ("deepseek_v2_decode", [1, 300, 2048]),
    ("qwen3_30b_ragged_decode", [1024, 1537]),
    # more splits than the merge folded into W_UV takes: the split plan is made
    # on the device from these lengths (sequences of 1 and 40 rows get one split)
    ("qwen3_30b_ragged_decode", [1, 40, 3000, 9000, 20000]),
    # the generic kernel's plan: one-tile splits, splits past a short sequence empty
    ("tiny_f32", [1, 31, 32, 33, 65, 300]),
    # the 576-wide row with a head count the 128-head kernel does not take: the
    # generic MFMA kernel, two workgroups of 64 heads per split
    ("deepseek_v2_h120", [1, 300, 2048]),
]
# reduced variants of the workloads, by the name the cases above use
DECODE_VARIANTS = {"deepseek_v2_h120": ("deepseek_v2_decode", dict(n_heads=120, d_model=1024))}


def _decode_cfg(name):
    if name in DECODE_VARIANTS:
        base, changes = DECODE_VARIANTS[name]
        return I.small_variant(I.CONFIGS[base], **changes)
    return I.CONFIGS[name]


@pytest.mark.parametrize("name,lengths", DECODE_CASES)
def test_decode_reduced(torch, name, lengths):
    from oracle import mla_oracle as O
    cfg = _decode_cfg(name)
    _print_case("decode_reduced", cfg=name, lengths=lengths)
    layer = Hh.make_layer(cfg)
    run = Hh.build_decode(layer, np.array(lengths))
    got = Hh.to_host(run.out)
    cache_h = Hh.to_host(run.cache)
    w = layer.w_host
    errs = {"write": 0.0, "attn": 0.0, "chain": 0.0, "q_lat": 0.0, "q_pe": 0.0}
    for b, n in enumerate(run.lengths):
        n = int(n)
        xb = I.x_rows(cfg, b, 0, n)
        rows_ref = O.cache_rows(xb, w["w_dkv"], w["w_kr"], np.arange(n), n_groups=cfg.n_groups,
                                d_rope=cfg.d_rope, theta=cfg.rope_theta,
                                latent_rmsnorm=cfg.latent_rmsnorm, eps=cfg.rms_eps)
        rows_gpu = cache_h[run.starts[b]:run.starts[b] + n]
        errs["write"] = max(errs["write"], Hh.write_err(cfg, rows_gpu, rows_ref))
        attn = Hh.oracle_decode_rows(cfg, w, None, run.x_query[b], n, cache_rows=rows_gpu)
        chain = Hh.oracle_decode_rows(cfg, w, xb, run.x_query[b], n, cache_rows=rows_ref)
        errs["attn"] = max(errs["attn"], Hh.rel_err_rows(got[b], attn))
        errs["chain"] = max(errs["chain"], Hh.rel_err_rows(got[b], chain))
        qn, qr = O.query(run.x_query[b:b + 1], w["w_qc"], w["w_qr"], np.array([n - 1]),
                         n_heads=cfg.n_heads, d_nope=cfg.d_nope, d_rope=cfg.d_rope, theta=cfg.rope_theta)
        errs["q_lat"] = max(errs["q_lat"], Hh.rel_err_rows(Hh.to_host(run.q_lat[b]), O.absorbed_query(qn, w["w_uk"])[0]))
        errs["q_pe"] = max(errs["q_pe"], Hh.rel_err_rows(Hh.to_host(run.q_pe[b]), qr[0]))
    print(f"{name} {lengths}: " + " ".join(f"{k}={v:.3e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= Hh.TOL[cfg.dtype], (k, v)


# The widest cache row the library takes (the largest rank, 512, and four
# 128-wide rotary keys: r + G·d_rope = 1024, the cache-row epilogue's limit),
# with latent RMSNorm: no MFMA instance covers it, so decode and prefill run
# the generic attention kernel.
WIDE_ROW = I.MLAConfig(name="wide_row_edge", seed=1101, d_model=512, n_heads=8, n_groups=4, rank=512,
                       d_rope=128, d_nope=64, d_v=64, dtype="bf16", mode="prefill+decode", batch=3,
                       latent_rmsnorm=True)


def test_widest_cache_row_decode_and_prefill(torch):
    """The largest row width (1024 values: r = 512 and four 128-wide rotary keys) with
    one-token, ragged and tile-spanning sequences, decode and causal prefill, against
    the oracle's whole chain."""
    import head_latent_attention_kv_amd as M
    from oracle import mla_oracle as O
    cfg = WIDE_ROW
    lengths = [1, 333, 70]
    _print_case("widest_row", lengths=lengths)
    layer = Hh.make_layer(cfg)
    T = sum(lengths)
    x = np.concatenate([I.x_rows(cfg, b, 0, n) for b, n in enumerate(lengths)])
    pos = np.concatenate([np.arange(n) for n in lengths])
    seg = np.concatenate([np.full(n, b) for b, n in enumerate(lengths)])
    cache = torch.empty((T, cfg.row_width), dtype=torch.bfloat16, device="cuda")
    xd = Hh.to_dev(x, cfg.dtype)
    Hh.write_cache(layer, xd, pos, np.arange(T), cache)
    q_lat, q_pe = Hh.absorb(layer, xd, pos)
    out = torch.empty((T, cfg.n_heads, cfg.d_v), dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int64, device="cuda")
    M.mla_prefill(layer.dims, q_lat, q_pe, cache, cu, max(lengths), layer.w_dev["w_uv"], out)
    # decode: the last token of each sequence against its rows
    last = np.cumsum(lengths) - 1
    out_d = torch.empty((len(lengths), cfg.n_heads, cfg.d_v), dtype=torch.bfloat16, device="cuda")
    M.mla_decode(layer.dims, q_lat[torch.from_numpy(last).cuda()].contiguous(),
                 q_pe[torch.from_numpy(last).cuda()].contiguous(), cache,
                 torch.from_numpy(np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)).cuda(),
                 torch.tensor(lengths, dtype=torch.int32, device="cuda"), max(lengths), layer.w_dev["w_uv"], out_d)
    torch.cuda.synchronize()
    ref = O.mla_layer(x, x, layer.w_host, k_pos=pos, q_pos=pos, k_seg=seg, q_seg=seg, n_heads=cfg.n_heads,
                      n_groups=cfg.n_groups, d_nope=cfg.d_nope, d_rope=cfg.d_rope, theta=cfg.rope_theta,
                      scale=cfg.softmax_scale, latent_rmsnorm=True, eps=cfg.rms_eps)
    err_p = Hh.rel_err_rows(Hh.to_host(out), ref)
    err_d = Hh.rel_err_rows(Hh.to_host(out_d), ref[last])
    print(f"widest row {lengths}: prefill {err_p:.3e}, decode {err_d:.3e}")
    assert err_p <= Hh.TOL["bf16"] and err_d <= Hh.TOL["bf16"]


@pytest.mark.parametrize("name,lengths", [("deepseek_v2_decode", [700, 2100, 90]),
                                          ("qwen25_7b_decode", [1500, 333])])
def test_decode_restart(torch, name, lengths):
    """Keys from position 40 on are scaled 30x (the query row is not), so the
    scores of later tiles pass the first tile's reference by 96..224 (log2) in
    every head, far beyond its 2^64 headroom, and the attention kernels take
    their second pass with the true maximum.  Logits this large make the bf16
    rounding of the query itself move the softmax by ~10%, so the reference is
    the oracle's attention definition on the query and rows the kernel reads."""
    cfg = I.CONFIGS[name]
    _print_case("decode_restart", cfg=name, lengths=lengths)
    boost = (40, 30.0)
    layer = Hh.make_layer(cfg)
    run = Hh.build_decode(layer, np.array(lengths), key_boost=boost)
    got = Hh.to_host(run.out)
    cache_h = Hh.to_host(run.cache)
    err = 0.0
    for b, n in enumerate(run.lengths):
        n = int(n)
        rows_gpu = cache_h[run.starts[b]:run.starts[b] + n]
        ref = Hh.oracle_absorbed_rows(cfg, layer.w_host, Hh.to_host(run.q_lat[b]), Hh.to_host(run.q_pe[b]),
                                      rows_gpu)
        err = max(err, Hh.rel_err_rows(got[b], ref))
    print(f"{name} restart {lengths}: attn={err:.3e}")
    assert err <= Hh.TOL[cfg.dtype], err


@pytest.mark.parametrize("tokens", [37, 64])
def test_absorb_wide_ragged_k(torch, tokens):
    """mla_absorb at H=128 (24576 projection columns, the column-tiled weight
    stream staged through LDS) with d_model = 5000, so the last k stage of the
    projection is partial, and a ragged token count: q_lat and q_pe against the
    oracle's query path."""
    from oracle import mla_oracle as O
    cfg = I.small_variant(I.CONFIGS["deepseek_v2_decode"], d_model=5000, seed=2001)
    _print_case("absorb_wide_ragged_k", tokens=tokens, d_model=cfg.d_model)
    layer = Hh.make_layer(cfg)
    x = I.x_rows(cfg, 0, 0, tokens)
    pos = np.arange(tokens) * 97 % 8192
    q_lat, q_pe = Hh.absorb(layer, Hh.to_dev(x, cfg.dtype), pos)
    w = layer.w_host
    qn, qr = O.query(x, w["w_qc"], w["w_qr"], pos, n_heads=cfg.n_heads, d_nope=cfg.d_nope,
                     d_rope=cfg.d_rope, theta=cfg.rope_theta)
    err_lat = Hh.rel_err_rows(Hh.to_host(q_lat), O.absorbed_query(qn, w["w_uk"]))
    err_pe = Hh.rel_err_rows(Hh.to_host(q_pe), qr)
    print(f"absorb tokens={tokens}: q_lat={err_lat:.3e} q_pe={err_pe:.3e}")
    assert err_lat <= Hh.TOL[cfg.dtype] and err_pe <= Hh.TOL[cfg.dtype], (err_lat, err_pe)


@pytest.mark.parametrize("n_split", [1, 3, None])
def test_decode_partials_merge(torch, n_split):
    """mla_decode_partials: the host merges the per-split partials (each split's
    normalised o_ and its (m, l)) by their stated definition in float64, applies
    W_UV, and must match the oracle's attention on the GPU-written rows; splits
    past a short sequence must come back empty."""
    import head_latent_attention_kv_amd as M
    cfg = I.CONFIGS["deepseek_v2_decode"]
    lengths = [1, 300, 2048]
    _print_case("decode_partials", cfg=cfg.name, lengths=lengths, n_split=n_split)
    layer = Hh.make_layer(cfg)
    run = Hh.build_decode(layer, np.array(lengths))
    B, H, r = len(lengths), cfg.n_heads, cfg.rank
    max_len = int(max(lengths))
    ns = M.mla_decode_splits(layer.dims, B, max_len) if n_split is None else n_split
    split_rows = (-(-max_len // ns) + 63) // 64 * 64
    part_o = torch.full((B, ns, H, r), float("nan"), dtype=torch.bfloat16, device="cuda")
    part_ml = torch.full((B, ns, H, 2), float("nan"), dtype=torch.float32, device="cuda")
    seq_start = torch.from_numpy(run.starts).cuda()
    seq_len = torch.from_numpy(run.lengths.astype(np.int32)).cuda()
    M.mla_decode_partials(layer.dims, run.q_lat, run.q_pe, run.cache, seq_start, seq_len, max_len, ns,
                          part_o, part_ml)
    torch.cuda.synchronize()
    po = Hh.to_host(part_o).astype(np.float64)
    pml = Hh.to_host(part_ml).astype(np.float64)
    assert np.isfinite(po).all() and not np.isnan(pml).any()
    cache_h = Hh.to_host(run.cache)
    w = layer.w_host
    err = 0.0
    for b, n in enumerate(run.lengths):
        n = int(n)
        empty = [j for j in range(ns) if j * split_rows >= n]
        for j in empty:
            assert np.all(pml[b, j, :, 0] == -np.inf) and np.all(pml[b, j, :, 1] == 0), (b, j)
            assert np.all(po[b, j] == 0), (b, j)
        m, lsum = pml[b, :, :, 0], pml[b, :, :, 1]           # [ns, H]
        mx = m.max(axis=0)
        wj = np.where(np.isneginf(m), 0.0, np.exp2(m - mx)) * lsum
        o_lat = (wj[:, :, None] * po[b]).sum(0) / wj.sum(0)[:, None]
        out = np.einsum("hdc,hc->hd", w["w_uv"].astype(np.float64), o_lat)
        ref = Hh.oracle_decode_rows(cfg, w, None, run.x_query[b], n,
                                    cache_rows=cache_h[run.starts[b]:run.starts[b] + n])
        err = max(err, Hh.rel_err_rows(out, ref))
    print(f"partials n_split={ns}: merged attention max rel err {err:.3e}")
    assert err <= Hh.TOL[cfg.dtype]


def test_decode_deterministic(torch):
    cfg = I.small_variant(I.CONFIGS["deepseek_v2_decode"], d_model=512)
    _print_case("decode_deterministic")
    layer = Hh.make_layer(cfg)
    a = Hh.build_decode(layer, np.array([777, 3000, 64]))
    b = Hh.build_decode(layer, np.array([777, 3000, 64]))
    assert torch.equal(a.out, b.out) and torch.equal(a.cache, b.cache)


# ----------------------------------------------------------------------------
# prefill (bf16) at the long-prefill layer dims, reduced length, ragged batch
# ----------------------------------------------------------------------------


def test_prefill_reduced_ragged(torch):
    import head_latent_attention_kv_amd as M
    from oracle import mla_oracle as O
    cfg = I.CONFIGS["long_prefill_131k"]
    lengths = [700, 1, 333]
    _print_case("prefill_reduced", lengths=lengths)
    layer = Hh.make_layer(cfg)
    T = sum(lengths)
    xs = [I.x_rows(cfg, b, 0, n) for b, n in enumerate(lengths)]
    x = np.concatenate(xs)
    pos = np.concatenate([np.arange(n) for n in lengths])
    seg = np.concatenate([np.full(n, b) for b, n in enumerate(lengths)])
    cache = torch.empty((T, cfg.row_width), dtype=torch.bfloat16, device="cuda")
    xd = Hh.to_dev(x, cfg.dtype)
    Hh.write_cache(layer, xd, pos, np.arange(T), cache)
    q_lat, q_pe = Hh.absorb(layer, xd, pos)
    out = torch.empty((T, cfg.n_heads, cfg.d_v), dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int64, device="cuda")
    M.mla_prefill(layer.dims, q_lat, q_pe, cache, cu, max(lengths), layer.w_dev["w_uv"], out)
    torch.cuda.synchronize()
    got = Hh.to_host(out)
    w = layer.w_host
    ref = O.mla_layer(x, x, w, k_pos=pos, q_pos=pos, k_seg=seg, q_seg=seg, n_heads=cfg.n_heads,
                      n_groups=cfg.n_groups, d_nope=cfg.d_nope, d_rope=cfg.d_rope,
                      theta=cfg.rope_theta, scale=cfg.softmax_scale, head_chunk=4)
    err = Hh.rel_err_rows(got, ref)
    print(f"prefill ragged {lengths}: chain max rel err {err:.3e}")
    assert err <= Hh.TOL["bf16"]


def test_prefill_full_size_sampled(torch):
    """The 131072-token causal prefill at full size: the whole chain runs on the
    GPU; 512 seeded rows spread over the sequence (row 0 and the last row
    included) are checked against the oracle on the GPU-written cache (attention
    parity), every eighth of them also against the oracle's own cache (chain
    parity), and their q_lat / q_pe against the oracle's queries."""
    from oracle import mla_oracle as O
    cfg = I.CONFIGS["long_prefill_131k"]
    L = cfg.prefill_len
    _print_case("prefill_full_size", cfg=cfg.name, L=L)
    layer = Hh.make_layer(cfg)
    run = Hh.build_prefill(layer, L)
    rows = I.sample_rows(cfg)
    print("  gpu chain done; oracle attention on the gpu cache", flush=True)
    got = Hh.to_host(run.out[torch.from_numpy(rows).cuda()])
    cache_h = Hh.to_host(run.cache)
    w = layer.w_host
    c, kr = O.split_rows(cache_h, cfg.rank, cfg.n_groups, cfg.d_rope)
    qn, qr = O.query(run.x_q[rows], w["w_qc"], w["w_qr"], rows, n_heads=cfg.n_heads, d_nope=cfg.d_nope,
                     d_rope=cfg.d_rope, theta=cfg.rope_theta)
    zeros_q, zeros_k = np.zeros(len(rows), int), np.zeros(L, int)
    ref = O.mla_attention(qn, qr, c, kr, w["w_uk"], w["w_uv"], rows, np.arange(L), zeros_q, zeros_k,
                          cfg.softmax_scale, head_chunk=1)
    err_attn = Hh.rel_err_rows(got, ref)
    err_qlat = Hh.rel_err_rows(Hh.to_host(run.q_lat[torch.from_numpy(rows).cuda()]), O.absorbed_query(qn, w["w_uk"]))
    err_qpe = Hh.rel_err_rows(Hh.to_host(run.q_pe[torch.from_numpy(rows).cuda()]), qr)
    print(f"  attention parity {err_attn:.3e}, q_lat {err_qlat:.3e}, q_pe {err_qpe:.3e}; oracle chain", flush=True)
    sub = rows[::8].copy()
    sub[-1] = rows[-1]
    rows_ref = O.cache_rows(run.x_q, w["w_dkv"], w["w_kr"], np.arange(L), n_groups=cfg.n_groups,
                            d_rope=cfg.d_rope, theta=cfg.rope_theta)
    err_write = Hh.write_err(cfg, cache_h, rows_ref)
    c_o, kr_o = O.split_rows(rows_ref, cfg.rank, cfg.n_groups, cfg.d_rope)
    sel = np.searchsorted(rows, sub)
    ref_chain = O.mla_attention(qn[sel], qr[sel], c_o, kr_o, w["w_uk"], w["w_uv"], sub, np.arange(L),
                                np.zeros(len(sub), int), zeros_k, cfg.softmax_scale, head_chunk=1)
    err_chain = Hh.rel_err_rows(got[sel], ref_chain)
    # the same prefill in the original order, checked against the same references
    xd = Hh.to_dev(run.x_q, cfg.dtype)
    q_nope, q_pe_e = Hh.query(layer, xd, np.arange(L))
    del xd
    out_e, ws_e = Hh.prefill_expanded(layer, q_nope, q_pe_e, run.cache, [L])
    torch.cuda.synchronize()
    got_e = Hh.to_host(out_e[torch.from_numpy(rows).cuda()])
    del ws_e, out_e
    err_e = Hh.rel_err_rows(got_e, ref)
    err_e_chain = Hh.rel_err_rows(got_e[sel], ref_chain)
    print(f"prefill {L}: attn={err_attn:.3e} chain={err_chain:.3e} write={err_write:.3e} "
          f"q_lat={err_qlat:.3e} q_pe={err_qpe:.3e}; original order attn={err_e:.3e} chain={err_e_chain:.3e}")
    for name, v in (("attn", err_attn), ("chain", err_chain), ("write", err_write), ("q_lat", err_qlat),
                    ("q_pe", err_qpe), ("expanded attn", err_e), ("expanded chain", err_e_chain)):
        assert v <= Hh.TOL[cfg.dtype], (name, v)


# ----------------------------------------------------------------------------
# prefill in the original order (expanded k_nope / v), long-prefill layer dims
# ----------------------------------------------------------------------------


@pytest.mark.parametrize("name", ["tiny_f32", "long_prefill_131k"])
def test_query_matches_oracle(torch, name):
    from oracle import mla_oracle as O
    cfg = I.CONFIGS[name]
    T = 300
    _print_case("query", cfg=name, T=T)
    layer = Hh.make_layer(cfg)
    x = I.x_rows(cfg, 0, 0, T)
    pos = np.random.default_rng(7).integers(0, 100000, T)
    q_nope, q_pe = Hh.query(layer, Hh.to_dev(x, cfg.dtype), pos)
    torch.cuda.synchronize()
    qn, qr = O.query(x, layer.w_host["w_qc"], layer.w_host["w_qr"], pos, n_heads=cfg.n_heads,
                     d_nope=cfg.d_nope, d_rope=cfg.d_rope, theta=cfg.rope_theta)
    e_n = Hh.rel_err_rows(Hh.to_host(q_nope), qn)
    e_r = Hh.rel_err_rows(Hh.to_host(q_pe), qr)
    print(f"{name} query: q_nope {e_n:.3e} q_pe {e_r:.3e}")
    assert e_n <= Hh.TOL[cfg.dtype] and e_r <= Hh.TOL[cfg.dtype]


@pytest.mark.parametrize("lengths", [[700, 1, 333], [256], [1], [300, 257, 513, 40]])
def test_prefill_expanded_ragged(torch, lengths):
    """Ragged batches (workgroups of 256 queries spanning sequence ends, a ragged
    last tile, one-token sequences) against the oracle's whole chain; the
    expanded k_nope / v the call leaves in its workspace against the oracle's
    expansion of the GPU-written latents; and the same call in the absorbed
    order (mla_prefill) against the same oracle."""
    import head_latent_attention_kv_amd as M
    from oracle import mla_oracle as O
    cfg = I.CONFIGS["long_prefill_131k"]
    _print_case("prefill_expanded", lengths=lengths)
    layer = Hh.make_layer(cfg)
    T = sum(lengths)
    x = np.concatenate([I.x_rows(cfg, b, 0, n) for b, n in enumerate(lengths)])
    pos = np.concatenate([np.arange(n) for n in lengths])
    seg = np.concatenate([np.full(n, b) for b, n in enumerate(lengths)])
    cache = torch.empty((T, cfg.row_width), dtype=torch.bfloat16, device="cuda")
    xd = Hh.to_dev(x, cfg.dtype)
    Hh.write_cache(layer, xd, pos, np.arange(T), cache)
    q_nope, q_pe = Hh.query(layer, xd, pos)
    out, ws = Hh.prefill_expanded(layer, q_nope, q_pe, cache, lengths)
    q_lat, q_pe_a = Hh.absorb(layer, xd, pos)
    out_abs = torch.empty_like(out)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int64, device="cuda")
    M.mla_prefill(layer.dims, q_lat, q_pe_a, cache, cu, max(lengths), layer.w_dev["w_uv"], out_abs)
    torch.cuda.synchronize()
    w = layer.w_host
    ref = O.mla_layer(x, x, w, k_pos=pos, q_pos=pos, k_seg=seg, q_seg=seg, n_heads=cfg.n_heads,
                      n_groups=cfg.n_groups, d_nope=cfg.d_nope, d_rope=cfg.d_rope,
                      theta=cfg.rope_theta, scale=cfg.softmax_scale, head_chunk=4)
    err = Hh.rel_err_rows(Hh.to_host(out), ref)
    err_abs = Hh.rel_err_rows(Hh.to_host(out_abs), ref)
    c, _ = O.split_rows(Hh.to_host(cache), cfg.rank, cfg.n_groups, cfg.d_rope)
    kn_ref, v_ref = O.expand_kv(c, w["w_uk"], w["w_uv"])          # [T, H, d]
    kn, v = Hh.expanded_kv(layer, ws, T)                             # [H, T, d]
    err_k = Hh.rel_err_rows(kn.transpose(1, 0, 2), kn_ref)
    err_v = Hh.rel_err_rows(v.transpose(1, 0, 2), v_ref)
    print(f"prefill expanded {lengths}: chain {err:.3e} (absorbed {err_abs:.3e}) k_nope {err_k:.3e} "
          f"v {err_v:.3e}")
    for nm, e in (("chain", err), ("absorbed", err_abs), ("k_nope", err_k), ("v", err_v)):
        assert e <= Hh.TOL["bf16"], (nm, e)


def test_yarn_table_at_million_positions(torch):
    """The Zebra page's YaRN extension (factor 32 over a 32K window) at positions near
    2^20: a frequency table from mla_rope_yarn_table in mla_dims.rope_freqs drives
    the cache write and the query rotation; the rotary keys, the absorbed prefill
    and the original-order prefill are checked against the oracle run with its own
    YaRN table."""
    import head_latent_attention_kv_amd as M
    from oracle import mla_oracle as O
    cfg = I.CONFIGS["long_prefill_131k"]
    lengths = [300, 45]
    starts = [1_048_576 - 300, 700_001]
    _print_case("yarn_table", lengths=lengths, starts=starts)
    table = torch.tensor(M.mla_rope_yarn_table(cfg.d_rope, cfg.rope_theta, 32.0, 32768.0),
                         dtype=torch.float64, device="cuda")
    layer = Hh.make_layer(cfg)
    layer.dims = M.dims_of(cfg, rope_freqs=table)
    inv = O.yarn_inv_freq(cfg.d_rope, cfg.rope_theta, 32.0, 32768.0)
    T = sum(lengths)
    x = np.concatenate([I.x_rows(cfg, b, 0, n) for b, n in enumerate(lengths)])
    pos = np.concatenate([np.arange(n) + p0 for n, p0 in zip(lengths, starts)])
    seg = np.concatenate([np.full(n, b) for b, n in enumerate(lengths)])
    cache = torch.empty((T, cfg.row_width), dtype=torch.bfloat16, device="cuda")
    xd = Hh.to_dev(x, cfg.dtype)
    Hh.write_cache(layer, xd, pos, np.arange(T), cache)
    q_lat, q_pe = Hh.absorb(layer, xd, pos)
    out_abs = torch.empty((T, cfg.n_heads, cfg.d_v), dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int64, device="cuda")
    M.mla_prefill(layer.dims, q_lat, q_pe, cache, cu, max(lengths), layer.w_dev["w_uv"], out_abs)
    q_nope, q_pe2 = Hh.query(layer, xd, pos)
    out, _ = Hh.prefill_expanded(layer, q_nope, q_pe2, cache, lengths)
    torch.cuda.synchronize()
    w = layer.w_host
    rows = O.cache_rows(x, w["w_dkv"], w["w_kr"], pos, n_groups=cfg.n_groups, d_rope=cfg.d_rope,
                        theta=cfg.rope_theta, inv_freq=inv)
    _, kr_ref = O.split_rows(rows, cfg.rank, cfg.n_groups, cfg.d_rope)
    _, kr = O.split_rows(Hh.to_host(cache), cfg.rank, cfg.n_groups, cfg.d_rope)
    _, qr_ref = O.query(x, w["w_qc"], w["w_qr"], pos, n_heads=cfg.n_heads, d_nope=cfg.d_nope,
                        d_rope=cfg.d_rope, theta=cfg.rope_theta, inv_freq=inv)
    ref = O.mla_layer(x, x, w, k_pos=pos, q_pos=pos, k_seg=seg, q_seg=seg, n_heads=cfg.n_heads,
                      n_groups=cfg.n_groups, d_nope=cfg.d_nope, d_rope=cfg.d_rope,
                      theta=cfg.rope_theta, scale=cfg.softmax_scale, head_chunk=4, inv_freq=inv)
    errs = {"kr": Hh.rel_err_rows(kr, kr_ref), "q_pe": Hh.rel_err_rows(Hh.to_host(q_pe2), qr_ref),
            "absorbed": Hh.rel_err_rows(Hh.to_host(out_abs), ref), "expanded": Hh.rel_err_rows(Hh.to_host(out), ref)}
    # without the table the rotation differs: the check above sees the table
    plain = O.cache_rows(x, w["w_dkv"], w["w_kr"], pos, n_groups=cfg.n_groups, d_rope=cfg.d_rope,
                         theta=cfg.rope_theta)
    errs_plain = Hh.rel_err_rows(kr, O.split_rows(plain, cfg.rank, cfg.n_groups, cfg.d_rope)[1])
    print("yarn table:", {k: f"{v:.3e}" for k, v in errs.items()}, f"(vs plain theta {errs_plain:.2e})")
    for nm, e in errs.items():
        assert e <= Hh.TOL["bf16"], (nm, e)
    assert errs_plain > 0.1


def test_prefill_expanded_restart(torch):
    """Hidden states from position 100 on are scaled 8x, so their queries and
    keys score ~64x higher against each other than against the first rows: the
    later tiles pass each query's first-tile reference by far more than the
    kernel's 2^15 headroom and the workgroups take their second pass with the
    true maximum.  At such logits the bf16 rounding of any operand moves the
    softmax, so the reference is the oracle's attention definition on exactly
    the operands the kernel reads: the GPU's q_nope / q_pe, the expanded
    k_nope / v from the workspace and the rotary keys of the GPU cache."""
    from oracle import mla_oracle as O
    cfg = I.CONFIGS["long_prefill_131k"]
    lengths = [600, 300]
    _print_case("prefill_expanded_restart", lengths=lengths)
    layer = Hh.make_layer(cfg)
    T = sum(lengths)
    xs = []
    for b, n in enumerate(lengths):
        xb = I.x_rows(cfg, b, 0, n, quantized=False)
        xb[100:] *= np.float32(8.0)
        xs.append(I.quantize(xb, cfg.dtype))
    x = np.concatenate(xs)
    pos = np.concatenate([np.arange(n) for n in lengths])
    seg = np.concatenate([np.full(n, b) for b, n in enumerate(lengths)])
    cache = torch.empty((T, cfg.row_width), dtype=torch.bfloat16, device="cuda")
    xd = Hh.to_dev(x, cfg.dtype)
    Hh.write_cache(layer, xd, pos, np.arange(T), cache)
    q_nope, q_pe = Hh.query(layer, xd, pos)
    out, ws = Hh.prefill_expanded(layer, q_nope, q_pe, cache, lengths)
    torch.cuda.synchronize()
    kn, v = Hh.expanded_kv(layer, ws, T)
    _, kr = O.split_rows(Hh.to_host(cache), cfg.rank, cfg.n_groups, cfg.d_rope)
    Q = np.concatenate([Hh.to_host(q_nope), Hh.to_host(q_pe)], axis=-1)          # [T, H, 192]
    K = np.concatenate([kn.transpose(1, 0, 2), np.repeat(kr, cfg.n_heads, 1)], axis=-1)
    allowed = (seg[:, None] == seg[None, :]) & (pos[None, :] <= pos[:, None])
    ref = O.softmax_attention(Q, K, v.transpose(1, 0, 2), allowed, cfg.softmax_scale)
    err = Hh.rel_err_rows(Hh.to_host(out), ref)
    print(f"prefill expanded restart {lengths}: attn {err:.3e}")
    assert err <= Hh.TOL["bf16"], err


def _quiet(t, sel, factor=0.02):
    """Scale the rows of t picked by the boolean index sel (a host mask over the
    leading axes it names) by factor, in t's own dtype."""
    torch = Hh.torch_mod()
    m = torch.ones(sel.shape, dtype=torch.float32)
    m[torch.from_numpy(sel)] = factor
    while m.dim() < t.dim():
        m = m.unsqueeze(-1)
    return (t.float() * m.to(t.device)).to(t.dtype).contiguous()


@pytest.mark.parametrize("name,lengths", [("deepseek_v2_decode", [700, 2100, 90]),
                                          ("qwen25_7b_decode", [1500, 333])])
def test_decode_restart_one_head(torch, name, lengths):
    """As the decode restart test, but every head's query except head 5 is scaled
    down 50x, so only head 5's scores pass the reference's headroom.  The lanes
    that see it are not the first lane of their wave, so this checks that the
    restart vote covers every lane."""
    import head_latent_attention_kv_amd as M
    cfg = I.CONFIGS[name]
    _print_case("decode_restart_one_head", cfg=name, lengths=lengths)
    layer = Hh.make_layer(cfg)
    run = Hh.build_decode(layer, np.array(lengths), key_boost=(40, 30.0))
    quiet = np.ones((len(lengths), cfg.n_heads), bool)
    quiet[:, 5] = False
    q_lat, q_pe = _quiet(run.q_lat, quiet), _quiet(run.q_pe, quiet)
    out = torch.empty_like(run.out)
    M.mla_decode(layer.dims, q_lat, q_pe, run.cache, torch.from_numpy(run.starts).cuda(),
                 torch.from_numpy(run.lengths.astype(np.int32)).cuda(), int(max(lengths)),
                 layer.w_dev["w_uv"], out)
    torch.cuda.synchronize()
    got, cache_h = Hh.to_host(out), Hh.to_host(run.cache)
    ql, qp = Hh.to_host(q_lat), Hh.to_host(q_pe)
    err = 0.0
    for b, n in enumerate(run.lengths):
        rows_gpu = cache_h[run.starts[b]:run.starts[b] + int(n)]
        ref = Hh.oracle_absorbed_rows(cfg, layer.w_host, ql[b], qp[b], rows_gpu)
        err = max(err, Hh.rel_err_rows(got[b], ref))
    print(f"{name} restart, head 5 only {lengths}: attn={err:.3e}")
    assert np.isfinite(got).all()
    assert err <= Hh.TOL[cfg.dtype], err


@pytest.mark.parametrize("order", ["expanded", "absorbed"])
def test_prefill_restart_not_first_lane(torch, order):
    """Hidden states from position 100 on are scaled 12x, so later tiles pass the
    first-tile reference of most queries by far more than either kernel's
    headroom; the queries the first lane of each wave holds are scaled down 50x
    (tokens t % 32 == 0 in the original order, head 0 in the absorbed order), so
    the restart must come from the other lanes' votes.  Reference: the oracle's
    attention definition on the operands the kernel reads."""
    import head_latent_attention_kv_amd as M
    from oracle import mla_oracle as O
    cfg = I.CONFIGS["long_prefill_131k"]
    lengths = [600, 300]
    _print_case("prefill_restart_not_first_lane", order=order, lengths=lengths)
    layer = Hh.make_layer(cfg)
    T = sum(lengths)
    xs = []
    for b, n in enumerate(lengths):
        xb = I.x_rows(cfg, b, 0, n, quantized=False)
        xb[100:] *= np.float32(12.0)
        xs.append(I.quantize(xb, cfg.dtype))
    x = np.concatenate(xs)
    pos = np.concatenate([np.arange(n) for n in lengths])
    seg = np.concatenate([np.full(n, b) for b, n in enumerate(lengths)])
    cache = torch.empty((T, cfg.row_width), dtype=torch.bfloat16, device="cuda")
    xd = Hh.to_dev(x, cfg.dtype)
    Hh.write_cache(layer, xd, pos, np.arange(T), cache)
    allowed = (seg[:, None] == seg[None, :]) & (pos[None, :] <= pos[:, None])
    c, kr = O.split_rows(Hh.to_host(cache), cfg.rank, cfg.n_groups, cfg.d_rope)
    if order == "expanded":
        q_nope, q_pe = Hh.query(layer, xd, pos)
        quiet = np.zeros((T, cfg.n_heads), bool)
        quiet[np.arange(T) % 32 == 0] = True
        q_nope, q_pe = _quiet(q_nope, quiet), _quiet(q_pe, quiet)
        out, ws = Hh.prefill_expanded(layer, q_nope, q_pe, cache, lengths)
        torch.cuda.synchronize()
        kn, v = Hh.expanded_kv(layer, ws, T)
        Q = np.concatenate([Hh.to_host(q_nope), Hh.to_host(q_pe)], axis=-1)
        K = np.concatenate([kn.transpose(1, 0, 2), np.repeat(kr, cfg.n_heads, 1)], axis=-1)
        ref = O.softmax_attention(Q, K, v.transpose(1, 0, 2), allowed, cfg.softmax_scale)
    else:
        q_lat, q_pe = Hh.absorb(layer, xd, pos)
        quiet = np.zeros((T, cfg.n_heads), bool)
        quiet[:, 0] = True
        q_lat, q_pe = _quiet(q_lat, quiet), _quiet(q_pe, quiet)
        out = torch.empty((T, cfg.n_heads, cfg.d_v), dtype=torch.bfloat16, device="cuda")
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int64, device="cuda")
        M.mla_prefill(layer.dims, q_lat, q_pe, cache, cu, max(lengths), layer.w_dev["w_uv"], out)
        torch.cuda.synchronize()
        Q = np.concatenate([Hh.to_host(q_lat), Hh.to_host(q_pe)], axis=-1)               # [T, H, r + dr]
        K = np.concatenate([c, kr[:, 0]], axis=-1)[:, None, :].repeat(cfg.n_heads, 1)
        o_lat = O.softmax_attention(Q, K, np.repeat(c[:, None, :], cfg.n_heads, 1), allowed, cfg.softmax_scale)
        ref = np.einsum("hvc,thc->thv", layer.w_host["w_uv"].astype(np.float64), o_lat)
    got = Hh.to_host(out)
    err = Hh.rel_err_rows(got, ref)
    print(f"prefill restart, first lanes quiet ({order}): attn {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= Hh.TOL["bf16"], err


# ----------------------------------------------------------------------------
# beyond the attention: the low-rank query path and the output projection
# ----------------------------------------------------------------------------


@pytest.mark.parametrize("name,T,q_rank", [("deepseek_v2_decode", 64, I.Q_LORA_RANK),
                                           ("deepseek_v2_decode", 300, I.Q_LORA_RANK),
                                           ("tiny_f32", 37, 96)])
def test_lowrank_query_matches_oracle(torch, name, T, q_rank):
    """mla_absorb_lowrank and mla_query_lowrank against the oracle's low-rank query
    (few tokens: weight-streaming projections; many: tiled GEMMs)."""
    import head_latent_attention_kv_amd as M
    from oracle import mla_oracle as O
    cfg = I.CONFIGS[name]
    _print_case("lowrank_query", cfg=name, T=T, q_rank=q_rank)
    layer = Hh.make_layer(cfg)
    lw = I.lowrank_query_weights(cfg, q_rank)
    lwd = {k: Hh.to_dev(v, cfg.dtype) for k, v in lw.items()}
    x = I.x_rows(cfg, 3, 0, T)
    pos = np.random.default_rng(11).integers(0, 50000, T)
    et = Hh.elem_dtype(cfg)
    xd = Hh.to_dev(x, cfg.dtype)
    posd = torch.from_numpy(pos.astype(np.int32)).cuda()
    q_lat = torch.empty((T, cfg.n_heads, cfg.rank), dtype=et, device="cuda")
    q_pe = torch.empty((T, cfg.n_heads, cfg.d_rope), dtype=et, device="cuda")
    q_nope = torch.empty((T, cfg.n_heads, cfg.d_nope), dtype=et, device="cuda")
    q_pe2 = torch.empty_like(q_pe)
    M.mla_absorb_lowrank(layer.dims, q_rank, xd, lwd["w_qa"], lwd["q_gain"], lwd["w_qb"], layer.w_dev["w_uk"],
                         posd, q_lat, q_pe)
    M.mla_query_lowrank(layer.dims, q_rank, xd, lwd["w_qa"], lwd["q_gain"], lwd["w_qb"], posd, q_nope, q_pe2)
    torch.cuda.synchronize()
    qn, qr = O.lowrank_query(x, lw["w_qa"], lw["q_gain"], lw["w_qb"], pos, n_heads=cfg.n_heads,
                             d_nope=cfg.d_nope, d_rope=cfg.d_rope, theta=cfg.rope_theta, eps=cfg.rms_eps)
    errs = {"q_lat": Hh.rel_err_rows(Hh.to_host(q_lat), O.absorbed_query(qn, layer.w_host["w_uk"])),
            "q_pe": Hh.rel_err_rows(Hh.to_host(q_pe), qr),
            "q_nope": Hh.rel_err_rows(Hh.to_host(q_nope), qn),
            "q_pe (query call)": Hh.rel_err_rows(Hh.to_host(q_pe2), qr)}
    print(f"{name} lowrank T={T}: " + " ".join(f"{k}={v:.3e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= Hh.TOL[cfg.dtype], (k, v)


@pytest.mark.parametrize("name,T", [("deepseek_v2_decode", 64), ("deepseek_v2_decode", 300),
                                    ("long_prefill_131k", 1000), ("tiny_f32", 17)])
def test_output_projection_matches_oracle(torch, name, T):
    """mla_output (u = o·W_oᵀ over all heads) against the oracle's eq. (3)/(6) product."""
    import head_latent_attention_kv_amd as M
    from oracle import mla_oracle as O
    cfg = I.CONFIGS[name]
    _print_case("output_projection", cfg=name, T=T)
    layer = Hh.make_layer(cfg)
    w_o = I.output_weight(cfg)
    o = I.draw_normal(cfg.seed, 40, (T,), (T, cfg.n_heads, cfg.d_v), 1.0, cfg.dtype)
    out = torch.empty((T, cfg.d_model), dtype=Hh.elem_dtype(cfg), device="cuda")
    M.mla_output(layer.dims, Hh.to_dev(o, cfg.dtype), Hh.to_dev(w_o, cfg.dtype), out)
    torch.cuda.synchronize()
    err = Hh.rel_err_rows(Hh.to_host(out), O.output_projection(o, w_o))
    print(f"{name} output projection T={T}: {err:.3e}")
    assert err <= Hh.TOL[cfg.dtype], err


# ----------------------------------------------------------------------------
# the DeepSeek-V4 / nanowhale variant
# ----------------------------------------------------------------------------


def _v4_setup(torch, cfg):
    import head_latent_attention_kv_amd as M
    w = I.v4_weights(cfg)
    wd = {k: (torch.from_numpy(v).cuda() if k == "sink" else Hh.to_dev(v, cfg.dtype)) for k, v in w.items()}
    return M.v4_dims_of(cfg), w, wd


def _v4_table(cfg):
    """A context-extension style frequency table: the lower half of the rotary
    frequencies divided by 32 (the Zebra page's YaRN factor), the rest unchanged."""
    f = cfg.rope_theta ** (-2.0 * np.arange(cfg.d_rope // 2) / cfg.d_rope)
    f[cfg.d_rope // 4:] /= 32.0
    return f


@pytest.mark.parametrize("lengths", [[700, 2048, 33, 1, 1500, 257]])
def test_v4_decode_chain(torch, lengths):
    """Cache rows, queries, decode with the sink and the inverse rotation, and the
    grouped output projection, against the oracle's V4 chain (nanowhale shape)."""
    import head_latent_attention_kv_amd as M
    from oracle import mla_oracle as O
    cfg = I.V4_CONFIGS["nanowhale_v4_decode"]
    _print_case("v4_decode", lengths=lengths)
    dims, w, wd = _v4_setup(torch, cfg)
    D, H = cfg.head_dim, cfg.n_heads
    lengths = np.array(lengths)
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]])
    rows = int(lengths.sum())
    cache = torch.empty((rows, D), dtype=torch.bfloat16, device="cuda")
    xs = [I.x_rows(cfg, b, 0, int(n)) for b, n in enumerate(lengths)]
    for b, n in enumerate(lengths):
        pos = torch.arange(int(n), dtype=torch.int32, device="cuda")
        slots = torch.arange(int(n), dtype=torch.int64, device="cuda") + int(starts[b])
        M.mla_v4_write_cache(dims, Hh.to_dev(xs[b], cfg.dtype), wd["w_kv"], wd["kv_gain"], pos, slots, cache)
    xq = np.stack([x[-1] for x in xs])
    q = torch.empty((len(lengths), H, D), dtype=torch.bfloat16, device="cuda")
    M.mla_v4_query(dims, Hh.to_dev(xq, cfg.dtype), wd["w_qa"], wd["q_gain"], wd["w_qb"],
                   torch.from_numpy((lengths - 1).astype(np.int32)).cuda(), q)
    out = torch.empty_like(q)
    M.mla_v4_decode(dims, q, cache, torch.from_numpy(starts.astype(np.int64)).cuda(),
                    torch.from_numpy(lengths.astype(np.int32)).cuda(), int(lengths.max()), wd["sink"], out)
    u = torch.empty((len(lengths), cfg.d_model), dtype=torch.bfloat16, device="cuda")
    M.mla_v4_output(dims, out, wd["w_oa"], wd["w_ob"], u)
    torch.cuda.synchronize()
    got, got_u = Hh.to_host(out), Hh.to_host(u)
    errs = []
    ref_all = []
    for b, n in enumerate(lengths):
        n = int(n)
        kv = O.v4_cache_rows(xs[b], w["w_kv"], w["kv_gain"], np.arange(n), d_rope=cfg.d_rope, eps=cfg.rms_eps)
        qr = O.v4_query(xs[b][-1:], w["w_qa"], w["q_gain"], w["w_qb"], [n - 1], n_heads=H, head_dim=D,
                        d_rope=cfg.d_rope, eps=cfg.rms_eps)
        ref = O.v4_attention(qr, kv, w["sink"], [n - 1], np.arange(n), [0], np.zeros(n, int),
                             cfg.softmax_scale, d_rope=cfg.d_rope)[0]
        ref_all.append(ref)
        errs.append(Hh.rel_err_rows(got[b], ref))
    err = max(errs)
    err_u = Hh.rel_err_rows(got_u, O.v4_output(got, w["w_oa"], w["w_ob"], cfg.o_groups))
    err_uc = Hh.rel_err_rows(got_u, O.v4_output(np.stack(ref_all), w["w_oa"], w["w_ob"], cfg.o_groups))
    print(f"v4 decode {list(lengths)}: attn chain {err:.3e}; output on gpu attn {err_u:.3e}, chain {err_uc:.3e}")
    assert err <= Hh.TOL["bf16"] and err_u <= Hh.TOL["bf16"] and err_uc <= Hh.TOL["bf16"]


def test_v4_full_size_sampled(torch):
    """The V4 bench's configuration: 256 sequences of 2048 cached rows decoded in one
    call (and the grouped output), and the causal prefill of the first 32 of them,
    checked on sampled sequences and query rows against the oracle's V4 chain."""
    import head_latent_attention_kv_amd as M
    from oracle import mla_oracle as O
    cfg = I.V4_CONFIGS["nanowhale_v4_decode"]
    B, L, D, H = cfg.batch, cfg.context, cfg.head_dim, cfg.n_heads
    _print_case("v4_full_size", batch=B, context=L)
    dims, w, wd = _v4_setup(torch, cfg)
    cache = torch.empty((B * L, D), dtype=torch.bfloat16, device="cuda")
    pos = torch.arange(L, dtype=torch.int32, device="cuda")
    xq = np.zeros((B, cfg.d_model), np.float32)
    seqs = [0, 97, 255]
    pf_b = 32
    xs = {}
    x_pf = []
    for b in range(B):
        xb = I.x_rows(cfg, b, 0, L)
        xq[b] = xb[-1]
        if b in seqs or b in (0, pf_b - 1):
            xs[b] = xb
        if b < pf_b:
            x_pf.append(xb)
        M.mla_v4_write_cache(dims, Hh.to_dev(xb, cfg.dtype), wd["w_kv"], wd["kv_gain"], pos,
                             torch.arange(L, dtype=torch.int64, device="cuda") + b * L, cache)
    starts = torch.arange(0, B * L, L, dtype=torch.int64, device="cuda")
    q = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
    M.mla_v4_query(dims, Hh.to_dev(xq, cfg.dtype), wd["w_qa"], wd["q_gain"], wd["w_qb"],
                   torch.full((B,), L - 1, dtype=torch.int32, device="cuda"), q)
    out = torch.empty_like(q)
    M.mla_v4_decode(dims, q, cache, starts, torch.full((B,), L, dtype=torch.int32, device="cuda"), L,
                    wd["sink"], out)
    u = torch.empty((B, cfg.d_model), dtype=torch.bfloat16, device="cuda")
    M.mla_v4_output(dims, out, wd["w_oa"], wd["w_ob"], u)
    # prefill of the first pf_b sequences, in one call
    q_pf = torch.empty((pf_b * L, H, D), dtype=torch.bfloat16, device="cuda")
    M.mla_v4_query(dims, Hh.to_dev(np.concatenate(x_pf), cfg.dtype), wd["w_qa"], wd["q_gain"], wd["w_qb"],
                   pos.repeat(pf_b), q_pf)
    out_pf = torch.empty_like(q_pf)
    M.mla_v4_prefill(dims, q_pf, cache, torch.arange(0, pf_b * L + 1, L, dtype=torch.int64, device="cuda"), L,
                     wd["sink"], out_pf)
    torch.cuda.synchronize()
    got, got_u = Hh.to_host(out), Hh.to_host(u)
    errs = {}
    kv_of = {}
    for b in sorted(xs):
        kv_of[b] = O.v4_cache_rows(xs[b], w["w_kv"], w["kv_gain"], np.arange(L), d_rope=cfg.d_rope, eps=cfg.rms_eps)
    for b in seqs:
        qr = O.v4_query(xs[b][-1:], w["w_qa"], w["q_gain"], w["w_qb"], [L - 1], n_heads=H, head_dim=D,
                        d_rope=cfg.d_rope, eps=cfg.rms_eps)
        ref = O.v4_attention(qr, kv_of[b], w["sink"], [L - 1], np.arange(L), [0], np.zeros(L, int),
                             cfg.softmax_scale, d_rope=cfg.d_rope)
        errs[f"decode seq {b}"] = Hh.rel_err_rows(got[b], ref[0])
        errs[f"output seq {b}"] = Hh.rel_err_rows(got_u[b:b + 1], O.v4_output(ref, w["w_oa"], w["w_ob"], cfg.o_groups))
    for b, rows in ((0, [0, 1, 1023, L - 1]), (pf_b - 1, [5, L - 1])):
        rows = np.array(rows)
        qr = O.v4_query(xs[b][rows], w["w_qa"], w["q_gain"], w["w_qb"], rows, n_heads=H, head_dim=D,
                        d_rope=cfg.d_rope, eps=cfg.rms_eps)
        ref = O.v4_attention(qr, kv_of[b], w["sink"], rows, np.arange(L), np.zeros(len(rows), int),
                             np.zeros(L, int), cfg.softmax_scale, d_rope=cfg.d_rope)
        got_pf = Hh.to_host(out_pf[torch.from_numpy(b * L + rows).cuda()])
        errs[f"prefill seq {b} rows {list(rows)}"] = Hh.rel_err_rows(got_pf, ref)
    print("v4 full size:", {k: f"{v:.3e}" for k, v in errs.items()})
    for k, e in errs.items():
        assert e <= Hh.TOL["bf16"], (k, e)


@pytest.mark.parametrize("table", [False, True])
def test_v4_prefill_ragged(torch, table):
    """Causal V4 prefill over a ragged batch (with the default rotary frequencies and
    with a caller's table), and the grouped output projection of many tokens."""
    import head_latent_attention_kv_amd as M
    from oracle import mla_oracle as O
    cfg = I.V4_CONFIGS["nanowhale_v4_decode"]
    lengths = [300, 1, 77]
    _print_case("v4_prefill", lengths=lengths, table=table)
    dims, w, wd = _v4_setup(torch, cfg)
    D, H = cfg.head_dim, cfg.n_heads
    f = _v4_table(cfg) if table else None
    fd = torch.from_numpy(f).cuda() if table else None
    T = sum(lengths)
    x = np.concatenate([I.x_rows(cfg, 10 + b, 0, n) for b, n in enumerate(lengths)])
    pos = np.concatenate([np.arange(n) for n in lengths])
    seg = np.concatenate([np.full(n, b) for b, n in enumerate(lengths)])
    xd = Hh.to_dev(x, cfg.dtype)
    posd = torch.from_numpy(pos.astype(np.int32)).cuda()
    cache = torch.empty((T, D), dtype=torch.bfloat16, device="cuda")
    M.mla_v4_write_cache(dims, xd, wd["w_kv"], wd["kv_gain"], posd, torch.arange(T, device="cuda"), cache,
                         rope_freqs=fd)
    q = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    M.mla_v4_query(dims, xd, wd["w_qa"], wd["q_gain"], wd["w_qb"], posd, q, rope_freqs=fd)
    out = torch.empty_like(q)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int64, device="cuda")
    M.mla_v4_prefill(dims, q, cache, cu, max(lengths), wd["sink"], out, rope_freqs=fd)
    u = torch.empty((T, cfg.d_model), dtype=torch.bfloat16, device="cuda")
    M.mla_v4_output(dims, out, wd["w_oa"], wd["w_ob"], u)
    torch.cuda.synchronize()
    kv = O.v4_cache_rows(x, w["w_kv"], w["kv_gain"], pos, d_rope=cfg.d_rope, eps=cfg.rms_eps, inv_freq=f)
    qr = O.v4_query(x, w["w_qa"], w["q_gain"], w["w_qb"], pos, n_heads=H, head_dim=D, d_rope=cfg.d_rope,
                    eps=cfg.rms_eps, inv_freq=f)
    ref = O.v4_attention(qr, kv, w["sink"], pos, pos, seg, seg, cfg.softmax_scale, d_rope=cfg.d_rope, inv_freq=f)
    got = Hh.to_host(out)
    err = Hh.rel_err_rows(got, ref)
    err_kv = Hh.rel_err_rows(Hh.to_host(cache), kv)
    err_u = Hh.rel_err_rows(Hh.to_host(u), O.v4_output(got, w["w_oa"], w["w_ob"], cfg.o_groups))
    print(f"v4 prefill {lengths} table={table}: attn chain {err:.3e}, cache rows {err_kv:.3e}, output {err_u:.3e}")
    for nm, e in (("attn", err), ("cache", err_kv), ("output", err_u)):
        assert e <= Hh.TOL["bf16"], (nm, e)


# ----------------------------------------------------------------------------
# ABI behaviour on the device
# ----------------------------------------------------------------------------


def test_abi_errors_leave_outputs_untouched(torch):
    import head_latent_attention_kv_amd as M
    cfg = I.small_variant(I.CONFIGS["deepseek_v2_decode"], d_model=256)
    layer = Hh.make_layer(cfg)
    B, L = 2, 100
    q_lat = torch.zeros((B, cfg.n_heads, cfg.rank), dtype=torch.bfloat16, device="cuda")
    q_pe = torch.zeros((B, cfg.n_heads, cfg.d_rope), dtype=torch.bfloat16, device="cuda")
    cache = torch.zeros((B * L, cfg.row_width), dtype=torch.bfloat16, device="cuda")
    out = torch.full((B, cfg.n_heads, cfg.d_v), 7.0, dtype=torch.bfloat16, device="cuda")
    ss = torch.tensor([0, L], dtype=torch.int64, device="cuda")
    sl = torch.tensor([L, L], dtype=torch.int32, device="cuda")
    need = M.mla_workspace_size(layer.dims, M.MLA_OP_DECODE, B, 0, L)
    small = torch.empty(max(0, need - 256), dtype=torch.uint8, device="cuda")
    with pytest.raises(M.MlaError) as e:
        M.mla_decode(layer.dims, q_lat, q_pe, cache, ss, sl, L, layer.w_dev["w_uv"], out, workspace=small)
    assert e.value.status == M.MLA_EWORKSPACE
    bad = M.make_dims(d_model=256, n_heads=128, n_groups=3, rank=512, d_rope=64, d_nope=128, d_v=128,
                      dtype="bf16")
    with pytest.raises(M.MlaError) as e:
        M.mla_decode(bad, q_lat, q_pe, cache, ss, sl, L, layer.w_dev["w_uv"], out)
    assert e.value.status == M.MLA_EINVAL
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


# ----------------------------------------------------------------------------
# full workload sizes, the launch configuration the benchmark times:
# sampled (sequence, head) outputs against the oracle, all outputs finite
# ----------------------------------------------------------------------------

_C4_LONGEST = int(np.argmax(I.context_lengths(I.CONFIGS["qwen3_30b_ragged_decode"])))
FULL_DECODE = [
    # name, {sampled sequence: its heads (None = all)}, sequences also checked end to end
    ("qwen25_7b_decode", {0: None, 13: None, 31: None}, [13]),
    # the benchmarked DeepSeek-V2 launch (64 x 8192, 4 splits of 2048 rows):
    # every head of the first and the last sequence, the last one also as a chain
    ("deepseek_v2_decode", {0: None, 21: [0, 37, 64, 127], 42: [5, 50, 99, 120], 63: None}, [63]),
    ("qwen3_30b_ragged_decode", {b: (None if b == _C4_LONGEST else [0, 9, 17, 31]) for b in range(8)},
     [_C4_LONGEST]),
]


@pytest.mark.parametrize("name,seq_heads,chain_seqs", FULL_DECODE)
def test_decode_full_size_sampled(torch, name, seq_heads, chain_seqs):
    from oracle import mla_oracle as O
    cfg = I.CONFIGS[name]
    lengths = I.context_lengths(cfg)
    _print_case("decode_full", cfg=name, batch=len(lengths), max_len=int(lengths.max()))
    layer = Hh.make_layer(cfg)
    run = Hh.build_decode(layer, lengths)
    assert bool(torch.isfinite(run.out.float()).all())
    got = Hh.to_host(run.out)
    w = layer.w_host
    worst = {"write": 0.0, "attn": 0.0, "chain": 0.0}
    for b, heads in seq_heads.items():
        n = int(lengths[b])
        hs = list(range(cfg.n_heads)) if heads is None else list(heads)
        rows_gpu = Hh.to_host(run.cache[int(run.starts[b]):int(run.starts[b]) + n])
        ref = Hh.oracle_decode_rows(cfg, w, None, run.x_query[b], n, cache_rows=rows_gpu, heads=hs)
        e = Hh.rel_err_rows(got[b, hs], ref)
        worst["attn"] = max(worst["attn"], e)
        if b in chain_seqs:
            xb = I.x_rows(cfg, b, 0, n)
            rows_ref = O.cache_rows(xb, w["w_dkv"], w["w_kr"], np.arange(n), n_groups=cfg.n_groups,
                                    d_rope=cfg.d_rope, theta=cfg.rope_theta,
                                    latent_rmsnorm=cfg.latent_rmsnorm, eps=cfg.rms_eps)
            worst["write"] = max(worst["write"], Hh.write_err(cfg, rows_gpu, rows_ref))
            ref_c = Hh.oracle_decode_rows(cfg, w, xb, run.x_query[b], n, cache_rows=rows_ref, heads=hs)
            worst["chain"] = max(worst["chain"], Hh.rel_err_rows(got[b, hs], ref_c))
        errs_h = [O.max_rel_err(got[b, h], ref[i]) for i, h in enumerate(hs)]
        worst_h = hs[int(np.argmax(errs_h))] if hs else -1
        print(f"  seq {b} (n={n}, {len(hs)} heads): attn max {e:.3e} (worst head {worst_h}); "
              f"per-head max errors {' '.join(f'{v:.1e}' for v in errs_h[:8])}{' ...' if len(hs) > 8 else ''}",
              flush=True)
    print(f"{name} full size: " + " ".join(f"{k}={v:.3e}" for k, v in worst.items()))
    for k, v in worst.items():
        assert v <= Hh.TOL[cfg.dtype], (k, v)
