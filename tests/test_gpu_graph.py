"""The library's calls captured into a HIP graph (torch.cuda.CUDAGraph on the
launch stream) and replayed.  Each call launches kernels only (no memset, copy or
allocation when the caller passes the workspace), so a replay must reproduce the
eager result bit for bit.  Every replay is checked, with eager work and
synchronisations between the replays, and the outputs are cleared before each
replay so a replay that did nothing cannot pass."""
import numpy as np
import pytest

import mla_inputs as I
from tests import harness as Hh

pytestmark = pytest.mark.gpu

N_REPLAYS = 3


@pytest.fixture(scope="module")
def torch():
    import torch
    import head_latent_attention_kv_amd as M
    M.load()
    assert torch.cuda.is_available()
    return torch


def _capture(torch, fn):
    """fn() once on a side stream, then captured into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replay_and_check(torch, g, outputs, expected, eager_noise):
    for k in range(N_REPLAYS):
        for t in outputs:
            t.zero_()
        eager_noise(k)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t, e in zip(expected, outputs, expected.values()):
            assert torch.equal(t, e), f"replay {k}: {name} differs from the eager result"
        print(f"  replay {k}: outputs identical to the eager run", flush=True)


def test_tiny_f32_run_in_a_graph(torch):
    """The fp32 layer's whole run (prefill of 256 tokens, then 16 decode steps of
    write + absorb + decode) as one graph."""
    import head_latent_attention_kv_amd as M
    from oracle import mla_oracle as O
    cfg = I.CONFIGS["tiny_f32"]
    print(f"[case] graph tiny_f32 L={cfg.prefill_len} steps={cfg.decode_steps}", flush=True)
    layer = Hh.make_layer(cfg)
    L, S = cfg.prefill_len, cfg.decode_steps
    n_all = L + S
    f32 = torch.float32
    xh = I.x_rows(cfg, 0, 0, n_all)
    x = Hh.to_dev(xh, cfg.dtype)
    dims, wd = layer.dims, layer.w_dev
    cache = torch.zeros((n_all, cfg.row_width), dtype=f32, device="cuda")
    q_lat = torch.zeros((n_all, cfg.n_heads, cfg.rank), dtype=f32, device="cuda")
    q_pe = torch.zeros((n_all, cfg.n_heads, cfg.d_rope), dtype=f32, device="cuda")
    out_pre = torch.zeros((L, cfg.n_heads, cfg.d_v), dtype=f32, device="cuda")
    out_dec = torch.zeros((S, cfg.n_heads, cfg.d_v), dtype=f32, device="cuda")
    pos = torch.arange(n_all, dtype=torch.int32, device="cuda")
    slots = torch.arange(n_all, dtype=torch.int64, device="cuda")
    cu = torch.tensor([0, L], dtype=torch.int64, device="cuda")
    seq_start = torch.zeros(1, dtype=torch.int64, device="cuda")
    seq_lens = [torch.tensor([L + s + 1], dtype=torch.int32, device="cuda") for s in range(S)]
    pos_1 = [torch.tensor([L + s], dtype=torch.int32, device="cuda") for s in range(S)]
    slot_1 = [torch.tensor([L + s], dtype=torch.int64, device="cuda") for s in range(S)]
    ws = {op: torch.empty(max(256, M.mla_workspace_size(dims, op, b, t, m)), dtype=torch.uint8, device="cuda")
          for op, b, t, m in ((M.MLA_OP_WRITE_CACHE, 0, L, 0), (M.MLA_OP_ABSORB, 0, L, 0),
                              (M.MLA_OP_PREFILL, 1, L, L), (M.MLA_OP_DECODE, 1, 0, n_all))}

    def run():
        M.mla_write_cache(dims, x[:L], wd["w_dkv"], wd["w_kr"], pos[:L], slots[:L], cache,
                          workspace=ws[M.MLA_OP_WRITE_CACHE])
        M.mla_absorb(dims, x[:L], wd["w_qc"], wd["w_qr"], wd["w_uk"], pos[:L], q_lat[:L], q_pe[:L],
                     workspace=ws[M.MLA_OP_ABSORB])
        M.mla_prefill(dims, q_lat[:L], q_pe[:L], cache, cu, L, wd["w_uv"], out_pre, workspace=ws[M.MLA_OP_PREFILL])
        for s in range(S):
            p = L + s
            M.mla_write_cache(dims, x[p:p + 1], wd["w_dkv"], wd["w_kr"], pos_1[s], slot_1[s], cache,
                              workspace=ws[M.MLA_OP_WRITE_CACHE])
            M.mla_absorb(dims, x[p:p + 1], wd["w_qc"], wd["w_qr"], wd["w_uk"], pos_1[s], q_lat[p:p + 1],
                         q_pe[p:p + 1], workspace=ws[M.MLA_OP_ABSORB])
            M.mla_decode(dims, q_lat[p:p + 1], q_pe[p:p + 1], cache, seq_start, seq_lens[s], p + 1, wd["w_uv"],
                         out_dec[s:s + 1], workspace=ws[M.MLA_OP_DECODE])

    run()
    torch.cuda.synchronize()
    expected = {"cache": cache.clone(), "q_lat": q_lat.clone(), "q_pe": q_pe.clone(),
                "out_pre": out_pre.clone(), "out_dec": out_dec.clone()}
    # the eager result against the oracle (the same check as the chain test)
    got = np.concatenate([Hh.to_host(out_pre), Hh.to_host(out_dec)])
    p = np.arange(n_all)
    ref = O.mla_layer(xh, xh, layer.w_host, k_pos=p, q_pos=p, k_seg=np.zeros(n_all, int), q_seg=np.zeros(n_all, int),
                      n_heads=cfg.n_heads, n_groups=cfg.n_groups, d_nope=cfg.d_nope, d_rope=cfg.d_rope,
                      theta=cfg.rope_theta, scale=cfg.softmax_scale)
    err = Hh.rel_err_rows(got, ref)
    print(f"  eager run max rel err {err:.3e}", flush=True)
    assert err <= Hh.TOL["f32"]

    g = _capture(torch, run)
    noise_src = torch.randn(1 << 16, device="cuda")

    def eager_noise(k):
        # unrelated eager work between replays, including a reduction over many blocks
        _ = (noise_src * (k + 1)).sum().item()

    _replay_and_check(torch, g, [cache, q_lat, q_pe, out_pre, out_dec], expected, eager_noise)


@pytest.mark.parametrize("name,lengths,tiled", [("deepseek_v2_decode", [1, 300, 2048, 4100], False),
                                                ("deepseek_v2_decode", [1, 300, 2048, 4100], True),
                                                ("qwen3_30b_ragged_decode", [33, 1537], False),
                                                ("qwen3_30b_ragged_decode", [1, 40, 3000, 9000, 20000], True)])
def test_decode_step_in_a_graph(torch, name, lengths, tiled):
    """One bf16 decode step (write the batch's new rows, absorb, decode) as a graph;
    tiled: the absorption reads [W_QC ; W_QR] tiled (mla_absorb_tiled)."""
    import head_latent_attention_kv_amd as M
    cfg = I.CONFIGS[name]
    print(f"[case] graph decode step {name} lengths={lengths} tiled={tiled}", flush=True)
    layer = Hh.make_layer(cfg)
    lengths = np.asarray(lengths, np.int64)
    run = Hh.build_decode(layer, lengths)
    dims, wd = layer.dims, layer.w_dev
    B = len(lengths)
    max_len = int(lengths.max())
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)
    # the step's new rows are the last row of each sequence
    xd = Hh.to_dev(run.x_query, cfg.dtype)
    pos = torch.from_numpy((lengths - 1).astype(np.int32)).cuda()
    slots = torch.from_numpy(starts + lengths - 1).cuda()
    ss = torch.from_numpy(starts).cuda()
    sl = torch.from_numpy(lengths.astype(np.int32)).cuda()
    cache = run.cache
    et = torch.bfloat16
    q_lat = torch.zeros((B, cfg.n_heads, cfg.rank), dtype=et, device="cuda")
    q_pe = torch.zeros((B, cfg.n_heads, cfg.d_rope), dtype=et, device="cuda")
    out = torch.zeros((B, cfg.n_heads, cfg.d_v), dtype=et, device="cuda")
    ws_w = torch.empty(max(256, M.mla_workspace_size(dims, M.MLA_OP_WRITE_CACHE, 0, B, 0)), dtype=torch.uint8,
                       device="cuda")
    ws_a = torch.empty(max(256, M.mla_workspace_size(dims, M.MLA_OP_ABSORB, 0, B, 0)), dtype=torch.uint8,
                       device="cuda")
    ws_d = torch.empty(max(256, M.mla_workspace_size(dims, M.MLA_OP_DECODE, B, 0, max_len)), dtype=torch.uint8,
                       device="cuda")

    wq_t = M.mla_tile_weights(wd["w_qc"], wd["w_qr"]) if tiled else None

    def step():
        M.mla_write_cache(dims, xd, wd["w_dkv"], wd["w_kr"], pos, slots, cache, workspace=ws_w)
        if tiled:
            M.mla_absorb_tiled(dims, xd, wq_t, wd["w_uk"], pos, q_lat, q_pe, workspace=ws_a)
        else:
            M.mla_absorb(dims, xd, wd["w_qc"], wd["w_qr"], wd["w_uk"], pos, q_lat, q_pe, workspace=ws_a)
        M.mla_decode(dims, q_lat, q_pe, cache, ss, sl, max_len, wd["w_uv"], out, workspace=ws_d)

    step()
    torch.cuda.synchronize()
    expected = {"q_lat": q_lat.clone(), "q_pe": q_pe.clone(), "out": out.clone()}
    new_rows = cache[slots].clone()
    g = _capture(torch, step)

    def eager_noise(k):
        # the same calls eagerly on other outputs, then a reduction over many blocks
        q2, p2 = torch.empty_like(q_lat), torch.empty_like(q_pe)
        M.mla_absorb(dims, xd, wd["w_qc"], wd["w_qr"], wd["w_uk"], pos, q2, p2, workspace=ws_a)
        _ = q2.float().abs().sum().item()

    _replay_and_check(torch, g, [q_lat, q_pe, out], expected, eager_noise)
    assert torch.equal(cache[slots], new_rows), "the replayed cache write differs from the eager one"
