"""mla_decode_noalloc (partials in the library's static scratch array) against
mla_decode (partials in a caller workspace prefilled with NaN bytes), on
consecutive calls of decreasing size, so neither a partial the kernels fail to
write nor the previous call's leftovers in the shared array can pass unseen.
The two entry points run the same kernels with the same split plan, so the
outputs must agree bit for bit."""
import numpy as np
import pytest

import mla_inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch
    import head_latent_attention_kv_amd as M
    M.load()
    assert torch.cuda.is_available()
    return torch


def _case(torch, M, cfg_name, lengths, seed):
    cfg = I.CONFIGS[cfg_name]
    dims = M.dims_of(cfg)
    g = torch.Generator(device="cuda").manual_seed(seed)
    lengths = np.asarray(lengths, np.int64)
    B, max_len = len(lengths), int(lengths.max())
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)
    bf = torch.bfloat16
    cache = torch.randn((int(lengths.sum()), cfg.row_width), generator=g, device="cuda").to(bf)
    q_lat = (torch.randn((B, cfg.n_heads, cfg.rank), generator=g, device="cuda") * 0.05).to(bf)
    q_pe = (torch.randn((B, cfg.n_heads, cfg.d_rope), generator=g, device="cuda") * 0.05).to(bf)
    w_uv = (torch.randn((cfg.n_heads, cfg.d_v, cfg.rank), generator=g, device="cuda") / cfg.rank ** 0.5).to(bf)
    ss = torch.from_numpy(starts).cuda()
    sl = torch.from_numpy(lengths.astype(np.int32)).cuda()
    need = M.mla_workspace_size(dims, M.MLA_OP_DECODE, B, 0, max_len)
    assert 0 < need <= M.MLA_NOALLOC_SCRATCH_BYTES
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")  # NaN in bf16 and fp32
    ref = torch.empty((B, cfg.n_heads, cfg.d_v), dtype=bf, device="cuda")
    got = torch.empty_like(ref)
    M.mla_decode(dims, q_lat, q_pe, cache, ss, sl, max_len, w_uv, ref, workspace=ws)
    M.mla_decode_noalloc(dims, q_lat, q_pe, cache, ss, sl, max_len, w_uv, got)
    torch.cuda.synchronize()
    return ref, got, M.mla_decode_splits(dims, B, max_len)


def test_noalloc_decode_matches_workspace_decode(torch):
    import head_latent_attention_kv_amd as M
    cases = [
        # the DeepSeek-V2 benchmark launch: 64 x 8192 rows, 4 splits (50.6 MB of scratch)
        ("deepseek_v2_decode", [8192] * 64, 11),
        # smaller and ragged, right after it: fewer sequences and splits than the call before
        ("deepseek_v2_decode", [1, 300, 2048, 4097, 777], 12),
        # the grouped-rotary kernel (Qwen3-30B shape), smaller again
        ("qwen3_30b_ragged_decode", [1024, 1537, 33], 13),
    ]
    for name, lengths, seed in cases:
        print(f"[case] noalloc {name} batch={len(lengths)} max_len={max(lengths)}", flush=True)
        ref, got, ns = _case(torch, M, name, lengths, seed)
        assert bool(torch.isfinite(ref.float()).all()), name
        same = torch.equal(got, ref)
        print(f"  {ns} splits: outputs {'identical' if same else 'DIFFER'}", flush=True)
        assert same, (name, lengths)


def test_noalloc_decode_refuses_oversize(torch):
    import head_latent_attention_kv_amd as M
    cfg = I.CONFIGS["deepseek_v2_decode"]
    dims = M.dims_of(cfg)
    B = 300  # one split, 78.6 MB of fp32 o_ > 64 MiB
    t = torch.zeros((B, cfg.n_heads, cfg.rank), dtype=torch.bfloat16, device="cuda")
    pe = torch.zeros((B, cfg.n_heads, cfg.d_rope), dtype=torch.bfloat16, device="cuda")
    out = torch.full((B, cfg.n_heads, cfg.d_v), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(M.MlaError) as e:
        M.mla_decode_noalloc(dims, t, pe, torch.zeros((16, cfg.row_width), dtype=torch.bfloat16, device="cuda"),
                             torch.zeros(B, dtype=torch.int64, device="cuda"),
                             torch.ones(B, dtype=torch.int32, device="cuda"), 8192,
                             torch.zeros((cfg.n_heads, cfg.d_v, cfg.rank), dtype=torch.bfloat16, device="cuda"), out)
    assert e.value.status == M.MLA_ESCRATCH
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())  # refused before any launch: the output is untouched
