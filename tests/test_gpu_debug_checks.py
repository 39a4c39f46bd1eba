"""The debug build (MLA_DEBUG_CHECKS): decode, prefill and cache-write calls copy
their index arrays to the host and refuse out-of-range ones before any launch;
in-range calls give the release build's results bit for bit."""
import ctypes

import numpy as np
import pytest

import mla_inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    import head_latent_attention_kv_amd as M
    from head_latent_attention_kv_amd import _abi, build
    M.load()
    assert torch.cuda.is_available()
    return torch, M, _abi.load(), _abi.load(build.lib_path("debug"))


def _stream(torch):
    return torch.cuda.current_stream().cuda_stream


def test_debug_build_refuses_bad_index_arrays(env):
    torch, M, rel, dbg = env
    cfg = I.CONFIGS["qwen25_7b_decode"]
    dims = M.dims_of(cfg)
    g = torch.Generator(device="cuda").manual_seed(5)
    bf = torch.bfloat16
    lengths = np.array([300, 17, 1024], np.int64)
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)
    B, max_len, rows = 3, 1024, int(lengths.sum())
    cache = torch.randn((rows, cfg.row_width), generator=g, device="cuda").to(bf)
    q_lat = (torch.randn((B, cfg.n_heads, cfg.rank), generator=g, device="cuda") * 0.1).to(bf)
    q_pe = (torch.randn((B, cfg.n_heads, cfg.d_rope), generator=g, device="cuda") * 0.1).to(bf)
    w_uv = (torch.randn((cfg.n_heads, cfg.d_v, cfg.rank), generator=g, device="cuda") / cfg.rank ** 0.5).to(bf)
    ss = torch.from_numpy(starts).cuda()
    need = M.mla_workspace_size(dims, M.MLA_OP_DECODE, B, 0, max_len)
    ws = torch.empty(max(256, need), dtype=torch.uint8, device="cuda")

    def decode(lib, seq_len, out):
        return lib.mla_decode(ctypes.byref(dims), q_lat.data_ptr(), q_pe.data_ptr(), cache.data_ptr(), ss.data_ptr(),
                              seq_len.data_ptr(), B, max_len, w_uv.data_ptr(), out.data_ptr(), ws.data_ptr(),
                              ws.numel(), _stream(torch))

    good = torch.from_numpy(lengths.astype(np.int32)).cuda()
    ref = torch.empty((B, cfg.n_heads, cfg.d_v), dtype=bf, device="cuda")
    got = torch.empty_like(ref)
    assert decode(rel, good, ref) == M.MLA_OK
    assert decode(dbg, good, got) == M.MLA_OK
    torch.cuda.synchronize()
    assert torch.equal(ref, got)
    for bad in ([300, 17, 1025], [300, 0, 1024]):  # above max_len; an empty context
        out = torch.full_like(ref, 7.0)
        assert decode(dbg, torch.tensor(bad, dtype=torch.int32, device="cuda"), out) == M.MLA_EINVAL, bad
        torch.cuda.synchronize()
        assert bool((out == 7.0).all())
    # prefill: segment offsets that do not end at n_tokens
    T = 64
    ql = torch.zeros((T, cfg.n_heads, cfg.rank), dtype=bf, device="cuda")
    qp = torch.zeros((T, cfg.n_heads, cfg.d_rope), dtype=bf, device="cuda")
    out_p = torch.full((T, cfg.n_heads, cfg.d_v), 7.0, dtype=bf, device="cuda")
    wsp = torch.empty(max(256, M.mla_workspace_size(dims, M.MLA_OP_PREFILL, 1, T, T)), dtype=torch.uint8, device="cuda")
    for cu, want in (([0, 64], M.MLA_OK), ([0, 63], M.MLA_EINVAL), ([1, 64], M.MLA_EINVAL)):
        cu_t = torch.tensor(cu, dtype=torch.int64, device="cuda")
        st = dbg.mla_prefill(ctypes.byref(dims), ql.data_ptr(), qp.data_ptr(), cache.data_ptr(), cu_t.data_ptr(), 1, T,
                             T, w_uv.data_ptr(), out_p.data_ptr(), wsp.data_ptr(), wsp.numel(), _stream(torch))
        assert st == want, cu
    # cache write: a slot past the cache, and one slot twice
    x = torch.zeros((2, cfg.d_model), dtype=bf, device="cuda")
    w_dkv = torch.zeros((cfg.rank, cfg.d_model), dtype=bf, device="cuda")
    w_kr = torch.zeros((cfg.n_groups * cfg.d_rope, cfg.d_model), dtype=bf, device="cuda")
    pos = torch.zeros(2, dtype=torch.int32, device="cuda")
    wsw = torch.empty(max(256, M.mla_workspace_size(dims, M.MLA_OP_WRITE_CACHE, 0, 2, 0)), dtype=torch.uint8,
                      device="cuda")
    before = cache.clone()
    for slots in ([rows, 0], [5, 5]):
        sl = torch.tensor(slots, dtype=torch.int64, device="cuda")
        st = dbg.mla_write_cache(ctypes.byref(dims), x.data_ptr(), w_dkv.data_ptr(), w_kr.data_ptr(), pos.data_ptr(),
                                 sl.data_ptr(), 2, cache.data_ptr(), rows, wsw.data_ptr(), wsw.numel(), _stream(torch))
        assert st == M.MLA_EINVAL, slots
    torch.cuda.synchronize()
    assert torch.equal(cache, before)
