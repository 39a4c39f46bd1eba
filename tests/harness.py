"""Shared test plumbing: the GPU chain through the C ABI on seeded inputs, and the
oracle on the same inputs.  Test infrastructure only."""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np

import mla_inputs as I
from mla_inputs.device import device_weights, raw_to_dev, to_dev  # noqa: F401  (used by the tests)
from oracle import mla_oracle as O

TOL = {"bf16": 1e-2, "f32": 1e-4}  # max relative error per (token, head), over d_v


def torch_mod():
    import torch
    return torch


def to_host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def elem_dtype(cfg):
    torch = torch_mod()
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


@dataclasses.dataclass
class DeviceLayer:
    cfg: I.MLAConfig
    w_host: Dict[str, np.ndarray]
    w_dev: Dict[str, object]
    dims: object


def make_layer(cfg: I.MLAConfig, device="cuda") -> DeviceLayer:
    import head_latent_attention_kv_amd as M
    w, wd = device_weights(cfg, device)
    return DeviceLayer(cfg, w, wd, M.dims_of(cfg))


def write_cache(layer: DeviceLayer, x_dev, positions: np.ndarray, slots: np.ndarray, cache,
                workspace=None):
    import head_latent_attention_kv_amd as M
    torch = torch_mod()
    pos = torch.from_numpy(positions.astype(np.int32)).to(cache.device)
    sl = torch.from_numpy(slots.astype(np.int64)).to(cache.device)
    M.mla_write_cache(layer.dims, x_dev, layer.w_dev["w_dkv"], layer.w_dev["w_kr"], pos, sl, cache,
                      workspace=workspace)


def absorb(layer: DeviceLayer, x_dev, positions: np.ndarray):
    import head_latent_attention_kv_amd as M
    torch = torch_mod()
    cfg = layer.cfg
    T = x_dev.shape[0]
    q_lat = torch.empty((T, cfg.n_heads, cfg.rank), dtype=elem_dtype(cfg), device=x_dev.device)
    q_pe = torch.empty((T, cfg.n_heads, cfg.d_rope), dtype=elem_dtype(cfg), device=x_dev.device)
    pos = torch.from_numpy(positions.astype(np.int32)).to(x_dev.device)
    M.mla_absorb(layer.dims, x_dev, layer.w_dev["w_qc"], layer.w_dev["w_qr"], layer.w_dev["w_uk"],
                 pos, q_lat, q_pe)
    return q_lat, q_pe


def query(layer: DeviceLayer, x_dev, positions: np.ndarray):
    """mla_query: q_nope [T, H, d_nope] and q_pe [T, H, d_rope] without absorption."""
    import head_latent_attention_kv_amd as M
    torch = torch_mod()
    cfg = layer.cfg
    T = x_dev.shape[0]
    q_nope = torch.empty((T, cfg.n_heads, cfg.d_nope), dtype=elem_dtype(cfg), device=x_dev.device)
    q_pe = torch.empty((T, cfg.n_heads, cfg.d_rope), dtype=elem_dtype(cfg), device=x_dev.device)
    pos = torch.from_numpy(positions.astype(np.int32)).to(x_dev.device)
    M.mla_query(layer.dims, x_dev, layer.w_dev["w_qc"], layer.w_dev["w_qr"], pos, q_nope, q_pe)
    return q_nope, q_pe


def prefill_expanded(layer: DeviceLayer, q_nope, q_pe, cache, lengths):
    """mla_prefill_expanded over packed sequences of the given lengths; returns the
    output and the workspace (k_nope [H, T, d_nope] then v [H, T, d_v], fp16)."""
    import head_latent_attention_kv_amd as M
    torch = torch_mod()
    cfg = layer.cfg
    T = q_nope.shape[0]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int64, device="cuda")
    need = M.mla_workspace_size(layer.dims, M.MLA_OP_PREFILL_EXPANDED, len(lengths), T, int(max(lengths)))
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, cfg.n_heads, cfg.d_v), dtype=elem_dtype(cfg), device="cuda")
    M.mla_prefill_expanded(layer.dims, q_nope, q_pe, cache, cu, int(max(lengths)), layer.w_dev["w_uk"],
                           layer.w_dev["w_uv"], out, workspace=ws)
    return out, ws


def expanded_kv(layer: DeviceLayer, ws, T: int):
    """The fp16 k_nope [H, T, d_nope] and v [H, T, d_v] an mla_prefill_expanded call
    left in its workspace, as host arrays.  The workspace holds k_nope [H, T, d_nope]
    and then vᵀ [H, d_v, T_pad] (T rounded up to 32, the pad columns zero); the pad
    is checked to be zero here."""
    torch = torch_mod()
    cfg = layer.cfg
    nk = cfg.n_heads * T * cfg.d_nope
    k_bytes = (nk * 2 + 255) // 256 * 256
    t_pad = (T + 31) // 32 * 32
    k = ws[:nk * 2].view(torch.float16).view(cfg.n_heads, T, cfg.d_nope)
    vt = ws[k_bytes:k_bytes + cfg.n_heads * cfg.d_v * t_pad * 2].view(torch.float16)
    vt = to_host(vt.view(cfg.n_heads, cfg.d_v, t_pad))
    assert not vt[:, :, T:].any(), "vᵀ pad columns not zero"
    return to_host(k), np.ascontiguousarray(vt[:, :, :T].transpose(0, 2, 1))


@dataclasses.dataclass
class DecodeRun:
    lengths: np.ndarray
    starts: np.ndarray
    cache: object
    q_lat: object
    q_pe: object
    out: object
    x_query: np.ndarray  # [B, d_model] float32 (representable values)


def key_rows(cfg, b: int, c0: int, c1: int, n: int, x_scale: float = 1.0,
             key_boost: Optional[Tuple[int, float]] = None) -> np.ndarray:
    """Unrounded hidden states of rows [c0, c1) of sequence b (length n).  With
    key_boost = (p0, f), rows at positions p0 <= p < n - 1 are multiplied by f
    (the query row n - 1 is not), so later keys score far above the first ones."""
    x = I.x_rows(cfg, b, c0, c1, scale=x_scale, quantized=False)
    if key_boost is not None:
        p0, f = key_boost
        pos = np.arange(c0, c1)
        x = np.where(((pos >= p0) & (pos < n - 1))[:, None], x * np.float32(f), x).astype(np.float32)
    return x


def build_decode(layer: DeviceLayer, lengths: np.ndarray, x_scale: float = 1.0,
                 chunk: int = 8192, threads: int = 8,
                 key_boost: Optional[Tuple[int, float]] = None) -> DecodeRun:
    """Fill a packed cache for sequences of the given lengths with mla_write_cache,
    absorb each sequence's last token, run mla_decode."""
    import concurrent.futures as cf

    import head_latent_attention_kv_amd as M
    torch = torch_mod()
    cfg = layer.cfg
    lengths = np.asarray(lengths, np.int64)
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)
    rows = int(lengths.sum())
    cache = torch.empty((rows, cfg.row_width), dtype=elem_dtype(cfg), device="cuda")
    ws = torch.empty(max(256, M.mla_workspace_size(layer.dims, M.MLA_OP_WRITE_CACHE, 0, chunk, 0)),
                     dtype=torch.uint8, device="cuda")
    xq = np.zeros((len(lengths), cfg.d_model), np.float32)
    jobs = [(b, c0, min(int(n), c0 + chunk)) for b, n in enumerate(lengths) for c0 in range(0, int(n), chunk)]

    def gen(job):
        b, c0, c1 = job
        return job, key_rows(cfg, b, c0, c1, int(lengths[b]), x_scale, key_boost)

    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        for (b, c0, c1), xb in ex.map(gen, jobs):
            if c1 == lengths[b]:
                xq[b] = I.quantize(xb[-1:], cfg.dtype)[0]
            write_cache(layer, raw_to_dev(xb, cfg.dtype), np.arange(c0, c1),
                        starts[b] + np.arange(c0, c1), cache, workspace=ws)
    q_lat, q_pe = absorb(layer, to_dev(xq, cfg.dtype), lengths - 1)
    out = torch.empty((len(lengths), cfg.n_heads, cfg.d_v), dtype=elem_dtype(cfg), device="cuda")
    seq_start = torch.from_numpy(starts).cuda()
    seq_len = torch.from_numpy(lengths.astype(np.int32)).cuda()
    M.mla_decode(layer.dims, q_lat, q_pe, cache, seq_start, seq_len, int(lengths.max()),
                 layer.w_dev["w_uv"], out)
    torch.cuda.synchronize()
    return DecodeRun(lengths, starts, cache, q_lat, q_pe, out, xq)


@dataclasses.dataclass
class PrefillRun:
    x_q: np.ndarray        # the bf16-exact hidden states (float32) the GPU received
    cache: object          # device [L, row_width]
    q_lat: object          # device [L, H, r]
    q_pe: object           # device [L, H, d_rope]
    out: object            # device [L, H, d_v]


def build_prefill(layer: DeviceLayer, L: int, chunk: int = 8192, threads: int = 8) -> PrefillRun:
    """One sequence of L tokens: cache rows and queries from seeded x (written and
    absorbed in chunks of ``chunk`` tokens), then one causal mla_prefill call."""
    import concurrent.futures as cf

    import head_latent_attention_kv_amd as M
    torch = torch_mod()
    cfg = layer.cfg
    et = elem_dtype(cfg)
    cache = torch.empty((L, cfg.row_width), dtype=et, device="cuda")
    q_lat = torch.empty((L, cfg.n_heads, cfg.rank), dtype=et, device="cuda")
    q_pe = torch.empty((L, cfg.n_heads, cfg.d_rope), dtype=et, device="cuda")
    x_q = np.empty((L, cfg.d_model), np.float32)
    ws_w = torch.empty(max(256, M.mla_workspace_size(layer.dims, M.MLA_OP_WRITE_CACHE, 0, chunk, 0)),
                       dtype=torch.uint8, device="cuda")
    ws_a = torch.empty(max(256, M.mla_workspace_size(layer.dims, M.MLA_OP_ABSORB, 0, chunk, 0)),
                       dtype=torch.uint8, device="cuda")
    jobs = [(c0, min(L, c0 + chunk)) for c0 in range(0, L, chunk)]

    def gen(job):
        c0, c1 = job
        return job, I.x_rows(cfg, 0, c0, c1, quantized=False)

    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        for (c0, c1), xb in ex.map(gen, jobs):
            x_q[c0:c1] = I.quantize(xb, cfg.dtype)
            xd = raw_to_dev(xb, cfg.dtype)
            pos = np.arange(c0, c1)
            write_cache(layer, xd, pos, pos, cache, workspace=ws_w)
            M.mla_absorb(layer.dims, xd, layer.w_dev["w_qc"], layer.w_dev["w_qr"], layer.w_dev["w_uk"],
                         torch.from_numpy(pos.astype(np.int32)).cuda(), q_lat[c0:c1], q_pe[c0:c1],
                         workspace=ws_a)
    out = torch.empty((L, cfg.n_heads, cfg.d_v), dtype=et, device="cuda")
    cu = torch.tensor([0, L], dtype=torch.int64, device="cuda")
    M.mla_prefill(layer.dims, q_lat, q_pe, cache, cu, L, layer.w_dev["w_uv"], out)
    torch.cuda.synchronize()
    return PrefillRun(x_q, cache, q_lat, q_pe, out)


def oracle_decode_rows(cfg, w, x_keys: np.ndarray, x_query: np.ndarray, n: int,
                       cache_rows: Optional[np.ndarray] = None, heads: Optional[List[int]] = None):
    """Oracle output [H or len(heads), d_v] for one decode query at position n-1.
    cache_rows given: attention parity on those (GPU-written) rows; else the oracle
    builds its own rows from x_keys (chain parity)."""
    from oracle import mla_oracle as O
    pos = np.arange(n)
    if cache_rows is None:
        cache_rows = O.cache_rows(x_keys, w["w_dkv"], w["w_kr"], pos, n_groups=cfg.n_groups,
                                  d_rope=cfg.d_rope, theta=cfg.rope_theta,
                                  latent_rmsnorm=cfg.latent_rmsnorm, eps=cfg.rms_eps)
    c, kr = O.split_rows(cache_rows, cfg.rank, cfg.n_groups, cfg.d_rope)
    qn, qr = O.query(x_query[None], w["w_qc"], w["w_qr"], np.array([n - 1]), n_heads=cfg.n_heads,
                     d_nope=cfg.d_nope, d_rope=cfg.d_rope, theta=cfg.rope_theta)
    heads = list(range(cfg.n_heads)) if heads is None else list(heads)
    g_of_h = O.head_groups(cfg.n_heads, cfg.n_groups)
    out = []
    for h in heads:
        o = O.mla_attention(qn[:, h:h + 1], qr[:, h:h + 1], c, kr[:, g_of_h[h]:g_of_h[h] + 1],
                            w["w_uk"][h:h + 1], w["w_uv"][h:h + 1], np.array([n - 1]), pos,
                            np.zeros(1, int), np.zeros(n, int), cfg.softmax_scale)
        out.append(o[0, 0])
    return np.stack(out)


def oracle_absorbed_rows(cfg, w, q_lat: np.ndarray, q_pe: np.ndarray, cache_rows: np.ndarray,
                         head_chunk: int = 16) -> np.ndarray:
    """Oracle output [H, d_v] of one decode query given the query the kernels see
    (the GPU's q_lat [H, r] and q_pe [H, d_rope]) and the GPU-written rows: the
    oracle's attention definition with Q = [q_lat ; q_pe], K = [c ; kr_g(h)] and
    V = c per head, then W_UV.  For logits so large that the bf16 rounding of the
    query alone moves the softmax (the oracle's own query is float64)."""
    from oracle import mla_oracle as O
    n = cache_rows.shape[0]
    c, kr = O.split_rows(cache_rows, cfg.rank, cfg.n_groups, cfg.d_rope)
    g_of_h = O.head_groups(cfg.n_heads, cfg.n_groups)
    out = np.zeros((cfg.n_heads, cfg.d_v))
    allowed = np.ones((1, n), bool)
    for h0 in range(0, cfg.n_heads, head_chunk):
        hs = np.arange(h0, min(cfg.n_heads, h0 + head_chunk))
        Q = np.concatenate([q_lat[hs], q_pe[hs]], axis=-1)[None]                      # [1, hc, r + dr]
        K = np.concatenate([np.repeat(c[:, None, :], len(hs), 1), kr[:, g_of_h[hs], :]], axis=-1)
        V = np.repeat(c[:, None, :], len(hs), 1)
        o_lat = O.softmax_attention(Q, K, V, allowed, cfg.softmax_scale)[0]           # [hc, r]
        out[hs] = np.einsum("hvc,hc->hv", w["w_uv"][hs].astype(np.float64), o_lat)
    return out


def write_err(cfg, rows_gpu: np.ndarray, rows_ref: np.ndarray) -> float:
    """Write parity of whole cache rows: the latent c per row and each rotary key
    kr_g per (row, group), each measured on its own (so neither hides the other)."""
    c_g, kr_g = O.split_rows(rows_gpu, cfg.rank, cfg.n_groups, cfg.d_rope)
    c_o, kr_o = O.split_rows(rows_ref, cfg.rank, cfg.n_groups, cfg.d_rope)
    return max(O.max_rel_err(c_g, c_o), O.max_rel_err(kr_g, kr_o))


# the parity metric of every GPU test: the oracle's own max_rel_err (pinned on
# hand-built values in tests/test_oracle_pins.py), not a second copy of it
rel_err_rows = O.max_rel_err
