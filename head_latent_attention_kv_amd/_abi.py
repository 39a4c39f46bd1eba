"""ctypes binding of libmla_amd.so (include/mla.h).  Argument marshalling only:
every step of the computation runs in the library's HIP kernels.  Torch tensors
provide device memory; the current torch stream is passed as the hipStream_t."""
from __future__ import annotations

import ctypes
import math
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# MLA_LIBRARY selects another build of the same library (the debug or the
# host-sanitizer variant of build.py); the release build by default
LIB_PATH = os.environ.get("MLA_LIBRARY") or os.path.join(PKG, "libmla_amd.so")

MLA_OK, MLA_EINVAL, MLA_ENOTSUP, MLA_EWORKSPACE, MLA_EHIP, MLA_ESCRATCH = 0, -1, -2, -3, -4, -5
MLA_NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024  # include/mla.h
MLA_F32, MLA_BF16 = 0, 1
MLA_OP_WRITE_CACHE, MLA_OP_ABSORB, MLA_OP_DECODE, MLA_OP_PREFILL = 0, 1, 2, 3
MLA_OP_QUERY, MLA_OP_PREFILL_EXPANDED, MLA_OP_OUTPUT = 4, 5, 6

# Functions declared in include/mla.h, with their ctypes signatures.
_vp, _sz, _i32, _i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64


class MlaDims(ctypes.Structure):
    _fields_ = [
        ("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("n_groups", ctypes.c_int32),
        ("rank", ctypes.c_int32), ("d_rope", ctypes.c_int32), ("d_nope", ctypes.c_int32),
        ("d_v", ctypes.c_int32), ("dtype", ctypes.c_int32), ("latent_rmsnorm", ctypes.c_int32),
        ("rms_eps", ctypes.c_float), ("softmax_scale", ctypes.c_float),
        ("rope_theta", ctypes.c_double), ("rope_freqs", ctypes.c_void_p),
    ]


class MlaV4Dims(ctypes.Structure):
    _fields_ = [
        ("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("d_rope", ctypes.c_int32), ("q_rank", ctypes.c_int32), ("o_groups", ctypes.c_int32),
        ("o_rank", ctypes.c_int32), ("dtype", ctypes.c_int32), ("rms_eps", ctypes.c_float),
        ("softmax_scale", ctypes.c_float), ("rope_theta", ctypes.c_double),
    ]


MLA_V4_OP_WRITE_CACHE, MLA_V4_OP_QUERY, MLA_V4_OP_DECODE, MLA_V4_OP_PREFILL, MLA_V4_OP_OUTPUT = range(5)

_PD = ctypes.POINTER(MlaDims)
_P4 = ctypes.POINTER(MlaV4Dims)
SIGNATURES = {
    "mla_workspace_size": (_sz, [_PD, ctypes.c_int, _i32, _i64, _i32]),
    "mla_check_dims": (ctypes.c_int, [_PD]),
    "mla_rope_yarn_table": (ctypes.c_int, [_i32, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                           ctypes.c_double, ctypes.c_double, ctypes.POINTER(ctypes.c_double)]),
    "mla_write_cache": (ctypes.c_int, [_PD, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _i64, _vp, _sz, _vp]),
    "mla_absorb": (ctypes.c_int, [_PD, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
    "mla_decode": (ctypes.c_int, [_PD, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _sz, _vp]),
    "mla_prefill": (ctypes.c_int, [_PD, _vp, _vp, _vp, _vp, _i32, _i64, _i32, _vp, _vp, _vp, _sz, _vp]),
    "mla_decode_splits": (_i32, [_PD, _i32, _i32]),
    "mla_decode_split_rows": (_i32, [_PD, _i32, _i32]),
    "mla_decode_partials": (ctypes.c_int, [_PD, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp]),
    "mla_decode_noalloc": (ctypes.c_int, [_PD, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp]),
    "mla_check_decode_rows": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i64]),
    "mla_check_prefill_rows": (ctypes.c_int, [_vp, _i32, _i64, _i32, _i64]),
    "mla_check_write_rows": (ctypes.c_int, [_vp, _i64, _i64]),
    "mla_query": (ctypes.c_int, [_PD, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
    "mla_prefill_expanded": (ctypes.c_int, [_PD, _vp, _vp, _vp, _vp, _i32, _i64, _i32, _vp, _vp, _vp, _vp,
                                            _sz, _vp]),
    "mla_lowrank_workspace_size": (_sz, [_PD, _i32, _i64]),
    "mla_absorb_lowrank": (ctypes.c_int, [_PD, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _sz,
                                          _vp]),
    "mla_query_lowrank": (ctypes.c_int, [_PD, _i32, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
    "mla_output": (ctypes.c_int, [_PD, _vp, _vp, _i64, _vp, _vp, _sz, _vp]),
    "mla_tiled_weight_bytes": (_sz, [_i64, _i64]),
    "mla_tile_weights": (ctypes.c_int, [_vp, _i64, _vp, _i64, _i64, _vp, _sz, _vp]),
    "mla_absorb_tiled": (ctypes.c_int, [_PD, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
    "mla_output_tiled": (ctypes.c_int, [_PD, _vp, _vp, _i64, _vp, _vp, _sz, _vp]),
    "mla_absorb_lowrank_tiled": (ctypes.c_int, [_PD, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp,
                                                _sz, _vp]),
    "mla_v4_check_dims": (ctypes.c_int, [_P4]),
    "mla_v4_workspace_size": (_sz, [_P4, ctypes.c_int, _i32, _i64, _i32]),
    "mla_v4_write_cache": (ctypes.c_int, [_P4, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _i64, _vp, _vp, _sz, _vp]),
    "mla_v4_query": (ctypes.c_int, [_P4, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
    "mla_v4_decode": (ctypes.c_int, [_P4, _vp, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "mla_v4_prefill": (ctypes.c_int, [_P4, _vp, _vp, _vp, _i32, _i64, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "mla_v4_output": (ctypes.c_int, [_P4, _vp, _vp, _vp, _i64, _vp, _vp, _sz, _vp]),
    "mla_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "mla_version": (ctypes.c_int, []),
}

_lib = None


class MlaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({strerror(status)})")


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the built library; raises if it has not been built (no fallback path)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m head_latent_attention_kv_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    if path == LIB_PATH:
        _lib = lib
    return lib


def strerror(status: int) -> str:
    try:
        return load().mla_strerror(status).decode()
    except ImportError:
        return "library not loaded"


def make_dims(*, d_model, n_heads, n_groups, rank, d_rope, d_nope, d_v, dtype, latent_rmsnorm=False,
              rms_eps=1e-6, softmax_scale=0.0, rope_theta=10000.0, rope_freqs=None) -> MlaDims:
    """rope_freqs: a contiguous float64 device tensor of d_rope/2 inverse frequencies
    (e.g. from mla_rope_yarn_table), or None for rope_theta.  The dims object keeps
    a reference to it, so it lives as long as the dims do."""
    dt = {"f32": MLA_F32, "bf16": MLA_BF16}.get(dtype, dtype)
    ptr = None
    if rope_freqs is not None:
        if getattr(rope_freqs, "dtype", None) is None or str(rope_freqs.dtype) != "torch.float64" \
                or not rope_freqs.is_contiguous() or rope_freqs.numel() != d_rope // 2:
            raise ValueError("rope_freqs must be a contiguous float64 tensor of d_rope/2 values")
        ptr = rope_freqs.data_ptr()
    d = MlaDims(d_model, n_heads, n_groups, rank, d_rope, d_nope, d_v, int(dt), int(bool(latent_rmsnorm)),
                float(rms_eps), float(softmax_scale), float(rope_theta), ptr)
    d._rope_freqs_ref = rope_freqs
    return d


def mla_rope_yarn_table(d_rope: int, theta: float, factor: float, original_window: float,
                        alpha: float = 1.0, beta: float = 32.0) -> list:
    """YaRN's rescaled inverse frequencies (d_rope/2 values, host), from the library."""
    out = (ctypes.c_double * max(1, d_rope // 2))()
    st = load().mla_rope_yarn_table(int(d_rope), float(theta), float(factor), float(original_window),
                                    float(alpha), float(beta), out)
    if st != MLA_OK:
        raise MlaError("mla_rope_yarn_table", st)
    return list(out)[: d_rope // 2]


def dims_of(cfg, rope_freqs=None) -> MlaDims:
    """mla_dims for a workload description with the usual field names."""
    return make_dims(d_model=cfg.d_model, n_heads=cfg.n_heads, n_groups=cfg.n_groups, rank=cfg.rank,
                     d_rope=cfg.d_rope, d_nope=cfg.d_nope, d_v=cfg.d_v, dtype=cfg.dtype,
                     latent_rmsnorm=cfg.latent_rmsnorm, rms_eps=cfg.rms_eps,
                     softmax_scale=cfg.softmax_scale, rope_theta=cfg.rope_theta, rope_freqs=rope_freqs)


# ----------------------------------------------------------------------------
# torch-tensor wrappers
# ----------------------------------------------------------------------------


def _torch():
    import torch
    return torch


def _elem_dtype(dims: MlaDims):
    torch = _torch()
    return torch.float32 if dims.dtype == MLA_F32 else torch.bfloat16


def _ptr(t, name, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _check(fn, status):
    if status != MLA_OK:
        raise MlaError(fn, status)


def mla_workspace_size(dims: MlaDims, op: int, batch: int = 0, n_tokens: int = 0, max_len: int = 0) -> int:
    return int(load().mla_workspace_size(ctypes.byref(dims), op, batch, n_tokens, max_len))


def _workspace(dims, op, batch, n_tokens, max_len, workspace, device):
    need = mla_workspace_size(dims, op, batch, n_tokens, max_len)
    if workspace is None:
        torch = _torch()
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def mla_write_cache(dims, x, w_dkv, w_kr, positions, slots, cache, workspace=None, stream=None):
    torch = _torch()
    et = _elem_dtype(dims)
    T = x.shape[0]
    ws, nbytes = _workspace(dims, MLA_OP_WRITE_CACHE, 0, T, 0, workspace, x.device)
    _check("mla_write_cache", load().mla_write_cache(
        ctypes.byref(dims), _ptr(x, "x", et), _ptr(w_dkv, "w_dkv", et), _ptr(w_kr, "w_kr", et),
        _ptr(positions, "positions", torch.int32), _ptr(slots, "slots", torch.int64), T,
        _ptr(cache, "cache", et), cache.shape[0], _ptr(ws, "workspace"), nbytes, _stream(stream)))
    return cache


def mla_absorb(dims, x, w_qc, w_qr, w_uk, positions, q_lat, q_pe, workspace=None, stream=None):
    torch = _torch()
    et = _elem_dtype(dims)
    T = x.shape[0]
    ws, nbytes = _workspace(dims, MLA_OP_ABSORB, 0, T, 0, workspace, x.device)
    _check("mla_absorb", load().mla_absorb(
        ctypes.byref(dims), _ptr(x, "x", et), _ptr(w_qc, "w_qc", et), _ptr(w_qr, "w_qr", et),
        _ptr(w_uk, "w_uk", et), _ptr(positions, "positions", torch.int32), T,
        _ptr(q_lat, "q_lat", et), _ptr(q_pe, "q_pe", et), _ptr(ws, "workspace"), nbytes,
        _stream(stream)))
    return q_lat, q_pe


def mla_decode(dims, q_lat, q_pe, cache, seq_start, seq_len, max_len, w_uv, out, workspace=None,
               stream=None):
    torch = _torch()
    et = _elem_dtype(dims)
    B = q_lat.shape[0]
    ws, nbytes = _workspace(dims, MLA_OP_DECODE, B, 0, max_len, workspace, q_lat.device)
    _check("mla_decode", load().mla_decode(
        ctypes.byref(dims), _ptr(q_lat, "q_lat", et), _ptr(q_pe, "q_pe", et), _ptr(cache, "cache", et),
        _ptr(seq_start, "seq_start", torch.int64), _ptr(seq_len, "seq_len", torch.int32), B,
        int(max_len), _ptr(w_uv, "w_uv", et), _ptr(out, "out", et), _ptr(ws, "workspace"), nbytes,
        _stream(stream)))
    return out


def mla_decode_noalloc(dims, q_lat, q_pe, cache, seq_start, seq_len, max_len, w_uv, out, stream=None):
    """mla_decode with the library's static scratch array in place of a workspace:
    no device memory is allocated on this path."""
    torch = _torch()
    et = _elem_dtype(dims)
    B = q_lat.shape[0]
    _check("mla_decode_noalloc", load().mla_decode_noalloc(
        ctypes.byref(dims), _ptr(q_lat, "q_lat", et), _ptr(q_pe, "q_pe", et), _ptr(cache, "cache", et),
        _ptr(seq_start, "seq_start", torch.int64), _ptr(seq_len, "seq_len", torch.int32), B,
        int(max_len), _ptr(w_uv, "w_uv", et), _ptr(out, "out", et), _stream(stream)))
    return out


def mla_decode_splits(dims, batch: int, max_len: int) -> int:
    n = int(load().mla_decode_splits(ctypes.byref(dims), int(batch), int(max_len)))
    if n < 0:
        raise MlaError("mla_decode_splits", n)
    return n


def mla_decode_split_rows(dims, batch: int, max_len: int) -> int:
    n = int(load().mla_decode_split_rows(ctypes.byref(dims), int(batch), int(max_len)))
    if n < 0:
        raise MlaError("mla_decode_split_rows", n)
    return n


def mla_decode_partials(dims, q_lat, q_pe, cache, seq_start, seq_len, max_len, n_split, part_o, part_ml,
                        stream=None):
    torch = _torch()
    et = _elem_dtype(dims)
    B = q_lat.shape[0]
    _check("mla_decode_partials", load().mla_decode_partials(
        ctypes.byref(dims), _ptr(q_lat, "q_lat", et), _ptr(q_pe, "q_pe", et), _ptr(cache, "cache", et),
        _ptr(seq_start, "seq_start", torch.int64), _ptr(seq_len, "seq_len", torch.int32), B,
        int(max_len), int(n_split), _ptr(part_o, "part_o", et),
        _ptr(part_ml, "part_ml", torch.float32), _stream(stream)))
    return part_o, part_ml


def mla_prefill(dims, q_lat, q_pe, cache, cu_seqlens, max_len, w_uv, out, workspace=None, stream=None):
    torch = _torch()
    et = _elem_dtype(dims)
    T = q_lat.shape[0]
    B = cu_seqlens.shape[0] - 1
    ws, nbytes = _workspace(dims, MLA_OP_PREFILL, B, T, max_len, workspace, q_lat.device)
    _check("mla_prefill", load().mla_prefill(
        ctypes.byref(dims), _ptr(q_lat, "q_lat", et), _ptr(q_pe, "q_pe", et), _ptr(cache, "cache", et),
        _ptr(cu_seqlens, "cu_seqlens", torch.int64), B, T, int(max_len), _ptr(w_uv, "w_uv", et),
        _ptr(out, "out", et), _ptr(ws, "workspace"), nbytes, _stream(stream)))
    return out


def mla_query(dims, x, w_qc, w_qr, positions, q_nope, q_pe, workspace=None, stream=None):
    torch = _torch()
    et = _elem_dtype(dims)
    T = x.shape[0]
    ws, nbytes = _workspace(dims, MLA_OP_QUERY, 0, T, 0, workspace, x.device)
    _check("mla_query", load().mla_query(
        ctypes.byref(dims), _ptr(x, "x", et), _ptr(w_qc, "w_qc", et), _ptr(w_qr, "w_qr", et),
        _ptr(positions, "positions", torch.int32), T, _ptr(q_nope, "q_nope", et), _ptr(q_pe, "q_pe", et),
        _ptr(ws, "workspace"), nbytes, _stream(stream)))
    return q_nope, q_pe


def mla_prefill_expanded(dims, q_nope, q_pe, cache, cu_seqlens, max_len, w_uk, w_uv, out, workspace=None,
                         stream=None):
    torch = _torch()
    et = _elem_dtype(dims)
    T = q_nope.shape[0]
    B = cu_seqlens.shape[0] - 1
    ws, nbytes = _workspace(dims, MLA_OP_PREFILL_EXPANDED, B, T, max_len, workspace, q_nope.device)
    _check("mla_prefill_expanded", load().mla_prefill_expanded(
        ctypes.byref(dims), _ptr(q_nope, "q_nope", et), _ptr(q_pe, "q_pe", et), _ptr(cache, "cache", et),
        _ptr(cu_seqlens, "cu_seqlens", torch.int64), B, T, int(max_len), _ptr(w_uk, "w_uk", et),
        _ptr(w_uv, "w_uv", et), _ptr(out, "out", et), _ptr(ws, "workspace"), nbytes, _stream(stream)))
    return out


def mla_lowrank_workspace_size(dims, q_rank: int, n_tokens: int) -> int:
    return int(load().mla_lowrank_workspace_size(ctypes.byref(dims), int(q_rank), int(n_tokens)))


def _lowrank_ws(dims, q_rank, T, workspace, device):
    if workspace is None:
        torch = _torch()
        need = mla_lowrank_workspace_size(dims, q_rank, T)
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def mla_absorb_lowrank(dims, q_rank, x, w_qa, q_gain, w_qb, w_uk, positions, q_lat, q_pe, workspace=None,
                       stream=None):
    torch = _torch()
    et = _elem_dtype(dims)
    T = x.shape[0]
    ws, nbytes = _lowrank_ws(dims, q_rank, T, workspace, x.device)
    gain = None if q_gain is None else _ptr(q_gain, "q_gain", et)
    _check("mla_absorb_lowrank", load().mla_absorb_lowrank(
        ctypes.byref(dims), int(q_rank), _ptr(x, "x", et), _ptr(w_qa, "w_qa", et), gain, _ptr(w_qb, "w_qb", et),
        _ptr(w_uk, "w_uk", et), _ptr(positions, "positions", torch.int32), T, _ptr(q_lat, "q_lat", et),
        _ptr(q_pe, "q_pe", et), _ptr(ws, "workspace"), nbytes, _stream(stream)))
    return q_lat, q_pe


def mla_absorb_lowrank_tiled(dims, q_rank, x, w_qa_tiled, q_gain, w_qb_tiled, w_uk, positions, q_lat, q_pe,
                             workspace=None, stream=None):
    torch = _torch()
    et = _elem_dtype(dims)
    T = x.shape[0]
    ws, nbytes = _lowrank_ws(dims, q_rank, T, workspace, x.device)
    gain = None if q_gain is None else _ptr(q_gain, "q_gain", et)
    _check("mla_absorb_lowrank_tiled", load().mla_absorb_lowrank_tiled(
        ctypes.byref(dims), int(q_rank), _ptr(x, "x", et), _ptr(w_qa_tiled, "w_qa_tiled"), gain,
        _ptr(w_qb_tiled, "w_qb_tiled"), _ptr(w_uk, "w_uk", et), _ptr(positions, "positions", torch.int32), T,
        _ptr(q_lat, "q_lat", et), _ptr(q_pe, "q_pe", et), _ptr(ws, "workspace"), nbytes, _stream(stream)))
    return q_lat, q_pe


def mla_query_lowrank(dims, q_rank, x, w_qa, q_gain, w_qb, positions, q_nope, q_pe, workspace=None,
                      stream=None):
    torch = _torch()
    et = _elem_dtype(dims)
    T = x.shape[0]
    ws, nbytes = _lowrank_ws(dims, q_rank, T, workspace, x.device)
    gain = None if q_gain is None else _ptr(q_gain, "q_gain", et)
    _check("mla_query_lowrank", load().mla_query_lowrank(
        ctypes.byref(dims), int(q_rank), _ptr(x, "x", et), _ptr(w_qa, "w_qa", et), gain, _ptr(w_qb, "w_qb", et),
        _ptr(positions, "positions", torch.int32), T, _ptr(q_nope, "q_nope", et), _ptr(q_pe, "q_pe", et),
        _ptr(ws, "workspace"), nbytes, _stream(stream)))
    return q_nope, q_pe


def mla_output(dims, attn, w_o, out, workspace=None, stream=None):
    et = _elem_dtype(dims)
    T = attn.shape[0]
    ws, nbytes = _workspace(dims, MLA_OP_OUTPUT, 0, T, 0, workspace, attn.device)
    _check("mla_output", load().mla_output(
        ctypes.byref(dims), _ptr(attn, "attn", et), _ptr(w_o, "w_o", et), T, _ptr(out, "out", et),
        _ptr(ws, "workspace"), nbytes, _stream(stream)))
    return out


def mla_tiled_weight_bytes(n_rows: int, k: int) -> int:
    return int(load().mla_tiled_weight_bytes(n_rows, k))


def mla_tile_weights(w0, w1=None, out=None, stream=None):
    """[w0 ; w1] (bf16 [n, k] each) in the library's tiled layout, as a uint8 tensor."""
    torch = _torch()
    n0, k = w0.shape
    n1 = 0 if w1 is None else w1.shape[0]
    if w1 is not None and w1.shape[1] != k:
        raise ValueError("w0 and w1 must have the same row length")
    need = mla_tiled_weight_bytes(n0 + n1, k)
    if out is None:
        out = torch.empty(need, dtype=torch.uint8, device=w0.device)
    _check("mla_tile_weights", load().mla_tile_weights(
        _ptr(w0, "w0", torch.bfloat16), n0, _ptr(w1, "w1", torch.bfloat16), n1, k, _ptr(out, "out"),
        out.numel() * out.element_size(), _stream(stream)))
    return out


def mla_absorb_tiled(dims, x, w_q_tiled, w_uk, positions, q_lat, q_pe, workspace=None, stream=None):
    torch = _torch()
    et = _elem_dtype(dims)
    T = x.shape[0]
    ws, nbytes = _workspace(dims, MLA_OP_ABSORB, 0, T, 0, workspace, x.device)
    _check("mla_absorb_tiled", load().mla_absorb_tiled(
        ctypes.byref(dims), _ptr(x, "x", et), _ptr(w_q_tiled, "w_q_tiled"), _ptr(w_uk, "w_uk", et),
        _ptr(positions, "positions", torch.int32), T, _ptr(q_lat, "q_lat", et), _ptr(q_pe, "q_pe", et),
        _ptr(ws, "workspace"), nbytes, _stream(stream)))
    return q_lat, q_pe


def mla_output_tiled(dims, attn, w_o_tiled, out, workspace=None, stream=None):
    et = _elem_dtype(dims)
    T = attn.shape[0]
    ws, nbytes = _workspace(dims, MLA_OP_OUTPUT, 0, T, 0, workspace, attn.device)
    _check("mla_output_tiled", load().mla_output_tiled(
        ctypes.byref(dims), _ptr(attn, "attn", et), _ptr(w_o_tiled, "w_o_tiled"), T, _ptr(out, "out", et),
        _ptr(ws, "workspace"), nbytes, _stream(stream)))
    return out


# ---- DeepSeek-V4 / nanowhale variant ----------------------------------------------


def v4_dims_of(cfg) -> MlaV4Dims:
    return MlaV4Dims(cfg.d_model, cfg.n_heads, cfg.head_dim, cfg.d_rope, cfg.q_rank, cfg.o_groups, cfg.o_rank,
                     MLA_F32 if cfg.dtype == "f32" else MLA_BF16, cfg.rms_eps, 0.0, cfg.rope_theta)


def mla_v4_workspace_size(dims: MlaV4Dims, op: int, batch: int = 0, n_tokens: int = 0, max_len: int = 0) -> int:
    return int(load().mla_v4_workspace_size(ctypes.byref(dims), op, batch, n_tokens, max_len))


def _v4_ws(dims, op, batch, n_tokens, max_len, workspace, device):
    if workspace is None:
        torch = _torch()
        need = mla_v4_workspace_size(dims, op, batch, n_tokens, max_len)
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def _v4_et(dims):
    torch = _torch()
    return torch.float32 if dims.dtype == MLA_F32 else torch.bfloat16


def mla_v4_write_cache(dims, x, w_kv, kv_gain, positions, slots, cache, rope_freqs=None, workspace=None,
                       stream=None):
    torch = _torch()
    et = _v4_et(dims)
    T = x.shape[0]
    ws, nbytes = _v4_ws(dims, MLA_V4_OP_WRITE_CACHE, 0, T, 0, workspace, x.device)
    _check("mla_v4_write_cache", load().mla_v4_write_cache(
        ctypes.byref(dims), _ptr(x, "x", et), _ptr(w_kv, "w_kv", et), _ptr(kv_gain, "kv_gain", et),
        _ptr(positions, "positions", torch.int32), _ptr(slots, "slots", torch.int64), T, _ptr(cache, "cache", et),
        cache.shape[0], _ptr(rope_freqs, "rope_freqs", torch.float64), _ptr(ws, "workspace"), nbytes,
        _stream(stream)))
    return cache


def mla_v4_query(dims, x, w_qa, q_gain, w_qb, positions, q, rope_freqs=None, workspace=None, stream=None):
    torch = _torch()
    et = _v4_et(dims)
    T = x.shape[0]
    ws, nbytes = _v4_ws(dims, MLA_V4_OP_QUERY, 0, T, 0, workspace, x.device)
    _check("mla_v4_query", load().mla_v4_query(
        ctypes.byref(dims), _ptr(x, "x", et), _ptr(w_qa, "w_qa", et), _ptr(q_gain, "q_gain", et),
        _ptr(w_qb, "w_qb", et), _ptr(positions, "positions", torch.int32), T,
        _ptr(rope_freqs, "rope_freqs", torch.float64), _ptr(q, "q", et), _ptr(ws, "workspace"), nbytes,
        _stream(stream)))
    return q


def mla_v4_decode(dims, q, cache, seq_start, seq_len, max_len, sink, out, rope_freqs=None, workspace=None,
                  stream=None):
    torch = _torch()
    et = _v4_et(dims)
    B = q.shape[0]
    ws, nbytes = _v4_ws(dims, MLA_V4_OP_DECODE, B, 0, max_len, workspace, q.device)
    _check("mla_v4_decode", load().mla_v4_decode(
        ctypes.byref(dims), _ptr(q, "q", et), _ptr(cache, "cache", et), _ptr(seq_start, "seq_start", torch.int64),
        _ptr(seq_len, "seq_len", torch.int32), B, int(max_len), _ptr(sink, "sink", torch.float32),
        _ptr(rope_freqs, "rope_freqs", torch.float64), _ptr(out, "out", et), _ptr(ws, "workspace"), nbytes,
        _stream(stream)))
    return out


def mla_v4_prefill(dims, q, cache, cu_seqlens, max_len, sink, out, rope_freqs=None, workspace=None, stream=None):
    torch = _torch()
    et = _v4_et(dims)
    T = q.shape[0]
    B = cu_seqlens.shape[0] - 1
    ws, nbytes = _v4_ws(dims, MLA_V4_OP_PREFILL, B, T, max_len, workspace, q.device)
    _check("mla_v4_prefill", load().mla_v4_prefill(
        ctypes.byref(dims), _ptr(q, "q", et), _ptr(cache, "cache", et), _ptr(cu_seqlens, "cu_seqlens", torch.int64),
        B, T, int(max_len), _ptr(sink, "sink", torch.float32), _ptr(rope_freqs, "rope_freqs", torch.float64),
        _ptr(out, "out", et), _ptr(ws, "workspace"), nbytes, _stream(stream)))
    return out


def mla_v4_output(dims, attn, w_oa, w_ob, out, workspace=None, stream=None):
    et = _v4_et(dims)
    T = attn.shape[0]
    ws, nbytes = _v4_ws(dims, MLA_V4_OP_OUTPUT, 0, T, 0, workspace, attn.device)
    _check("mla_v4_output", load().mla_v4_output(
        ctypes.byref(dims), _ptr(attn, "attn", et), _ptr(w_oa, "w_oa", et), _ptr(w_ob, "w_ob", et), T,
        _ptr(out, "out", et), _ptr(ws, "workspace"), nbytes, _stream(stream)))
    return out


def default_scale(d_nope: int, d_rope: int) -> float:
    return 1.0 / math.sqrt(d_nope + d_rope)
