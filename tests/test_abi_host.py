"""Host-only checks of the C ABI: the header compiles as C and C++, the library
loads and exports every function the header declares, and argument validation
(which runs before any HIP call) returns the documented status codes."""
import ctypes
import os
import re
import subprocess

import pytest

import mla_inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")


def _lib():
    from head_latent_attention_kv_amd import _abi
    if not os.path.exists(_abi.LIB_PATH):
        from head_latent_attention_kv_amd import build
        build.build()
    return _abi, _abi.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))


def test_header_compiles_as_c_and_cpp(tmp_path):
    for lang, comp in (("c", "gcc"), ("c++", "g++")):
        src = tmp_path / ("t." + ("c" if lang == "c" else "cpp"))
        src.write_text('#include "mla.h"\nint main(void){ return (int)sizeof(mla_dims); }\n')
        r = subprocess.run([comp, "-Wall", "-Werror", "-I", os.path.dirname(HEADER), "-c", str(src),
                            "-o", str(tmp_path / "t.o")], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_library_exports_every_declared_symbol():
    abi, lib = _lib()
    names = _declared()
    assert {"mla_write_cache", "mla_absorb", "mla_decode", "mla_prefill"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
        assert n in abi.SIGNATURES, n
    assert lib.mla_version() >= 100
    assert ctypes.sizeof(abi.MlaDims) == 64


def test_dims_validation_codes():
    abi, lib = _lib()
    for cfg in I.CONFIGS.values():
        assert lib.mla_check_dims(ctypes.byref(abi.dims_of(cfg))) == abi.MLA_OK, cfg.name
    base = dict(d_model=256, n_heads=8, n_groups=2, rank=64, d_rope=16, d_nope=32, d_v=32, dtype="bf16")
    cases = [
        (dict(n_groups=3), abi.MLA_EINVAL),       # H % G != 0
        (dict(d_rope=15), abi.MLA_EINVAL),        # odd rotary width
        (dict(d_model=0), abi.MLA_EINVAL),
        (dict(dtype=7), abi.MLA_EINVAL),
        (dict(rank=1024), abi.MLA_ENOTSUP),       # above the kernels' latent limit
        (dict(rank=40), abi.MLA_ENOTSUP),         # not a multiple of 16
        (dict(d_model=260), abi.MLA_ENOTSUP),     # bf16 rows must be 16-byte multiples
        (dict(softmax_scale=float("nan")), abi.MLA_EINVAL),
        (dict(rope_theta=-1.0), abi.MLA_EINVAL),
        # fp32 rows of 1016 values fit the generic kernel's 160 KB LDS tile, 1018 do not
        (dict(dtype="f32", rank=512, n_groups=1, d_rope=504), abi.MLA_OK),
        (dict(dtype="f32", rank=512, n_groups=1, d_rope=506), abi.MLA_ENOTSUP),
        (dict(dtype="f32", rank=512, n_groups=2, d_rope=256), abi.MLA_ENOTSUP),
        (dict(dtype="bf16", rank=512, n_groups=2, d_rope=256), abi.MLA_OK),
    ]
    for change, want in cases:
        d = abi.make_dims(**{**base, **change})
        assert lib.mla_check_dims(ctypes.byref(d)) == want, change
        if want != abi.MLA_OK:
            assert lib.mla_workspace_size(ctypes.byref(d), abi.MLA_OP_DECODE, 4, 0, 100) == 0


def test_calls_reject_bad_arguments_before_any_launch():
    abi, lib = _lib()
    d = abi.dims_of(I.CONFIGS["deepseek_v2_decode"])
    null = None
    # null pointers
    assert lib.mla_decode(ctypes.byref(d), null, null, null, null, null, 4, 100, null, null, null, 0, null) == abi.MLA_EINVAL
    assert lib.mla_prefill(ctypes.byref(d), null, null, null, null, 1, 10, 10, null, null, null, 0, null) == abi.MLA_EINVAL
    assert lib.mla_write_cache(ctypes.byref(d), null, null, null, null, null, 3, null, 3, null, 0, null) == abi.MLA_EINVAL
    assert lib.mla_absorb(ctypes.byref(d), null, null, null, null, null, 3, null, null, null, 0, null) == abi.MLA_EINVAL
    # misaligned (never dereferenced: validation fails first)
    odd = 0x1001
    assert lib.mla_decode(ctypes.byref(d), odd, odd, odd, odd, odd, 4, 100, odd, odd, odd, 1 << 30, null) == abi.MLA_EINVAL
    # negative sizes, empty calls
    assert lib.mla_decode(ctypes.byref(d), null, null, null, null, null, -1, 100, null, null, null, 0, null) == abi.MLA_EINVAL
    assert lib.mla_decode(ctypes.byref(d), null, null, null, null, null, 0, 100, null, null, null, 0, null) == abi.MLA_OK
    assert lib.mla_write_cache(ctypes.byref(d), null, null, null, null, null, 0, null, 0, null, 0, null) == abi.MLA_OK
    assert lib.mla_decode(None, null, null, null, null, null, 4, 100, null, null, null, 0, null) == abi.MLA_EINVAL
    assert lib.mla_decode_partials(ctypes.byref(d), null, null, null, null, null, 4, 100, 2, null, null, null) == abi.MLA_EINVAL
    assert lib.mla_decode_partials(ctypes.byref(d), null, null, null, null, null, 4, 100, 0, null, null, null) == abi.MLA_EINVAL
    assert lib.mla_decode_partials(ctypes.byref(d), null, null, null, null, null, 0, 100, 2, null, null, null) == abi.MLA_OK
    assert lib.mla_strerror(abi.MLA_EWORKSPACE) == b"workspace too small"


def test_noalloc_decode_refuses_before_any_hip_call():
    """mla_decode_noalloc checks dims, pointers and the static scratch's size on the
    host: a refused call makes no HIP call (none is possible here)."""
    abi, lib = _lib()
    d = abi.dims_of(I.CONFIGS["deepseek_v2_decode"])
    f = lib.mla_decode_noalloc
    p = 1 << 20  # aligned, never dereferenced
    # 64 sequences x 8192 rows fit the 64 MiB array, 300 sequences (one split, 78.6 MB of fp32 o_) do not
    assert lib.mla_workspace_size(ctypes.byref(d), abi.MLA_OP_DECODE, 64, 0, 8192) <= abi.MLA_NOALLOC_SCRATCH_BYTES
    need = lib.mla_workspace_size(ctypes.byref(d), abi.MLA_OP_DECODE, 300, 0, 8192)
    assert need > abi.MLA_NOALLOC_SCRATCH_BYTES
    assert f(ctypes.byref(d), p, p, p, p, p, 300, 8192, p, p, None) == abi.MLA_ESCRATCH
    assert b"static scratch" in lib.mla_strerror(abi.MLA_ESCRATCH)
    assert f(ctypes.byref(d), None, p, p, p, p, 4, 100, p, p, None) == abi.MLA_EINVAL
    assert f(ctypes.byref(d), p + 8, p, p, p, p, 4, 100, p, p, None) == abi.MLA_EINVAL
    assert f(ctypes.byref(d), p, p, p, p, p, -1, 100, p, p, None) == abi.MLA_EINVAL
    assert f(ctypes.byref(d), p, p, p, p, p, 4, 0, p, p, None) == abi.MLA_EINVAL
    assert f(ctypes.byref(d), p, p, p, p, p, 0, 100, p, p, None) == abi.MLA_OK
    bad = abi.make_dims(d_model=256, n_heads=8, n_groups=3, rank=64, d_rope=16, d_nope=32, d_v=32, dtype="bf16")
    assert f(ctypes.byref(bad), p, p, p, p, p, 4, 100, p, p, None) == abi.MLA_EINVAL


def test_decode_split_queries():
    abi, lib = _lib()
    d = abi.dims_of(I.CONFIGS["deepseek_v2_decode"])
    ns = lib.mla_decode_splits(ctypes.byref(d), 64, 8192)
    rows = lib.mla_decode_split_rows(ctypes.byref(d), 64, 8192)
    assert ns >= 1 and rows % 64 == 0 and ns * rows >= 8192 and (ns - 1) * rows < 8192
    assert lib.mla_decode_splits(ctypes.byref(d), 64, 0) == abi.MLA_EINVAL
    assert lib.mla_decode_splits(None, 64, 10) == abi.MLA_EINVAL


def test_workspace_sizes_cover_the_plan():
    abi, lib = _lib()
    d = abi.dims_of(I.CONFIGS["deepseek_v2_decode"])
    B, L = 64, 8192
    ws = lib.mla_workspace_size(ctypes.byref(d), abi.MLA_OP_DECODE, B, 0, L)
    assert ws >= B * 128 * 512 * 4  # at least the merged latent outputs
    assert lib.mla_workspace_size(ctypes.byref(d), abi.MLA_OP_WRITE_CACHE, 0, 1000, 0) >= 1000 * 576 * 4
    assert lib.mla_workspace_size(ctypes.byref(d), abi.MLA_OP_ABSORB, 0, 64, 0) >= 64 * 128 * 192 * 4
    assert lib.mla_workspace_size(ctypes.byref(d), 99, 1, 1, 1) == 0


def test_original_order_prefill_entry_points():
    """mla_query / mla_prefill_expanded: argument checks, shapes without a
    compiled kernel, and the workspace that holds the expanded keys and values."""
    abi, lib = _lib()
    null = None
    d = abi.dims_of(I.CONFIGS["long_prefill_131k"])
    T = 131072
    ws = lib.mla_workspace_size(ctypes.byref(d), abi.MLA_OP_PREFILL_EXPANDED, 1, T, T)
    assert ws >= T * 16 * (128 + 128) * 2
    assert lib.mla_workspace_size(ctypes.byref(d), abi.MLA_OP_QUERY, 0, 64, 0) >= 64 * 16 * 192 * 4
    assert lib.mla_query(ctypes.byref(d), null, null, null, null, 3, null, null, null, 0, null) == abi.MLA_EINVAL
    assert lib.mla_query(ctypes.byref(d), null, null, null, null, 0, null, null, null, 0, null) == abi.MLA_OK
    assert lib.mla_query(ctypes.byref(d), null, null, null, null, -1, null, null, null, 0, null) == abi.MLA_EINVAL
    pe = lib.mla_prefill_expanded
    assert pe(ctypes.byref(d), null, null, null, null, 1, 10, 10, null, null, null, null, 0, null) == abi.MLA_EINVAL
    assert pe(ctypes.byref(d), null, null, null, null, 0, 10, 10, null, null, null, null, 0, null) == abi.MLA_OK
    assert pe(ctypes.byref(d), null, null, null, null, 1, 10, 0, null, null, null, null, 0, null) == abi.MLA_EINVAL
    # aligned stand-in pointers that are never dereferenced: the workspace check fails first
    p = 0x10000
    assert pe(ctypes.byref(d), p, p, p, p, 1, 10, 10, p, p, p, p, 16, null) == abi.MLA_EWORKSPACE
    # shapes without a compiled kernel: fp32 layers, other rotary or value widths
    for cfg in ("tiny_f32", "qwen25_7b_decode", "qwen3_30b_ragged_decode"):
        dd = abi.dims_of(I.CONFIGS[cfg])
        assert pe(ctypes.byref(dd), p, p, p, p, 1, 10, 10, p, p, p, p, 1 << 40, null) == abi.MLA_ENOTSUP, cfg


def test_lowrank_query_and_output_entry_points():
    abi, lib = _lib()
    null = None
    d = abi.dims_of(I.CONFIGS["deepseek_v2_decode"])
    ws = lib.mla_lowrank_workspace_size(ctypes.byref(d), 1536, 64)
    assert ws >= 64 * (1536 * 4 + 1536 * 2 + 128 * 192 * 4)
    assert lib.mla_lowrank_workspace_size(ctypes.byref(d), 0, 64) == 0
    assert lib.mla_lowrank_workspace_size(None, 1536, 64) == 0
    a = lib.mla_absorb_lowrank
    assert a(ctypes.byref(d), 1536, null, null, null, null, null, null, 0, null, null, null, 0, null) == abi.MLA_OK
    assert a(ctypes.byref(d), 1536, null, null, null, null, null, null, 4, null, null, null, 0, null) == abi.MLA_EINVAL
    p = 0x10000
    assert a(ctypes.byref(d), 0, p, p, null, p, p, p, 4, p, p, p, 1 << 40, null) == abi.MLA_EINVAL
    assert a(ctypes.byref(d), 100, p, p, null, p, p, p, 4, p, p, p, 1 << 40, null) == abi.MLA_ENOTSUP  # q_rank % 8
    assert a(ctypes.byref(d), 8192, p, p, null, p, p, p, 4, p, p, p, 1 << 40, null) == abi.MLA_ENOTSUP  # > 4096
    assert a(ctypes.byref(d), 1536, p, p, null, p, p, p, 4, p, p, p, 16, null) == abi.MLA_EWORKSPACE
    assert a(ctypes.byref(d), 1536, p, p, 0x10001, p, p, p, 4, p, p, p, 1 << 40, null) == abi.MLA_EINVAL
    q = lib.mla_query_lowrank
    assert q(ctypes.byref(d), 1536, p, p, null, p, p, 4, null, p, p, 1 << 40, null) == abi.MLA_EINVAL
    o = lib.mla_output
    assert lib.mla_workspace_size(ctypes.byref(d), abi.MLA_OP_OUTPUT, 0, 64, 0) >= 64 * 5120 * 4
    assert lib.mla_workspace_size(ctypes.byref(d), abi.MLA_OP_OUTPUT, 0, 5000, 0) == 0  # tiled GEMM, no scratch
    assert o(ctypes.byref(d), null, null, 0, null, null, 0, null) == abi.MLA_OK
    assert o(ctypes.byref(d), null, null, 4, null, null, 0, null) == abi.MLA_EINVAL
    assert o(ctypes.byref(d), p, p, 4, p, p, 16, null) == abi.MLA_EWORKSPACE


def test_tiled_weight_entry_points():
    """Sizes of the tiled layout (96-row x 128-k blocks of 24 KB) and the argument
    errors of the tiled calls, all decided before any HIP call."""
    abi, lib = _lib()
    null = None
    p = 0x10000
    blk = 96 * 128 * 2
    assert lib.mla_tiled_weight_bytes(24576, 5120) == 256 * 40 * blk == 251658240  # [W_QC ; W_QR] at H = 128
    assert lib.mla_tiled_weight_bytes(5120, 16384) == 54 * 128 * blk              # W_o
    assert lib.mla_tiled_weight_bytes(237, 264) == 3 * 3 * blk                     # partial blocks both ways
    assert lib.mla_tiled_weight_bytes(0, 8) == 0 and lib.mla_tiled_weight_bytes(8, 0) == 0
    t = lib.mla_tile_weights
    need = lib.mla_tiled_weight_bytes(200, 264)
    assert t(p, 200, null, 0, 12, p, 1 << 40, null) == abi.MLA_EINVAL       # k not a multiple of 8
    assert t(p, -1, null, 0, 264, p, 1 << 40, null) == abi.MLA_EINVAL       # negative rows
    assert t(p, 0, null, 0, 264, p, 1 << 40, null) == abi.MLA_EINVAL        # no rows
    assert t(p, 100, null, 100, 264, p, 1 << 40, null) == abi.MLA_EINVAL    # w1 missing for its rows
    assert t(0x10001, 200, null, 0, 264, p, 1 << 40, null) == abi.MLA_EINVAL  # misaligned w0
    assert t(p, 200, null, 0, 264, p, need - 16, null) == abi.MLA_EINVAL    # output too small
    assert t(p, 200, null, 0, 264, null, need, null) == abi.MLA_EINVAL      # no output
    d = abi.dims_of(I.CONFIGS["deepseek_v2_decode"])
    f32 = abi.dims_of(I.CONFIGS["tiny_f32"])
    a = lib.mla_absorb_tiled
    assert a(ctypes.byref(d), null, null, null, null, 0, null, null, null, 0, null) == abi.MLA_OK  # no-op
    assert a(ctypes.byref(d), p, p, p, p, 65, p, p, p, 1 << 40, null) == abi.MLA_ENOTSUP        # > 64 tokens
    assert a(ctypes.byref(f32), p, p, p, p, 4, p, p, p, 1 << 40, null) == abi.MLA_ENOTSUP       # fp32 layer
    assert a(ctypes.byref(d), p, null, p, p, 4, p, p, p, 1 << 40, null) == abi.MLA_EINVAL
    assert a(ctypes.byref(d), p, p, p, p, 4, p, p, p, 16, null) == abi.MLA_EWORKSPACE
    assert a(ctypes.byref(d), p, p, p, p, -1, p, p, p, 1 << 40, null) == abi.MLA_EINVAL
    o = lib.mla_output_tiled
    assert o(ctypes.byref(d), p, p, 65, p, p, 1 << 40, null) == abi.MLA_ENOTSUP
    assert o(ctypes.byref(f32), p, p, 4, p, p, 1 << 40, null) == abi.MLA_ENOTSUP
    assert o(ctypes.byref(d), p, null, 4, p, p, 1 << 40, null) == abi.MLA_EINVAL
    assert o(ctypes.byref(d), p, p, 4, p, p, 16, null) == abi.MLA_EWORKSPACE
    lr = lib.mla_absorb_lowrank_tiled
    assert lr(ctypes.byref(d), 1536, p, p, null, p, p, p, 65, p, p, p, 1 << 40, null) == abi.MLA_ENOTSUP
    assert lr(ctypes.byref(f32), 96, p, p, null, p, p, p, 4, p, p, p, 1 << 40, null) == abi.MLA_ENOTSUP
    assert lr(ctypes.byref(d), 1536, p, p, null, p, p, p, 4, p, p, p, 16, null) == abi.MLA_EWORKSPACE
    assert lr(ctypes.byref(d), 1536, null, null, null, null, null, null, 0, null, null, null, 0, null) == abi.MLA_OK


def test_v4_entry_points_validate_arguments():
    abi, lib = _lib()
    null = None
    cfg = I.V4_CONFIGS["nanowhale_v4_decode"]
    d = abi.v4_dims_of(cfg)
    assert ctypes.sizeof(abi.MlaV4Dims) == 48
    assert lib.mla_v4_check_dims(ctypes.byref(d)) == abi.MLA_OK
    bad = abi.v4_dims_of(cfg)
    bad.d_rope = 7
    assert lib.mla_v4_check_dims(ctypes.byref(bad)) == abi.MLA_EINVAL
    bad = abi.v4_dims_of(cfg)
    bad.o_groups = 3   # H*D not divisible
    assert lib.mla_v4_check_dims(ctypes.byref(bad)) == abi.MLA_EINVAL
    bad = abi.v4_dims_of(cfg)
    bad.head_dim = 1024
    assert lib.mla_v4_check_dims(ctypes.byref(bad)) == abi.MLA_ENOTSUP
    bad = abi.v4_dims_of(cfg)
    bad.dtype = abi.MLA_F32
    assert lib.mla_v4_check_dims(ctypes.byref(bad)) == abi.MLA_ENOTSUP
    B, L = 256, 2048
    assert lib.mla_v4_workspace_size(ctypes.byref(d), abi.MLA_V4_OP_DECODE, B, 0, L) >= B * 8 * 512 * 2
    assert lib.mla_v4_workspace_size(ctypes.byref(d), abi.MLA_V4_OP_OUTPUT, 0, 64, 0) >= 64 * 8 * 1024 * 2
    p = 0x10000
    assert lib.mla_v4_decode(ctypes.byref(d), null, null, null, null, 0, L, null, null, null, null, 0, null) == abi.MLA_OK
    assert lib.mla_v4_decode(ctypes.byref(d), p, p, p, p, 4, L, null, null, p, p, 1 << 40, null) == abi.MLA_EINVAL
    assert lib.mla_v4_decode(ctypes.byref(d), p, p, p, p, 4, L, p, 0x10001, p, p, 1 << 40, null) == abi.MLA_EINVAL
    assert lib.mla_v4_decode(ctypes.byref(d), p, p, p, p, 4, L, p, null, p, p, 16, null) == abi.MLA_EWORKSPACE
    assert lib.mla_v4_prefill(ctypes.byref(d), p, p, p, 1, 10, 0, p, null, p, p, 1 << 40, null) == abi.MLA_EINVAL
    assert lib.mla_v4_query(ctypes.byref(d), p, p, null, p, p, 4, null, p, p, 1 << 40, null) == abi.MLA_EINVAL
    assert lib.mla_v4_output(ctypes.byref(d), p, p, p, 4, p, p, 16, null) == abi.MLA_EWORKSPACE
    assert lib.mla_v4_write_cache(ctypes.byref(d), p, p, p, p, p, 4, p, 10, null, p, 16, null) == abi.MLA_EWORKSPACE


def test_yarn_table_and_frequency_pointer():
    """mla_rope_yarn_table (host code of the library) against the oracle's own YaRN
    table at the Zebra page's factor 32 over a 32K window; its argument checks; and
    mla_dims.rope_freqs: accepted when null or 16-byte aligned, rejected otherwise
    (checked on the host, nothing is dereferenced)."""
    import numpy as np
    from oracle import mla_oracle as O
    abi, lib = _lib()
    for d_rope, theta, s, win in ((64, 10000.0, 32.0, 32768.0), (8, 10000.0, 32.0, 32768.0),
                                  (64, 1e6, 4.0, 4096.0), (16, 10000.0, 1.0, 2048.0)):
        got = np.array(abi.mla_rope_yarn_table(d_rope, theta, s, win))
        np.testing.assert_allclose(got, O.yarn_inv_freq(d_rope, theta, s, win), rtol=1e-14, atol=0)
    out = (ctypes.c_double * 32)()
    f = lib.mla_rope_yarn_table
    assert f(64, 10000.0, 32.0, 32768.0, 1.0, 32.0, out) == abi.MLA_OK
    assert f(63, 10000.0, 32.0, 32768.0, 1.0, 32.0, out) == abi.MLA_EINVAL
    assert f(64, 10000.0, 0.0, 32768.0, 1.0, 32.0, out) == abi.MLA_EINVAL
    assert f(64, 10000.0, 32.0, 32768.0, 32.0, 1.0, out) == abi.MLA_EINVAL
    assert f(64, 10000.0, 32.0, 32768.0, 1.0, 32.0, None) == abi.MLA_EINVAL
    d = abi.dims_of(I.CONFIGS["long_prefill_131k"])
    assert d.rope_freqs is None and lib.mla_check_dims(ctypes.byref(d)) == abi.MLA_OK
    d.rope_freqs = 0x10000
    assert lib.mla_check_dims(ctypes.byref(d)) == abi.MLA_OK
    d.rope_freqs = 0x10008
    assert lib.mla_check_dims(ctypes.byref(d)) == abi.MLA_EINVAL
    with pytest.raises(ValueError):
        import torch
        abi.dims_of(I.CONFIGS["long_prefill_131k"], rope_freqs=torch.zeros(31, dtype=torch.float64))


def test_host_range_checks_of_index_arrays():
    """mla_check_*_rows: the range checks a debug build runs on host copies of the
    index arrays before a launch (the release calls never read them)."""
    import numpy as np
    abi, lib = _lib()
    OK, BAD = abi.MLA_OK, abi.MLA_EINVAL

    def P(a):
        return a.ctypes.data_as(ctypes.c_void_p)

    big = (1 << 63) - 1
    ss, sl = np.array([0, 10, 30], np.int64), np.array([10, 20, 5], np.int32)
    dec = lib.mla_check_decode_rows
    assert dec(P(ss), P(sl), 3, 20, 35) == OK
    assert dec(P(ss), P(sl), 3, 20, big) == OK
    assert dec(P(ss), P(sl), 3, 19, 35) == BAD                      # a length above max_len
    assert dec(P(ss), P(sl), 3, 20, 34) == BAD                      # rows past the cache
    assert dec(P(np.array([0, 10, -1], np.int64)), P(sl), 3, 20, 35) == BAD
    assert dec(P(ss), P(np.array([10, 0, 5], np.int32)), 3, 20, 35) == BAD  # an empty context
    assert dec(None, None, 0, 20, 35) == OK and dec(None, None, -1, 20, 35) == BAD
    pre = lib.mla_check_prefill_rows
    cu = np.array([0, 5, 5, 12], np.int64)
    assert pre(P(cu), 3, 12, 7, 12) == OK                            # an empty segment is allowed
    assert pre(P(cu), 3, 12, 6, 12) == BAD                           # a segment of 7 > max_len
    assert pre(P(cu), 3, 12, 7, 11) == BAD                           # the rows past the cache
    assert pre(P(cu), 3, 13, 7, 13) == BAD                           # cu[batch] != n_tokens
    assert pre(P(np.array([1, 5, 5, 12], np.int64)), 3, 12, 7, 12) == BAD
    assert pre(P(np.array([0, 6, 5, 12], np.int64)), 3, 12, 7, 12) == BAD  # decreasing
    wr = lib.mla_check_write_rows
    assert wr(P(np.array([3, 0, 7], np.int64)), 3, 8) == OK
    assert wr(P(np.array([3, 8], np.int64)), 2, 8) == BAD
    assert wr(P(np.array([-1], np.int64)), 1, 8) == BAD
    assert wr(P(np.array([2, 5, 2], np.int64)), 3, 8) == BAD        # one slot written twice
    assert wr(None, 0, 8) == OK
