"""Seeded synthetic inputs for the MLA hot path: workload shapes and tensor generators.

This module is shared by the GPU path's tests/bench and by the CPU oracle's tests.
It holds only workload definitions (shapes, hyper-parameters) and seeded random
number streams; it contains none of the attention arithmetic.

Every tensor is drawn in float32 from
``np.random.Generator(Philox(SeedSequence([seed, tensor_id, *stream])))``
and, for bf16 workloads, rounded to bfloat16 with round-to-nearest-even, so the
oracle (which upcasts the stored values exactly to float64) and the GPU (which
receives the bf16 bit patterns) see identical values.

Weight layouts follow the projection-module convention of the DeepSeek-V2 code
quoted on the page that explains MLA's matrix absorption ("关于矩阵吸收十倍提速"):
projections are stored ``[out_features, in_features]`` and the up-projection is
``kv_b_proj.weight.view(H, d_nope + d_v, r)`` split into W_UK ``[H, d_nope, r]``
and W_UV ``[H, d_v, r]``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import numpy as np

# ----------------------------------------------------------------------------
# bfloat16 helpers (input preparation only)
# ----------------------------------------------------------------------------


def rne_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return uint16 bit patterns.

    Inputs here are finite (normal draws), so no NaN special case is needed; NaN
    inputs are still mapped to a quiet NaN to keep the function total.
    """
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += u
    r += np.uint32(0x7FFF)
    r >>= np.uint32(16)
    out = r.astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def quantize(a: np.ndarray, dtype: str) -> np.ndarray:
    """Return float32 values exactly representable in ``dtype`` ('f32' or 'bf16')."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "f32":
        return a
    if dtype == "bf16":
        return bf16_bits_to_f32(rne_bf16_bits(a))
    raise ValueError(f"unknown dtype {dtype!r}")


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

# tensor ids for the seed sequence
T_X, T_WDKV, T_WKR, T_WQC, T_WQR, T_WUK, T_WUV, T_LEN, T_SAMPLE = range(9)
T_WQA, T_QGAIN, T_WQB, T_WO = range(9, 13)
T_V4 = 13  # base id of the DeepSeek-V4 variant's tensors (13 .. 20)

# Query down-projection width of the low-rank query path: DeepSeek-V2 factors its
# 5120 -> 24576 query map through 1536 dims (MLA principle page, section 'steps').
Q_LORA_RANK = 1536

X_BLOCK = 1024  # x is drawn in independent blocks of this many tokens per sequence


@dataclasses.dataclass(frozen=True)
class MLAConfig:
    name: str
    seed: int
    d_model: int
    n_heads: int           # H, query heads
    n_groups: int          # G, rotary-key groups (G == 1: one shared k_pe head)
    rank: int              # r, latent width (kv_lora_rank)
    d_rope: int            # rotary dims per query head and per key group
    d_nope: int
    d_v: int
    dtype: str             # 'f32' or 'bf16' (storage of x, weights, cache, q, out)
    mode: str              # 'decode', 'prefill', or 'prefill+decode'
    batch: int
    context: Optional[int] = None        # fixed decode context length
    ragged_lengths: Optional[Tuple[int, int]] = None  # closed range for ragged decode
    prefill_len: int = 0
    decode_steps: int = 0
    latent_rmsnorm: bool = False
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0
    description: str = ""

    @property
    def row_width(self) -> int:
        """Cache row width: latent r plus G rotary-key slices."""
        return self.rank + self.n_groups * self.d_rope

    @property
    def softmax_scale(self) -> float:
        """1/sqrt(d_nope + d_rope), the scale every workload states."""
        return 1.0 / math.sqrt(self.d_nope + self.d_rope)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def weight_shapes(self) -> Dict[str, Tuple[int, ...]]:
        H, G = self.n_heads, self.n_groups
        return {
            "w_dkv": (self.rank, self.d_model),
            "w_kr": (G * self.d_rope, self.d_model),
            "w_qc": (H * self.d_nope, self.d_model),
            "w_qr": (H * self.d_rope, self.d_model),
            "w_uk": (H, self.d_nope, self.rank),
            "w_uv": (H, self.d_v, self.rank),
        }


CONFIGS: Dict[str, MLAConfig] = {
    "tiny_f32": MLAConfig(
        name="tiny_f32", seed=1001, d_model=256, n_heads=8, n_groups=1, rank=64,
        d_rope=16, d_nope=32, d_v=32, dtype="f32", mode="prefill+decode", batch=1,
        prefill_len=256, decode_steps=16,
        description="tiny fp32 MLA layer: causal prefill of 256 tokens, then 16 decode steps"),
    "qwen25_7b_decode": MLAConfig(
        name="qwen25_7b_decode", seed=1002, d_model=3584, n_heads=28, n_groups=4,
        rank=128, d_rope=8, d_nope=128, d_v=128, dtype="bf16", mode="decode",
        batch=32, context=4096,
        description="Qwen2.5-7B-shaped decode, 28 heads in 4 rotary-key groups, r=128"),
    "deepseek_v2_decode": MLAConfig(
        name="deepseek_v2_decode", seed=1003, d_model=5120, n_heads=128, n_groups=1,
        rank=512, d_rope=64, d_nope=128, d_v=128, dtype="bf16", mode="decode",
        batch=64, context=8192,
        description="DeepSeek-V2-shaped absorbed decode, H=128, r=512, context 8192, batch 64"),
    "qwen3_30b_ragged_decode": MLAConfig(
        name="qwen3_30b_ragged_decode", seed=1004, d_model=2048, n_heads=32, n_groups=4,
        rank=512, d_rope=8, d_nope=128, d_v=128, dtype="bf16", mode="decode",
        batch=8, ragged_lengths=(1024, 32768), latent_rmsnorm=True,
        description="Qwen3-30B-A3B-shaped ragged decode, latent RMSNorm, lengths U[1024, 32768]"),
    "long_prefill_131k": MLAConfig(
        name="long_prefill_131k", seed=1005, d_model=2048, n_heads=16, n_groups=1,
        rank=256, d_rope=64, d_nope=128, d_v=128, dtype="bf16", mode="prefill",
        batch=1, prefill_len=131072,
        description="causal prefill of one 131072-token sequence, H=16, r=256"),
}

CONFIG_ORDER = ["tiny_f32", "qwen25_7b_decode", "deepseek_v2_decode",
                "qwen3_30b_ragged_decode", "long_prefill_131k"]


def small_variant(cfg: MLAConfig, **changes) -> MLAConfig:
    """A copy of ``cfg`` with some fields changed (used for reduced-size parity cases)."""
    return dataclasses.replace(cfg, **changes)


# ----------------------------------------------------------------------------
# generators
# ----------------------------------------------------------------------------


def _rng(seed: int, tensor_id: int, *stream: int) -> np.random.Generator:
    ss = np.random.SeedSequence([int(seed), int(tensor_id), *[int(s) for s in stream]])
    return np.random.Generator(np.random.Philox(ss))


def draw_normal(seed: int, tensor_id: int, stream: Tuple[int, ...], shape, std: float,
                dtype: str) -> np.ndarray:
    """float32 N(0, std^2) draw, quantized to ``dtype``'s representable values."""
    g = _rng(seed, tensor_id, *stream)
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return quantize(a, dtype)


def weights(cfg: MLAConfig) -> Dict[str, np.ndarray]:
    """All six weight tensors, N(0, 1/fan_in); fan_in is d_model for the projections
    from x and r for the up-projections out of the latent."""
    shapes = cfg.weight_shapes()
    ids = {"w_dkv": T_WDKV, "w_kr": T_WKR, "w_qc": T_WQC, "w_qr": T_WQR,
           "w_uk": T_WUK, "w_uv": T_WUV}
    out = {}
    for k, shp in shapes.items():
        fan_in = cfg.rank if k in ("w_uk", "w_uv") else cfg.d_model
        out[k] = draw_normal(cfg.seed, ids[k], (0,), shp, 1.0 / math.sqrt(fan_in), cfg.dtype)
    return out


def lowrank_query_weights(cfg: MLAConfig, q_rank: int = Q_LORA_RANK) -> Dict[str, np.ndarray]:
    """The low-rank query path's weights: W_QA [q_rank, d_model] ~ N(0, 1/d_model),
    the RMSNorm gain [q_rank] ~ 1 + N(0, 0.1^2), and W_QB [H·(d_nope + d_rope), q_rank]
    ~ N(0, 1/q_rank), its rows head-major with each head's d_nope rows first."""
    H = cfg.n_heads
    gain = draw_normal(cfg.seed, T_QGAIN, (0,), (q_rank,), 0.1, "f32") + np.float32(1.0)
    return {
        "w_qa": draw_normal(cfg.seed, T_WQA, (0,), (q_rank, cfg.d_model), 1.0 / math.sqrt(cfg.d_model), cfg.dtype),
        "q_gain": quantize(gain, cfg.dtype),
        "w_qb": draw_normal(cfg.seed, T_WQB, (0,), (H * (cfg.d_nope + cfg.d_rope), q_rank),
                            1.0 / math.sqrt(q_rank), cfg.dtype),
    }


def output_weight(cfg: MLAConfig) -> np.ndarray:
    """W_o [d_model, H·d_v] ~ N(0, 1/(H·d_v)): the output projection after W_UV."""
    k = cfg.n_heads * cfg.d_v
    return draw_normal(cfg.seed, T_WO, (0,), (cfg.d_model, k), 1.0 / math.sqrt(k), cfg.dtype)


@dataclasses.dataclass(frozen=True)
class V4Config:
    """The DeepSeek-V4 / nanowhale MLA variant (nanowhale MLA page): one KV head of
    head_dim values (its last d_rope rotary) shared by all query heads as key and
    value, a low-rank query, an attention sink, grouped low-rank output."""
    name: str
    seed: int
    d_model: int
    n_heads: int
    head_dim: int
    d_rope: int
    q_rank: int
    o_groups: int
    o_rank: int
    dtype: str
    batch: int
    context: int
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


# nanowhale-100m's attention (page: hidden 320, 8 query heads, one KV head,
# q_lora_rank 160, head_dim 512 = 448 + 64 rotary, o_groups 8, o_lora_rank 1024,
# context 2048), decoded for 256 sequences at full context.
V4_CONFIGS: Dict[str, V4Config] = {
    "nanowhale_v4_decode": V4Config(
        name="nanowhale_v4_decode", seed=1006, d_model=320, n_heads=8, head_dim=512, d_rope=64,
        q_rank=160, o_groups=8, o_rank=1024, dtype="bf16", batch=256, context=2048),
}


def v4_weights(cfg: V4Config) -> Dict[str, np.ndarray]:
    """W_KV [head_dim, d_model], kv_gain [head_dim], W_QA [q_rank, d_model], q_gain
    [q_rank], W_QB [H·head_dim, q_rank], W_OA [o_groups·o_rank, H·head_dim/o_groups],
    W_OB [d_model, o_groups·o_rank] ~ N(0, 1/fan_in); gains ~ 1 + N(0, 0.1^2);
    sink [H] ~ N(0, 1) (fp32)."""
    H, D = cfg.n_heads, cfg.head_dim
    gdim = H * D // cfg.o_groups
    sd = lambda k: 1.0 / math.sqrt(k)  # noqa: E731
    g = lambda i, n: quantize(draw_normal(cfg.seed, T_V4 + i, (0,), (n,), 0.1, "f32") + np.float32(1.0), cfg.dtype)  # noqa: E731
    return {
        "w_kv": draw_normal(cfg.seed, T_V4, (0,), (D, cfg.d_model), sd(cfg.d_model), cfg.dtype),
        "kv_gain": g(1, D),
        "w_qa": draw_normal(cfg.seed, T_V4 + 2, (0,), (cfg.q_rank, cfg.d_model), sd(cfg.d_model), cfg.dtype),
        "q_gain": g(3, cfg.q_rank),
        "w_qb": draw_normal(cfg.seed, T_V4 + 4, (0,), (H * D, cfg.q_rank), sd(cfg.q_rank), cfg.dtype),
        "w_oa": draw_normal(cfg.seed, T_V4 + 5, (0,), (cfg.o_groups * cfg.o_rank, gdim), sd(gdim), cfg.dtype),
        "w_ob": draw_normal(cfg.seed, T_V4 + 6, (0,), (cfg.d_model, cfg.o_groups * cfg.o_rank),
                            sd(cfg.o_groups * cfg.o_rank), cfg.dtype),
        "sink": draw_normal(cfg.seed, T_V4 + 7, (0,), (H,), 1.0, "f32"),
    }


def x_rows(cfg: MLAConfig, seq: int, start: int, stop: int, scale: float = 1.0,
           quantized: bool = True) -> np.ndarray:
    """Hidden states x ~ N(0, 1) for tokens [start, stop) of sequence ``seq``.

    Rows are drawn in independent blocks of X_BLOCK tokens, so any slice can be
    regenerated without drawing the whole sequence.  ``quantized=False`` returns
    the raw float32 draw; rounding it to bf16 with round-to-nearest-even (on the
    host or on the device) gives exactly the quantized values.
    """
    if stop <= start:
        return np.zeros((0, cfg.d_model), np.float32)
    b0, b1 = start // X_BLOCK, (stop - 1) // X_BLOCK
    parts = []
    for blk in range(b0, b1 + 1):
        g = _rng(cfg.seed, T_X, seq, blk)
        a = g.standard_normal(size=(X_BLOCK, cfg.d_model), dtype=np.float32)
        lo = max(start, blk * X_BLOCK) - blk * X_BLOCK
        hi = min(stop, (blk + 1) * X_BLOCK) - blk * X_BLOCK
        parts.append(a[lo:hi])
    a = parts[0] if len(parts) == 1 else np.concatenate(parts, axis=0)
    if scale != 1.0:
        a = a * np.float32(scale)
    return quantize(a, cfg.dtype) if quantized else np.ascontiguousarray(a)


def context_lengths(cfg: MLAConfig) -> np.ndarray:
    """Per-sequence context lengths (cache rows attended by each decode query)."""
    if cfg.ragged_lengths is not None:
        lo, hi = cfg.ragged_lengths
        return _rng(cfg.seed, T_LEN, 0).integers(lo, hi, endpoint=True, size=cfg.batch).astype(np.int64)
    if cfg.context is not None:
        return np.full(cfg.batch, cfg.context, np.int64)
    if cfg.mode == "prefill":
        return np.full(cfg.batch, cfg.prefill_len, np.int64)
    return np.full(cfg.batch, cfg.prefill_len + cfg.decode_steps, np.int64)


def sample_rows(cfg: MLAConfig, n_rows: int = 512) -> np.ndarray:
    """Seeded query rows spread across a long prefill: ``n_rows`` equal strata, one
    uniform pick in each; the first pick is replaced by row 0 and the last by the
    final row, so both ends of the causal range are always checked."""
    L = cfg.prefill_len
    n_rows = min(n_rows, L)
    edges = np.linspace(0, L, n_rows + 1).astype(np.int64)
    g = _rng(cfg.seed, T_SAMPLE, 0)
    picks = np.array([g.integers(edges[i], max(edges[i] + 1, edges[i + 1])) for i in range(n_rows)],
                     dtype=np.int64)
    picks[0] = 0
    picks[-1] = L - 1
    return picks
