"""Device copies of the seeded inputs: float32 draws to torch tensors on the GPU.

Shared by the benchmark and the GPU tests.  Like the rest of ``mla_inputs`` it
holds no attention arithmetic: only dtype conversion and host-to-device copies.
"""
from __future__ import annotations

from typing import Dict, Tuple

import numpy as np

from . import MLAConfig, rne_bf16_bits, weights


def to_dev(a: np.ndarray, dtype: str, device="cuda"):
    """float32 array of representable values -> device tensor of the workload dtype
    (bf16 bit patterns rounded on the host, RNE)."""
    import torch
    if dtype == "bf16":
        bits = rne_bf16_bits(a).view(np.int16)
        return torch.from_numpy(bits).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)


def raw_to_dev(a: np.ndarray, dtype: str, device="cuda"):
    """Unrounded float32 draw -> device tensor; the bf16 rounding (RNE) happens on
    the device and gives the same values as ``mla_inputs.quantize`` on the host."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def device_weights(cfg: MLAConfig, device="cuda") -> Tuple[Dict[str, np.ndarray], Dict[str, object]]:
    """The six seeded weight tensors on the host (float32 of representable values)
    and as device tensors of the workload dtype."""
    w = weights(cfg)
    return w, {k: to_dev(v, cfg.dtype, device) for k, v in w.items()}
