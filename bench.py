#!/usr/bin/env python3
"""Benchmark of the absorbed-MLA hot path on one MI355X.

Default workload (the headline): DeepSeek-V2-shaped decode, H=128 heads, latent
rank r=512, 64 rotary dims (one shared rotary key), d_model=5120, batch 64,
context 8192, bf16.  One step = the whole hot path for one new token per sequence:
  mla_write_cache (append the token's [c ; kr] row)  ->  mla_absorb (q_lat, q_pe)
  ->  mla_decode (attention over the 8192 cached rows, W_UV).
The cache (rows 0..8190 of every sequence) is built once with mla_write_cache
from seeded x ~ N(0,1) before timing; inputs are resident in HBM when the timed
region starts.  Enough copies of the cache alternate between steps that no step
reads rows the 256 MB Infinity Cache still holds from the step before.

Other workloads (``--workload``): qwen25_7b_decode and qwen3_30b_ragged_decode
(the same step at their shapes), long_prefill_131k (cache write + absorb + causal
prefill of 131072 tokens, and the original-order prefill beside it), tiny_f32
(fp32 prefill of 256 tokens then 16 decode steps) and nanowhale_v4_decode (the
DeepSeek-V4 variant).

Prints one JSON line: tokens/s of whole steps with the per-step spread, the
roofline of the dominant kernel, and the float64 CPU oracle timed on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MLA absorbed decode tokens/s + % of HBM/MFMA roofline, H=128 r=512 ctx 8K"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, published
COMPONENT_WARMUP = 100       # least untimed launches before a component loop (~20 ms of load settles the clock)
FP32_VECTOR_PEAK_TFS = 157.3  # MI355X fp32 vector, published
CSRC = os.path.join(ROOT, "head_latent_attention_kv_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps before each timed loop (the shader clock takes ~20 ms of load to settle)")
    ap.add_argument("--workload", default="deepseek_v2_decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work the CPU baseline aims for (at least one unit is timed)")
    ap.add_argument("--threads", type=int, default=0, help="host threads for input generation (0: all)")
    ap.add_argument("--copy-calib-mb", type=int, default=0,
                    help="finish with one plain device copy of this many MB (calibrates HBM byte counters)")
    return ap.parse_args()


def host_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# ----------------------------------------------------------------------------
# timing: HIP events on the stream the library launches on (torch's current one)
# ----------------------------------------------------------------------------


class Timer:
    def __init__(self, torch, warmup: int):
        self.torch = torch
        self.warmup = warmup

    def run(self, fn, steps: int, warmup: int | None = None) -> dict:
        """Mean over ``steps`` calls between two events (nothing else in the
        stream), then the per-call spread from a second run with an event between
        consecutive calls.  Times in ms."""
        torch = self.torch
        import numpy as np
        stream = torch.cuda.current_stream()
        for i in range(self.warmup if warmup is None else warmup):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        mean = e0.elapsed_time(e1) / steps
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(stream)
        for i in range(steps):
            fn(i)
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
        p10, p50, p90 = np.percentile(per, [10, 50, 90])
        return {"mean_ms": mean, "median_ms": float(p50), "p10_ms": float(p10), "p90_ms": float(p90),
                "n": steps}


def spread(t: dict, scale: float = 1.0, unit: str = "ms") -> dict:
    """Per-call quantiles from the run with an event between calls (each event
    record adds a few microseconds to the call it follows)."""
    return {"unit": unit, "median": round(t["median_ms"] * scale, 4), "p10": round(t["p10_ms"] * scale, 4),
            "p90": round(t["p90_ms"] * scale, 4), "n": t["n"], "timing": "one event between calls"}


def counters(kernel_file: str, summary: str):
    """The rocprofv3 counter summary ``profiles/<summary>`` of a kernel: its
    key = value lines, or None when the kernel's source has changed since the
    counters were taken (then they describe another build)."""
    try:
        text = open(os.path.join(PROFILES, summary)).read()
        src = hashlib.sha256(open(os.path.join(CSRC, kernel_file), "rb").read()).hexdigest()
    except OSError:
        return None
    kv = {}
    for line in text.split("\n"):
        line = line.strip()
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != src:
        return None
    return kv


def oracle_threads():
    """Context that pins the oracle's BLAS to the host's cores, and the count used."""
    cores = host_threads()
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except ImportError:  # pragma: no cover
        return None, cores
    ctx = threadpool_limits(limits=cores)
    info = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    used = min(cores, int(info[0].get("num_threads", cores))) if info else cores
    return ctx, used


# ----------------------------------------------------------------------------
# algorithmic work (bytes and flops the method must move / compute)
# ----------------------------------------------------------------------------


def decode_alg_bytes(cfg, lengths) -> int:
    """Bytes the decode call must move: cache rows read, queries, W_UV, outputs."""
    e = cfg.elem_bytes
    rows = int(sum(lengths))
    B = len(lengths)
    return (rows * cfg.row_width * e + B * cfg.n_heads * (cfg.rank + cfg.d_rope) * e
            + cfg.n_heads * cfg.d_v * cfg.rank * e + B * cfg.n_heads * cfg.d_v * e)


def attention_alg_bytes(cfg, lengths) -> int:
    """Bytes the split attention kernel must move: cache rows read and the queries
    (the per-split partials it writes are overhead of the split, not counted)."""
    e = cfg.elem_bytes
    rows = int(sum(lengths))
    return rows * cfg.row_width * e + len(lengths) * cfg.n_heads * (cfg.rank + cfg.d_rope) * e


def attention_alg_flops(cfg, lengths) -> int:
    """Score (2(r + d_rope) per row and head: a head reads its own group's rotary
    key only) and P·c (2r)."""
    rows = int(sum(lengths))
    return rows * cfg.n_heads * (2 * (cfg.rank + cfg.d_rope) + 2 * cfg.rank)


def decode_alg_flops(cfg, lengths) -> int:
    B = len(lengths)
    return attention_alg_flops(cfg, lengths) + B * cfg.n_heads * 2 * cfg.rank * cfg.d_v


def prefill_alg_flops(cfg, L: int) -> int:
    """Causal absorbed attention over one sequence of L tokens: every (query,
    key <= query, head) pair costs 2(r + d_rope) for the score and 2r for P·c."""
    pairs = L * (L + 1) // 2
    return pairs * cfg.n_heads * (2 * (cfg.rank + cfg.d_rope) + 2 * cfg.rank)


def prefill_orig_alg_flops(cfg, L: int) -> int:
    """The same attention in the original order: per (query, key <= query, head)
    2(d_nope + d_rope) for the score and 2 d_v for P·v."""
    pairs = L * (L + 1) // 2
    return pairs * cfg.n_heads * (2 * (cfg.d_nope + cfg.d_rope) + 2 * cfg.d_v)


def attention_kernel(cfg):
    """The decode attention kernel the library runs at this shape, and its source."""
    if cfg.dtype == "bf16" and cfg.n_heads == 128 and cfg.n_groups == 1 and cfg.rank == 512 \
            and cfg.row_width == 576:
        return "decode_wide_kernel", "decode_wide.hip"
    if cfg.dtype == "bf16":
        return "decode_mfma_kernel", "decode_mfma.hip"
    return "attend_generic_kernel", "attend_generic.hip"


# ----------------------------------------------------------------------------
# CPU baselines: the float64 oracle as it stands, on a bounded sample
# ----------------------------------------------------------------------------


def cpu_baseline_decode(cfg, I, lengths, budget_s: float):
    """The oracle's decode of whole sequences, one after another, until the budget
    is spent: per sequence the query of its last token, K/V expansion of every
    cached row for every head, softmax attention (its cache rows are computed
    outside the timing, as the GPU's cache exists before the step)."""
    import numpy as np

    from oracle import mla_oracle as O
    w = I.weights(cfg)
    ctx, used = oracle_threads()
    done, dt, rows = 0, 0.0, 0
    try:
        for b in range(len(lengths)):
            n = int(lengths[b])
            x = I.x_rows(cfg, b, 0, n)
            cr = O.cache_rows(x, w["w_dkv"], w["w_kr"], np.arange(n), n_groups=cfg.n_groups,
                              d_rope=cfg.d_rope, theta=cfg.rope_theta,
                              latent_rmsnorm=cfg.latent_rmsnorm, eps=cfg.rms_eps)
            c, kr = O.split_rows(cr, cfg.rank, cfg.n_groups, cfg.d_rope)
            t0 = time.perf_counter()
            qn, qr = O.query(x[-1:], w["w_qc"], w["w_qr"], np.array([n - 1]), n_heads=cfg.n_heads,
                             d_nope=cfg.d_nope, d_rope=cfg.d_rope, theta=cfg.rope_theta)
            O.mla_attention(qn, qr, c, kr, w["w_uk"], w["w_uv"], np.array([n - 1]), np.arange(n),
                            np.zeros(1, int), np.zeros(n, int), cfg.softmax_scale, head_chunk=16)
            dt += time.perf_counter() - t0
            done += 1
            rows += n
            if dt >= budget_s:
                break
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    return {"value": round(done / dt, 4), "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"{done} of {len(lengths)} sequences ({rows} cached rows): float64 non-absorbed "
                      f"oracle per sequence (query, K/V expansion of every cached row for {cfg.n_heads} "
                      f"heads, softmax attention) = {done} decode tokens in {dt:.2f} s"}


def cpu_baseline_prefill(cfg, I, n_rows: int = 32):
    """The oracle on ``n_rows`` of the seeded checked rows (row 0 and the last row
    included), each against its full causal prefix, with the cache-row projection
    of the whole sequence and the K/V expansion of every row inside the timing.
    tokens/s charges every token of the sequence the sample's average cost per
    row, one-off projections included: a lower bound on the oracle's rate over
    the whole prefill."""
    import numpy as np

    from oracle import mla_oracle as O
    L = cfg.prefill_len
    rows = I.sample_rows(cfg)
    sel = np.unique(np.concatenate([rows[::max(1, len(rows) // n_rows)][:n_rows - 1], rows[-1:]]))
    w = I.weights(cfg)
    x = I.x_rows(cfg, 0, 0, L)
    ctx, used = oracle_threads()
    try:
        t0 = time.perf_counter()
        cr = O.cache_rows(x, w["w_dkv"], w["w_kr"], np.arange(L), n_groups=cfg.n_groups, d_rope=cfg.d_rope,
                          theta=cfg.rope_theta)
        c, kr = O.split_rows(cr, cfg.rank, cfg.n_groups, cfg.d_rope)
        qn, qr = O.query(x[sel], w["w_qc"], w["w_qr"], sel, n_heads=cfg.n_heads, d_nope=cfg.d_nope,
                         d_rope=cfg.d_rope, theta=cfg.rope_theta)
        O.mla_attention(qn, qr, c, kr, w["w_uk"], w["w_uv"], sel, np.arange(L), np.zeros(len(sel), int),
                        np.zeros(L, int), cfg.softmax_scale, head_chunk=1)
        dt = time.perf_counter() - t0
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    return {"value": round(len(sel) / dt, 4), "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"{len(sel)} of the {len(rows)} checked rows of the {L}-token sequence, each against "
                      f"its full causal prefix, with the cache-row projection of all {L} tokens and the "
                      f"K/V expansion of every row for {cfg.n_heads} heads, in {dt:.2f} s; value = rows/s, "
                      f"a lower bound on the whole-sequence rate (the one-off work is charged per row)"}


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------


def build_cache(torch, M, I, dims, wd, cfg, lengths, starts, threads):
    """Rows 0..n-2 of every sequence, written by mla_write_cache from x ~ N(0,1)."""
    rows = int(sum(lengths))
    cache = torch.empty((rows, cfg.row_width), dtype=torch.bfloat16, device="cuda")
    chunk = max(int(n) - 1 for n in lengths)
    ws = torch.empty(max(256, M.mla_workspace_size(dims, M.MLA_OP_WRITE_CACHE, 0, chunk, 0)),
                     dtype=torch.uint8, device="cuda")

    def gen(b):
        n = int(lengths[b])
        return b, I.x_rows(cfg, b, 0, n - 1, quantized=False)

    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        for b, xb in ex.map(gen, range(len(lengths))):
            n = int(lengths[b])
            xd = torch.from_numpy(xb).cuda().to(torch.bfloat16)  # RNE on device
            pos = torch.arange(n - 1, dtype=torch.int32, device="cuda")
            slots = torch.arange(n - 1, dtype=torch.int64, device="cuda") + int(starts[b])
            M.mla_write_cache(dims, xd, wd["w_dkv"], wd["w_kr"], pos, slots, cache, workspace=ws)
            del xd
    torch.cuda.synchronize()
    return cache


def bench_decode(args, torch, M, I, D, cfg):
    import numpy as np
    threads = args.threads or min(16, host_threads())
    lengths = I.context_lengths(cfg)
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)
    B = len(lengths)
    t_setup = time.perf_counter()
    _, wd = D.device_weights(cfg)
    dims = M.dims_of(cfg)
    cache0 = build_cache(torch, M, I, dims, wd, cfg, lengths, starts, threads)
    cache_bytes = cache0.numel() * cache0.element_size()
    n_copies = max(2, math.ceil(512e6 / cache_bytes) + 1)
    caches = [cache0] + [cache0.clone() for _ in range(n_copies - 1)]
    # the new token of each sequence (position n-1): its x, position and slot
    x_new = np.stack([I.x_rows(cfg, b, int(n) - 1, int(n))[0] for b, n in enumerate(lengths)])
    x_new_d = D.to_dev(x_new, cfg.dtype)
    pos_new = torch.from_numpy((lengths - 1).astype(np.int32)).cuda()
    slots_new = torch.from_numpy(starts + lengths - 1).cuda()
    seq_start = torch.from_numpy(starts).cuda()
    seq_len = torch.from_numpy(lengths.astype(np.int32)).cuda()
    max_len = int(lengths.max())
    et = torch.bfloat16
    q_lat = torch.empty((B, cfg.n_heads, cfg.rank), dtype=et, device="cuda")
    q_pe = torch.empty((B, cfg.n_heads, cfg.d_rope), dtype=et, device="cuda")
    out = torch.empty((B, cfg.n_heads, cfg.d_v), dtype=et, device="cuda")
    ws_w = torch.empty(max(256, M.mla_workspace_size(dims, M.MLA_OP_WRITE_CACHE, 0, B, 0)), dtype=torch.uint8,
                       device="cuda")
    ws_a = torch.empty(max(256, M.mla_workspace_size(dims, M.MLA_OP_ABSORB, 0, B, 0)), dtype=torch.uint8,
                       device="cuda")
    ws_d = torch.empty(max(256, M.mla_workspace_size(dims, M.MLA_OP_DECODE, B, 0, max_len)), dtype=torch.uint8,
                       device="cuda")
    # few-token steps read [W_QC ; W_QR] in the tiled layout, made once here
    tiled = cfg.dtype == "bf16" and B <= 64
    wq_t = M.mla_tile_weights(wd["w_qc"], wd["w_qr"]) if tiled else None
    setup_s = time.perf_counter() - t_setup
    T = Timer(torch, args.warmup)
    # the component loops (the decode call, the attention kernel, the other
    # projections) report steady-state kernel times: each runs at least
    # COMPONENT_WARMUP untimed launches first, enough load for the shader clock
    # to settle; the step itself takes exactly the requested warm-up
    comp_warmup = max(args.warmup, COMPONENT_WARMUP)

    def absorb(i):
        if tiled:
            M.mla_absorb_tiled(dims, x_new_d, wq_t, wd["w_uk"], pos_new, q_lat, q_pe, workspace=ws_a)
        else:
            M.mla_absorb(dims, x_new_d, wd["w_qc"], wd["w_qr"], wd["w_uk"], pos_new, q_lat, q_pe, workspace=ws_a)

    def step(i):
        c = caches[i % n_copies]
        M.mla_write_cache(dims, x_new_d, wd["w_dkv"], wd["w_kr"], pos_new, slots_new, c, workspace=ws_w)
        absorb(i)
        M.mla_decode(dims, q_lat, q_pe, c, seq_start, seq_len, max_len, wd["w_uv"], out, workspace=ws_d)

    def step_in_place(i):
        # the same step with the weights read in place (mla_absorb)
        c = caches[i % n_copies]
        M.mla_write_cache(dims, x_new_d, wd["w_dkv"], wd["w_kr"], pos_new, slots_new, c, workspace=ws_w)
        M.mla_absorb(dims, x_new_d, wd["w_qc"], wd["w_qr"], wd["w_uk"], pos_new, q_lat, q_pe, workspace=ws_a)
        M.mla_decode(dims, q_lat, q_pe, c, seq_start, seq_len, max_len, wd["w_uv"], out, workspace=ws_d)

    def decode_only(i):
        M.mla_decode(dims, q_lat, q_pe, caches[i % n_copies], seq_start, seq_len, max_len, wd["w_uv"],
                     out, workspace=ws_d)

    # one whole step first, so q_lat / q_pe hold this workload's queries before
    # the decode call and the attention kernel are timed on them; the whole step
    # (the headline) is timed last, each measurement after its own warm-up steps
    step(0)
    torch.cuda.synchronize()
    t_dec = T.run(decode_only, args.steps, warmup=comp_warmup)
    ms_dec = t_dec["mean_ms"]

    # the dominant kernel alone: the split attention (mla_decode_partials launches
    # exactly that kernel, with mla_decode's split plan), HIP events on its stream
    n_split = M.mla_decode_splits(dims, B, max_len)
    part_o = torch.empty((B, n_split, cfg.n_heads, cfg.rank), dtype=et, device="cuda")
    part_ml = torch.empty((B, n_split, cfg.n_heads, 2), dtype=torch.float32, device="cuda")

    def attention_only(i):
        M.mla_decode_partials(dims, q_lat, q_pe, caches[i % n_copies], seq_start, seq_len, max_len, n_split,
                              part_o, part_ml)

    t_att = T.run(attention_only, args.steps, warmup=comp_warmup)
    ms_att = t_att["mean_ms"]
    t_inplace = T.run(step_in_place, args.steps, warmup=comp_warmup) if tiled else None
    t_step = T.run(step, args.steps)
    ms_step = t_step["mean_ms"]
    print(f"[bench] {cfg.name}: {args.steps} steps: {ms_step * 1e3:.1f} us/step (median "
          f"{t_step['median_ms'] * 1e3:.1f}, p10 {t_step['p10_ms'] * 1e3:.1f}, p90 {t_step['p90_ms'] * 1e3:.1f}) "
          f"(setup {setup_s:.1f} s, {n_copies} cache copies)", file=sys.stderr, flush=True)
    alg_bytes = attention_alg_bytes(cfg, lengths)
    alg_flops = attention_alg_flops(cfg, lengths)
    achieved = alg_bytes / (ms_att * 1e-3) / 1e9
    kname, ksrc = attention_kernel(cfg)
    kc = counters(ksrc, f"{kname}_{cfg.name}_counters.txt")
    traffic_b = int(float(kc["hbm_bytes_per_launch"])) if kc and "hbm_bytes_per_launch" in kc else None
    mfma_busy = float(kc["mfma_busy_frac"]) if kc and "mfma_busy_frac" in kc else None
    # what the busy cycles are divided by (the summaries of short dispatches use the CUs' busy
    # cycles, since the GRBM window of a dispatch of a few microseconds is mostly profiler overhead)
    busy_basis = (kc.get("mfma_busy_basis", "SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs)")
                  if mfma_busy is not None else None)
    print(f"[bench] decode call: {ms_dec * 1e3:.1f} us; attention kernel {kname} ({n_split} splits): "
          f"{ms_att * 1e3:.1f} us, {achieved:.0f} GB/s algorithmic", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all(), "non-finite decode output"

    beyond = None
    if cfg.name == "deepseek_v2_decode":
        beyond = bench_beyond(args, torch, M, I, D, cfg, dims, wd, caches, n_copies, x_new_d, pos_new, slots_new,
                              seq_start, seq_len, max_len, q_lat, q_pe, out, ws_w, ws_d, T)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_decode(cfg, I, lengths, args.cpu_budget)
        print(f"[bench] cpu oracle: {cpu['sample']}", file=sys.stderr, flush=True)

    line = {
        "metric": METRIC if cfg.name == "deepseek_v2_decode" else
        f"MLA absorbed decode tokens/s + % of HBM roofline ({cfg.name})",
        "value": round(B / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "component_warmup": comp_warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_spread": spread(t_step),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded x ~ N(0,1), weights ~ N(0,1/fan_in)",
        "config": {"workload": cfg.name, "batch": B, "context": int(max_len),
                   "context_total_rows": int(lengths.sum()), "heads": cfg.n_heads,
                   "kv_groups": cfg.n_groups, "rank": cfg.rank, "d_rope": cfg.d_rope, "d_model": cfg.d_model,
                   "latent_rmsnorm": bool(cfg.latent_rmsnorm), "cache_copies": n_copies,
                   "step": "mla_write_cache + " + ("mla_absorb_tiled" if tiled else "mla_absorb") + " + mla_decode",
                   "weights": ("[W_QC ; W_QR] tiled once at setup (mla_tile_weights), the rest in place"
                               if tiled else "in place")},
        "roofline": {"bound": "hbm", "kernel": f"{kname} (split attention over the latent cache)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": (round(traffic_b / (ms_att * 1e-3) / 1e9, 1) if traffic_b else None),
                     "traffic_bytes_per_launch": traffic_b,
                     "alg_bytes_per_launch": alg_bytes,
                     "alg_flops_per_launch": alg_flops,
                     "mfma_frac_algorithmic": round(alg_flops / (ms_att * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 4),
                     "mfma_busy_frac_counter": mfma_busy,
                     "mfma_busy_basis": busy_basis,
                     "us_per_launch": round(ms_att * 1e3, 2),
                     "us_spread": spread(t_att, 1e3, "us"),
                     "n_split": n_split},
        "decode_call": {"us": round(ms_dec * 1e3, 2), "us_spread": spread(t_dec, 1e3, "us"),
                        "alg_bytes": decode_alg_bytes(cfg, lengths),
                        "alg_flops": decode_alg_flops(cfg, lengths),
                        "hbm_frac": round(decode_alg_bytes(cfg, lengths) / (ms_dec * 1e-3) / 1e9
                                          / HBM_PEAK_GBS, 4),
                        "cache_gbs": round(int(lengths.sum()) * cfg.row_width * cfg.elem_bytes
                                           / (ms_dec * 1e-3) / 1e9, 1)},
        "cpu_baseline": cpu,
    }
    if t_inplace is not None:
        line["step_weights_in_place"] = {"step": "mla_write_cache + mla_absorb + mla_decode",
                                         "us": round(t_inplace["mean_ms"] * 1e3, 2),
                                         "us_spread": spread(t_inplace, 1e3, "us"),
                                         "tokens_per_s": round(B / (t_inplace["mean_ms"] * 1e-3), 1)}
    if beyond is not None:
        line["beyond_attention"] = beyond
    print(json.dumps(line), flush=True)

    if args.copy_calib_mb > 0:
        # one plain copy of known size: its FETCH_SIZE / WRITE_SIZE calibrate the counters
        n = args.copy_calib_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration copy: {n * 4} bytes read, {n * 4} bytes written", file=sys.stderr)


def bench_beyond(args, torch, M, I, D, cfg, dims, wd, caches, n_copies, x_new_d, pos_new, slots_new, seq_start,
                 seq_len, max_len, q_lat, q_pe, out, ws_w, ws_d, T):
    """Beyond the attention at the DeepSeek-V2 shape: the low-rank query path (its
    1536-wide query factorisation) in place of [W_QC | W_QR], and the output
    projection W_o, their weights tiled once here."""
    B = q_lat.shape[0]
    q_rank = I.Q_LORA_RANK
    lw = {k: D.to_dev(v, cfg.dtype) for k, v in I.lowrank_query_weights(cfg, q_rank).items()}
    w_o = D.to_dev(I.output_weight(cfg), cfg.dtype)
    w_o_t = M.mla_tile_weights(w_o)
    wqa_t, wqb_t = M.mla_tile_weights(lw["w_qa"]), M.mla_tile_weights(lw["w_qb"])
    u = torch.empty((B, cfg.d_model), dtype=torch.bfloat16, device="cuda")
    ws_l = torch.empty(max(256, M.mla_lowrank_workspace_size(dims, q_rank, B)), dtype=torch.uint8, device="cuda")
    ws_o = torch.empty(max(256, M.mla_workspace_size(dims, M.MLA_OP_OUTPUT, 0, B, 0)), dtype=torch.uint8,
                       device="cuda")

    def lowrank_only(i):
        M.mla_absorb_lowrank_tiled(dims, q_rank, x_new_d, wqa_t, lw["q_gain"], wqb_t, wd["w_uk"], pos_new,
                                   q_lat, q_pe, workspace=ws_l)

    def output_only(i):
        M.mla_output_tiled(dims, out, w_o_t, u, workspace=ws_o)

    def layer_step(i):
        c = caches[i % n_copies]
        M.mla_write_cache(dims, x_new_d, wd["w_dkv"], wd["w_kr"], pos_new, slots_new, c, workspace=ws_w)
        lowrank_only(i)
        M.mla_decode(dims, q_lat, q_pe, c, seq_start, seq_len, max_len, wd["w_uv"], out, workspace=ws_d)
        output_only(i)

    comp_warmup = max(args.warmup, COMPONENT_WARMUP)
    t_lr, t_out, t_layer = T.run(lowrank_only, args.steps, warmup=comp_warmup), \
        T.run(output_only, args.steps, warmup=comp_warmup), T.run(layer_step, args.steps, warmup=comp_warmup)
    ms_lr, ms_out, ms_layer = t_lr["mean_ms"], t_out["mean_ms"], t_layer["mean_ms"]
    assert torch.isfinite(u.float()).all(), "non-finite output projection"
    lr_bytes = 2 * (q_rank * cfg.d_model + cfg.n_heads * (cfg.d_nope + cfg.d_rope) * q_rank +
                    cfg.n_heads * cfg.d_nope * cfg.rank + q_rank)
    wo_bytes = 2 * cfg.d_model * cfg.n_heads * cfg.d_v
    print(f"[bench] low-rank query {ms_lr * 1e3:.1f} us, output projection {ms_out * 1e3:.1f} us, "
          f"layer step {ms_layer * 1e3:.1f} us", file=sys.stderr, flush=True)
    return {
        "lowrank_query": {"call": "mla_absorb_lowrank_tiled", "q_rank": q_rank, "us": round(ms_lr * 1e3, 2),
                          "weight_bytes": lr_bytes,
                          "hbm_frac": round(lr_bytes / (ms_lr * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "output_projection": {"call": "mla_output_tiled", "us": round(ms_out * 1e3, 2), "weight_bytes": wo_bytes,
                              "hbm_frac": round(wo_bytes / (ms_out * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "layer_step": {"step": "mla_write_cache + mla_absorb_lowrank_tiled + mla_decode + mla_output_tiled",
                       "us": round(ms_layer * 1e3, 2), "us_spread": spread(t_layer, 1e3, "us"),
                       "tokens_per_s": round(B / (ms_layer * 1e-3), 1)},
    }


def bench_tiny(args, torch, M, I, D, cfg):
    """The fp32 layer: one step = causal prefill of 256 tokens (write + absorb +
    prefill) then 16 decode steps (write the token's row, absorb it, attend over
    every row so far), the whole run for one sequence."""
    import numpy as np
    L, S = cfg.prefill_len, cfg.decode_steps
    n_all = L + S
    w, wd = D.device_weights(cfg)
    dims = M.dims_of(cfg)
    f32 = torch.float32
    x = D.to_dev(I.x_rows(cfg, 0, 0, n_all), cfg.dtype)
    cache = torch.zeros((n_all, cfg.row_width), dtype=f32, device="cuda")
    q_lat = torch.empty((n_all, cfg.n_heads, cfg.rank), dtype=f32, device="cuda")
    q_pe = torch.empty((n_all, cfg.n_heads, cfg.d_rope), dtype=f32, device="cuda")
    out_pre = torch.empty((L, cfg.n_heads, cfg.d_v), dtype=f32, device="cuda")
    out_dec = torch.empty((S, cfg.n_heads, cfg.d_v), dtype=f32, device="cuda")
    pos = torch.arange(n_all, dtype=torch.int32, device="cuda")
    slots = torch.arange(n_all, dtype=torch.int64, device="cuda")
    cu = torch.tensor([0, L], dtype=torch.int64, device="cuda")
    seq_start = torch.zeros(1, dtype=torch.int64, device="cuda")
    seq_lens = [torch.tensor([L + s + 1], dtype=torch.int32, device="cuda") for s in range(S)]
    # one-element tensors per decode step (the library takes 16-byte aligned pointers)
    pos_1 = [torch.tensor([L + s], dtype=torch.int32, device="cuda") for s in range(S)]
    slot_1 = [torch.tensor([L + s], dtype=torch.int64, device="cuda") for s in range(S)]
    ws_w = torch.empty(max(256, M.mla_workspace_size(dims, M.MLA_OP_WRITE_CACHE, 0, L, 0)), dtype=torch.uint8,
                       device="cuda")
    ws_a = torch.empty(max(256, M.mla_workspace_size(dims, M.MLA_OP_ABSORB, 0, L, 0)), dtype=torch.uint8,
                       device="cuda")
    ws_p = torch.empty(max(256, M.mla_workspace_size(dims, M.MLA_OP_PREFILL, 1, L, L)), dtype=torch.uint8,
                       device="cuda")
    ws_d = torch.empty(max(256, M.mla_workspace_size(dims, M.MLA_OP_DECODE, 1, 0, n_all)), dtype=torch.uint8,
                       device="cuda")
    T = Timer(torch, args.warmup)

    def prefill_only(i):
        M.mla_prefill(dims, q_lat[:L], q_pe[:L], cache, cu, L, wd["w_uv"], out_pre, workspace=ws_p)

    def run(i):
        M.mla_write_cache(dims, x[:L], wd["w_dkv"], wd["w_kr"], pos[:L], slots[:L], cache, workspace=ws_w)
        M.mla_absorb(dims, x[:L], wd["w_qc"], wd["w_qr"], wd["w_uk"], pos[:L], q_lat[:L], q_pe[:L],
                     workspace=ws_a)
        prefill_only(i)
        for s in range(S):
            p = L + s
            M.mla_write_cache(dims, x[p:p + 1], wd["w_dkv"], wd["w_kr"], pos_1[s], slot_1[s], cache,
                              workspace=ws_w)
            M.mla_absorb(dims, x[p:p + 1], wd["w_qc"], wd["w_qr"], wd["w_uk"], pos_1[s], q_lat[p:p + 1],
                         q_pe[p:p + 1], workspace=ws_a)
            M.mla_decode(dims, q_lat[p:p + 1], q_pe[p:p + 1], cache, seq_start, seq_lens[s], p + 1, wd["w_uv"],
                         out_dec[s:s + 1], workspace=ws_d)

    t_run = T.run(run, args.steps)
    t_pf = T.run(prefill_only, args.steps)
    assert torch.isfinite(out_dec).all() and torch.isfinite(out_pre).all(), "non-finite tiny output"
    eager_out = (out_pre.clone(), out_dec.clone())
    # The same run captured once into a HIP graph (the library's calls launch
    # kernels only; workspaces are preallocated) and replayed: the host-side cost
    # of 51 library calls is paid once, at capture.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(0)
    out_pre.zero_()
    out_dec.zero_()
    t_graph = T.run(lambda i: graph.replay(), args.steps)
    assert torch.equal(out_pre, eager_out[0]) and torch.equal(out_dec, eager_out[1]), \
        "graph replay differs from the eager run"
    flops = prefill_alg_flops(cfg, L)
    tfs = flops / (t_pf["mean_ms"] * 1e-3) / 1e12
    print(f"[bench] tiny_f32: run {t_graph['mean_ms'] * 1e3:.1f} us as a graph replay, {t_run['mean_ms'] * 1e3:.1f} us "
          f"as eager calls ({n_all} tokens), mla_prefill {t_pf['mean_ms'] * 1e3:.1f} us", file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import mla_oracle as O
        xh = I.x_rows(cfg, 0, 0, n_all)
        p = np.arange(n_all)
        z = np.zeros(n_all, int)
        ctx, used = oracle_threads()
        reps, dt = 0, 0.0
        try:
            while dt < args.cpu_budget:
                t0 = time.perf_counter()
                # decode at position p equals causal prefill row p, so one causal
                # pass over all 272 tokens is the prefill and the 16 decode steps
                O.mla_layer(xh, xh, w, k_pos=p, q_pos=p, k_seg=z, q_seg=z, n_heads=cfg.n_heads,
                            n_groups=cfg.n_groups, d_nope=cfg.d_nope, d_rope=cfg.d_rope, theta=cfg.rope_theta,
                            scale=cfg.softmax_scale)
                dt += time.perf_counter() - t0
                reps += 1
        finally:
            if ctx is not None:
                ctx.__exit__(None, None, None)
        cpu = {"value": round(reps * n_all / dt, 1), "unit": "tokens/s", "cores": used, "kind": "oracle",
               "sample": f"the whole run ({L}-token prefill + {S} decode steps as one causal pass over "
                         f"{n_all} tokens: cache rows, queries, K/V expansion, attention) repeated "
                         f"{reps} times in {dt:.2f} s"}
    line = {
        "metric": "MLA tiny fp32 layer tokens/s (prefill 256 + 16 decode steps)",
        "value": round(n_all / (t_graph["mean_ms"] * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_graph["mean_ms"], 4),
        "ms_per_step_spread": spread(t_graph),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic: seeded x ~ N(0,1), weights ~ N(0,1/fan_in)",
        "config": {"workload": cfg.name, "prefill": L, "decode_steps": S, "heads": cfg.n_heads, "rank": cfg.rank,
                   "d_rope": cfg.d_rope, "d_model": cfg.d_model,
                   "step": "prefill (mla_write_cache + mla_absorb + mla_prefill) then 16 x (mla_write_cache + "
                           "mla_absorb + mla_decode)",
                   "launch": "the whole step captured once into a HIP graph and replayed; outputs checked "
                             "equal to the eager run"},
        "eager": {"ms_per_step": round(t_run["mean_ms"], 4), "ms_per_step_spread": spread(t_run),
                  "tokens_per_s": round(n_all / (t_run["mean_ms"] * 1e-3), 1)},
        "roofline": {"bound": "alu", "kernel": "attend_generic_kernel<float> (mla_prefill of 256 tokens)",
                     "achieved": round(tfs, 4), "peak": FP32_VECTOR_PEAK_TFS, "unit": "TFLOP/s",
                     "frac": round(tfs / FP32_VECTOR_PEAK_TFS, 6), "traffic": None,
                     "alg_flops_per_launch": flops, "us_per_launch": round(t_pf["mean_ms"] * 1e3, 2),
                     "note": "launch-latency bound: 51 library calls per step on a 256-token layer (eager)"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def bench_v4(args, torch, M, I, D, cfg):
    """DeepSeek-V4-variant decode at the nanowhale shape: one step = mla_v4_write_cache
    (the new token of each sequence) + mla_v4_query + mla_v4_decode + mla_v4_output
    over `batch` sequences of `context` cached rows (one 512-wide KV head)."""
    import numpy as np
    from oracle import mla_oracle as O
    B, L, Dh, H = cfg.batch, cfg.context, cfg.head_dim, cfg.n_heads
    dims = M.v4_dims_of(cfg)
    t_setup = time.perf_counter()
    w = I.v4_weights(cfg)
    wd = {k: (torch.from_numpy(v).cuda() if k == "sink" else D.to_dev(v, cfg.dtype)) for k, v in w.items()}
    starts = np.arange(B, dtype=np.int64) * L
    cache0 = torch.empty((B * L, Dh), dtype=torch.bfloat16, device="cuda")
    ws_w = torch.empty(M.mla_v4_workspace_size(dims, M.MLA_V4_OP_WRITE_CACHE, 0, L, 0), dtype=torch.uint8,
                       device="cuda")
    threads = args.threads or min(16, host_threads())

    def gen(b):
        return b, I.x_rows(cfg, b, 0, L - 1, quantized=False)

    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        for b, xb in ex.map(gen, range(B)):
            xd = torch.from_numpy(xb).cuda().to(torch.bfloat16)
            pos = torch.arange(L - 1, dtype=torch.int32, device="cuda")
            M.mla_v4_write_cache(dims, xd, wd["w_kv"], wd["kv_gain"], pos,
                                 pos.to(torch.int64) + int(starts[b]), cache0, workspace=ws_w)
    torch.cuda.synchronize()
    cache_bytes = cache0.numel() * 2
    n_copies = max(2, math.ceil(512e6 / cache_bytes) + 1)
    caches = [cache0] + [cache0.clone() for _ in range(n_copies - 1)]
    x_new = D.to_dev(np.stack([I.x_rows(cfg, b, L - 1, L)[0] for b in range(B)]), cfg.dtype)
    pos_new = torch.full((B,), L - 1, dtype=torch.int32, device="cuda")
    slots_new = torch.from_numpy(starts + L - 1).cuda()
    seq_start = torch.from_numpy(starts).cuda()
    seq_len = torch.full((B,), L, dtype=torch.int32, device="cuda")
    q = torch.empty((B, H, Dh), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    u = torch.empty((B, cfg.d_model), dtype=torch.bfloat16, device="cuda")
    ws = {op: torch.empty(max(256, M.mla_v4_workspace_size(dims, op, B, B, L)), dtype=torch.uint8, device="cuda")
          for op in (M.MLA_V4_OP_WRITE_CACHE, M.MLA_V4_OP_QUERY, M.MLA_V4_OP_DECODE, M.MLA_V4_OP_OUTPUT)}
    setup_s = time.perf_counter() - t_setup
    T = Timer(torch, args.warmup)

    def step(i):
        c = caches[i % n_copies]
        M.mla_v4_write_cache(dims, x_new, wd["w_kv"], wd["kv_gain"], pos_new, slots_new, c,
                             workspace=ws[M.MLA_V4_OP_WRITE_CACHE])
        M.mla_v4_query(dims, x_new, wd["w_qa"], wd["q_gain"], wd["w_qb"], pos_new, q,
                       workspace=ws[M.MLA_V4_OP_QUERY])
        M.mla_v4_decode(dims, q, c, seq_start, seq_len, L, wd["sink"], out, workspace=ws[M.MLA_V4_OP_DECODE])
        M.mla_v4_output(dims, out, wd["w_oa"], wd["w_ob"], u, workspace=ws[M.MLA_V4_OP_OUTPUT])

    def decode_only(i):
        M.mla_v4_decode(dims, q, caches[i % n_copies], seq_start, seq_len, L, wd["sink"], out,
                        workspace=ws[M.MLA_V4_OP_DECODE])

    t_step, t_dec = T.run(step, args.steps), T.run(decode_only, args.steps)
    ms_step, ms_dec = t_step["mean_ms"], t_dec["mean_ms"]
    assert torch.isfinite(u.float()).all(), "non-finite V4 output"
    # causal prefill of the first pf_b sequences (their queries from mla_v4_query)
    pf_b = min(32, B)
    x_pf = D.to_dev(np.concatenate([I.x_rows(cfg, b, 0, L) for b in range(pf_b)]), cfg.dtype)
    pos_pf = torch.arange(L, dtype=torch.int32, device="cuda").repeat(pf_b)
    q_pf = torch.empty((pf_b * L, H, Dh), dtype=torch.bfloat16, device="cuda")
    M.mla_v4_query(dims, x_pf, wd["w_qa"], wd["q_gain"], wd["w_qb"], pos_pf, q_pf)
    cu_pf = torch.arange(0, pf_b * L + 1, L, dtype=torch.int64, device="cuda")
    out_pf = torch.empty_like(q_pf)
    ws_pf = torch.empty(max(256, M.mla_v4_workspace_size(dims, M.MLA_V4_OP_PREFILL, pf_b, pf_b * L, L)),
                        dtype=torch.uint8, device="cuda")

    def prefill_only(i):
        M.mla_v4_prefill(dims, q_pf, caches[0], cu_pf, L, wd["sink"], out_pf, workspace=ws_pf)

    t_pf = T.run(prefill_only, max(3, min(10, args.steps)), warmup=1)
    ms_pf = t_pf["mean_ms"]
    assert torch.isfinite(out_pf.float()).all(), "non-finite V4 prefill output"
    pf_flops = pf_b * L * (L + 1) / 2 * H * 4 * Dh
    pf_tfs = pf_flops / (ms_pf * 1e-3) / 1e12
    dec_bytes = B * L * Dh * 2 + 2 * B * H * Dh * 2
    dec_flops = B * L * H * 4 * Dh
    gbs = dec_bytes / (ms_dec * 1e-3) / 1e9
    print(f"[bench] v4 decode: step {ms_step * 1e3:.1f} us, mla_v4_decode {ms_dec * 1e3:.1f} us "
          f"({gbs:.0f} GB/s algorithmic); mla_v4_prefill {pf_b}x{L}: {ms_pf:.2f} ms ({pf_tfs:.0f} TFLOP/s) "
          f"(setup {setup_s:.1f} s)", file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle on whole sequences until the budget is spent: cache rows, query, attention
        ctx, used = oracle_threads()
        n_s, dt = 0, 0.0
        try:
            for b in range(B):
                t0 = time.perf_counter()
                xb = I.x_rows(cfg, b, 0, L)
                kv = O.v4_cache_rows(xb, w["w_kv"], w["kv_gain"], np.arange(L), d_rope=cfg.d_rope, eps=cfg.rms_eps)
                qq = O.v4_query(xb[-1:], w["w_qa"], w["q_gain"], w["w_qb"], [L - 1], n_heads=H, head_dim=Dh,
                                d_rope=cfg.d_rope, eps=cfg.rms_eps)
                O.v4_attention(qq, kv, w["sink"], [L - 1], np.arange(L), [0], np.zeros(L, int),
                               cfg.softmax_scale, d_rope=cfg.d_rope)
                dt += time.perf_counter() - t0
                n_s += 1
                if dt >= args.cpu_budget:
                    break
        finally:
            if ctx is not None:
                ctx.__exit__(None, None, None)
        cpu = {"value": round(n_s / dt, 3), "unit": "tokens/s", "cores": used, "kind": "oracle",
               "sample": f"{n_s} of {B} sequences: float64 oracle (cache rows of {L} tokens, query, "
                         f"V4 attention) = {n_s} decode tokens, {dt:.2f} s"}
    line = {
        "metric": "MLA V4-variant decode tokens/s + % of HBM roofline (one 512-wide KV head, nanowhale shape)",
        "value": round(B / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_spread": spread(t_step),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded x ~ N(0,1), weights ~ N(0,1/fan_in), gains 1 + N(0, 0.01), sink N(0,1)",
        "config": {"workload": cfg.name, "batch": B, "context": L, "heads": H, "head_dim": Dh, "d_rope": cfg.d_rope,
                   "d_model": cfg.d_model, "q_rank": cfg.q_rank, "o_groups": cfg.o_groups, "o_rank": cfg.o_rank,
                   "step": "mla_v4_write_cache + mla_v4_query + mla_v4_decode + mla_v4_output"},
        "roofline": {"bound": "hbm", "kernel": "mla_v4_decode (decode_mfma_kernel<512, 512> + sink/rotation merge)",
                     "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "alg_bytes_per_launch": dec_bytes,
                     "alg_flops_per_launch": dec_flops, "us_per_launch": round(ms_dec * 1e3, 2),
                     "us_spread": spread(t_dec, 1e3, "us")},
        "prefill": {"call": "mla_v4_prefill", "sequences": pf_b, "tokens_per_sequence": L,
                    "ms_per_call": round(ms_pf, 4), "tokens_per_s": round(pf_b * L / (ms_pf * 1e-3), 1),
                    "alg_flops_per_call": pf_flops, "achieved_tflops": round(pf_tfs, 1),
                    "mfma_bf16_peak_tflops": MFMA_BF16_PEAK_TFS, "frac": round(pf_tfs / MFMA_BF16_PEAK_TFS, 4),
                    "note": "8 heads fill the 16 MFMA columns as 2 tokens x 8 heads; the PV takes the "
                            "weights as a bf16 hi + lo pair (2 MFMAs), not counted in the algorithmic flops"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def bench_prefill(args, torch, M, I, D, cfg):
    """Long causal prefill: one step = mla_write_cache + mla_absorb + mla_prefill over
    the whole sequence (x resident in HBM); the attention call is timed alone for
    the MFMA roofline.  The same prefill in the original order is timed beside it."""
    L = cfg.prefill_len
    _, wd = D.device_weights(cfg)
    dims = M.dims_of(cfg)
    et = torch.bfloat16
    t_setup = time.perf_counter()
    x = torch.empty((L, cfg.d_model), dtype=et, device="cuda")
    for c0 in range(0, L, 8192):
        c1 = min(L, c0 + 8192)
        x[c0:c1] = D.raw_to_dev(I.x_rows(cfg, 0, c0, c1, quantized=False), cfg.dtype)
    pos = torch.arange(L, dtype=torch.int32, device="cuda")
    slots = torch.arange(L, dtype=torch.int64, device="cuda")
    cu = torch.tensor([0, L], dtype=torch.int64, device="cuda")
    cache = torch.empty((L, cfg.row_width), dtype=et, device="cuda")
    q_lat = torch.empty((L, cfg.n_heads, cfg.rank), dtype=et, device="cuda")
    q_pe = torch.empty((L, cfg.n_heads, cfg.d_rope), dtype=et, device="cuda")
    out = torch.empty((L, cfg.n_heads, cfg.d_v), dtype=et, device="cuda")
    ws_w = torch.empty(M.mla_workspace_size(dims, M.MLA_OP_WRITE_CACHE, 0, L, 0), dtype=torch.uint8, device="cuda")
    ws_a = torch.empty(M.mla_workspace_size(dims, M.MLA_OP_ABSORB, 0, L, 0), dtype=torch.uint8, device="cuda")
    ws_p = torch.empty(M.mla_workspace_size(dims, M.MLA_OP_PREFILL, 1, L, L), dtype=torch.uint8, device="cuda")
    q_nope = torch.empty((L, cfg.n_heads, cfg.d_nope), dtype=et, device="cuda")
    ws_e = torch.empty(M.mla_workspace_size(dims, M.MLA_OP_PREFILL_EXPANDED, 1, L, L), dtype=torch.uint8,
                       device="cuda")
    setup_s = time.perf_counter() - t_setup

    def step(i):
        M.mla_write_cache(dims, x, wd["w_dkv"], wd["w_kr"], pos, slots, cache, workspace=ws_w)
        M.mla_absorb(dims, x, wd["w_qc"], wd["w_qr"], wd["w_uk"], pos, q_lat, q_pe, workspace=ws_a)
        M.mla_prefill(dims, q_lat, q_pe, cache, cu, L, wd["w_uv"], out, workspace=ws_p)

    def attention(i):
        M.mla_prefill(dims, q_lat, q_pe, cache, cu, L, wd["w_uv"], out, workspace=ws_p)

    # the same prefill in the original order (k_nope and v expanded once per row)
    def step_orig(i):
        M.mla_write_cache(dims, x, wd["w_dkv"], wd["w_kr"], pos, slots, cache, workspace=ws_w)
        M.mla_query(dims, x, wd["w_qc"], wd["w_qr"], pos, q_nope, q_pe, workspace=ws_a)
        M.mla_prefill_expanded(dims, q_nope, q_pe, cache, cu, L, wd["w_uk"], wd["w_uv"], out, workspace=ws_e)

    def attention_orig(i):
        M.mla_prefill_expanded(dims, q_nope, q_pe, cache, cu, L, wd["w_uk"], wd["w_uv"], out, workspace=ws_e)

    T = Timer(torch, min(args.warmup, 1))
    steps = max(2, min(args.steps, 5))
    t_step = T.run(step, steps)
    t_attn = T.run(attention, steps)
    ms_step, ms_attn = t_step["mean_ms"], t_attn["mean_ms"]
    flops = prefill_alg_flops(cfg, L)
    tflops = flops / (ms_attn * 1e-3) / 1e12
    print(f"[bench] prefill {L}: step {ms_step:.2f} ms, mla_prefill {ms_attn:.2f} ms "
          f"({tflops:.0f} TFLOP/s on the attention) (setup {setup_s:.1f} s)", file=sys.stderr, flush=True)
    assert torch.isfinite(out.float()).all(), "non-finite prefill output"
    t_step_o = T.run(step_orig, steps)
    t_attn_o = T.run(attention_orig, steps)
    ms_step_o, ms_attn_o = t_step_o["mean_ms"], t_attn_o["mean_ms"]
    flops_o = prefill_orig_alg_flops(cfg, L)
    tflops_o = flops_o / (ms_attn_o * 1e-3) / 1e12
    print(f"[bench] original order: step {ms_step_o:.2f} ms, mla_prefill_expanded {ms_attn_o:.2f} ms "
          f"({tflops_o:.0f} TFLOP/s)", file=sys.stderr, flush=True)
    assert torch.isfinite(out.float()).all(), "non-finite original-order prefill output"
    ka = counters("prefill_mfma.hip", f"prefill_mfma_kernel_{cfg.name}_counters.txt")
    ke = counters("prefill_expanded.hip", f"prefill_fa_kernel_{cfg.name}_counters.txt")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_prefill(cfg, I)
        print(f"[bench] cpu oracle: {cpu['sample']}", file=sys.stderr, flush=True)
    line = {
        "metric": "MLA absorbed causal prefill tokens/s + % of MFMA roofline, H=16 r=256 L=131072",
        "value": round(L / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": T.warmup,
        "ms_per_step": round(ms_step, 3),
        "ms_per_step_spread": spread(t_step),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded x ~ N(0,1), weights ~ N(0,1/fan_in)",
        "config": {"workload": cfg.name, "tokens": L, "heads": cfg.n_heads, "rank": cfg.rank,
                   "d_rope": cfg.d_rope, "d_model": cfg.d_model,
                   "step": "mla_write_cache + mla_absorb + mla_prefill"},
        "roofline": {"bound": "mfma", "kernel": "mla_prefill (prefill_mfma_kernel + W_UV)",
                     "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFS, 4), "traffic": None,
                     "mfma_busy_frac_counter": float(ka["mfma_busy_frac"]) if ka and "mfma_busy_frac" in ka else None,
                     "alg_flops_per_launch": flops, "ms_per_launch": round(ms_attn, 3),
                     "ms_spread": spread(t_attn)},
        "original_order": {
            "step": "mla_write_cache + mla_query + mla_prefill_expanded",
            "tokens_per_s": round(L / (ms_step_o * 1e-3), 1), "ms_per_step": round(ms_step_o, 3),
            "ms_per_step_spread": spread(t_step_o),
            "kernel": "mla_prefill_expanded (K/V expansion + prefill_fa_kernel)",
            "achieved": round(tflops_o, 1), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
            "frac": round(tflops_o / MFMA_BF16_PEAK_TFS, 4), "alg_flops_per_launch": flops_o,
            "mfma_busy_frac_counter": float(ke["mfma_busy_frac"]) if ke and "mfma_busy_frac" in ke else None,
            "ms_per_launch": round(ms_attn_o, 3), "ms_spread": spread(t_attn_o)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}); the decode "
              "path is measured on one GPU's share only.", file=sys.stderr)
        sys.exit(2)
    import torch

    import head_latent_attention_kv_amd as M
    import mla_inputs as I
    import mla_inputs.device as D

    M.load()
    torch.cuda.set_device(0)
    if args.workload in I.V4_CONFIGS:
        return bench_v4(args, torch, M, I, D, I.V4_CONFIGS[args.workload])
    if args.workload not in I.CONFIGS:
        raise SystemExit(f"unknown workload {args.workload!r}; one of {sorted(I.CONFIGS) + sorted(I.V4_CONFIGS)}")
    cfg = I.CONFIGS[args.workload]
    if cfg.mode == "prefill":
        return bench_prefill(args, torch, M, I, D, cfg)
    if cfg.mode == "prefill+decode":
        return bench_tiny(args, torch, M, I, D, cfg)
    return bench_decode(args, torch, M, I, D, cfg)


if __name__ == "__main__":
    main()
