#!/usr/bin/env python3
"""Benchmark of the absorbed-MLA decode hot path on one MI355X.

Workload: DeepSeek-V2-shaped decode, H=128 heads, latent rank r=512, 64 rotary
dims (one shared rotary key), d_model=5120, batch 64, context 8192, bf16.
One step = the whole hot path for one new token per sequence:
  mla_write_cache (append the token's [c ; kr] row)  ->  mla_absorb (q_lat, q_pe)
  ->  mla_decode (attention over the 8192 cached rows, W_UV).
The cache (rows 0..8190 of every sequence) is built once with mla_write_cache
from seeded x ~ N(0,1) before timing; inputs are resident in HBM when the timed
region starts.  Two copies of the cache alternate between steps so no step reads
rows the 256 MB Infinity Cache still holds from the step before.

Prints one JSON line: tokens/s of whole steps, the roofline of the dominant
kernel (the decode attention), and the float64 CPU oracle timed on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MLA absorbed decode tokens/s + % of HBM/MFMA roofline, H=128 r=512 ctx 8K"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16, published


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="deepseek_v2_decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--threads", type=int, default=0, help="host threads for input generation (0: all)")
    ap.add_argument("--copy-calib-mb", type=int, default=0,
                    help="finish with one plain device copy of this many MB (calibrates HBM byte counters)")
    return ap.parse_args()


def host_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


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
    rows = int(sum(lengths))
    return rows * cfg.n_heads * (2 * (cfg.rank + cfg.d_rope) + 2 * cfg.rank)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_attention_deepseek_v2_traffic.txt")
KERNEL_SOURCE = os.path.join(ROOT, "head_latent_attention_kv_amd", "csrc", "decode_wide.hip")


def measured_traffic():
    """HBM bytes per launch of the attention kernel from the committed rocprofv3
    counter summary, or None when the kernel source has changed since."""
    import hashlib
    try:
        kv = dict(line.split("=", 1) for line in open(TRAFFIC_FILE).read().split("\n")
                  if "=" in line and not line.startswith("#"))
        src = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
    except OSError:
        return None
    if kv.get("kernel_source_sha256", "").strip() != src:
        return None
    return int(float(kv["hbm_bytes_per_launch"]))


def decode_alg_flops(cfg, lengths) -> int:
    rows = int(sum(lengths))
    B = len(lengths)
    H, r, dr = cfg.n_heads, cfg.rank, cfg.d_rope
    return rows * H * (2 * (r + dr) + 2 * r) + B * H * 2 * r * cfg.d_v


def build_cache(torch, M, I, layer, cfg, lengths, starts, threads):
    """Rows 0..n-2 of every sequence, written by mla_write_cache from x ~ N(0,1)."""
    rows = int(sum(lengths))
    cache = torch.empty((rows, cfg.row_width), dtype=torch.bfloat16, device="cuda")
    chunk = max(int(n) - 1 for n in lengths)
    ws = torch.empty(M.mla_workspace_size(layer.dims, M.MLA_OP_WRITE_CACHE, 0, chunk, 0),
                     dtype=torch.uint8, device="cuda")
    import numpy as np

    def gen(b):
        n = int(lengths[b])
        return b, I.x_rows(cfg, b, 0, n - 1, quantized=False)

    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        for b, xb in ex.map(gen, range(len(lengths))):
            n = int(lengths[b])
            xd = torch.from_numpy(xb).cuda().to(torch.bfloat16)  # RNE on device
            pos = torch.arange(n - 1, dtype=torch.int32, device="cuda")
            slots = torch.arange(n - 1, dtype=torch.int64, device="cuda") + int(starts[b])
            M.mla_write_cache(layer.dims, xd, layer.w_dev["w_dkv"], layer.w_dev["w_kr"], pos, slots,
                              cache, workspace=ws)
            del xd
    torch.cuda.synchronize()
    return cache


def cpu_baseline(cfg, I, lengths):
    """float64 oracle on one sequence's decode: query, K/V expansion, attention over
    its whole context (cache rows precomputed by the oracle outside the timing)."""
    import numpy as np

    from oracle import mla_oracle as O
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_info = None
        threadpool_limits = None
    cores = host_threads()
    n = int(lengths[0])
    w = I.weights(cfg)
    x = I.x_rows(cfg, 0, 0, n)
    ctx = threadpool_limits(limits=cores) if threadpool_limits else None
    try:
        rows = O.cache_rows(x, w["w_dkv"], w["w_kr"], np.arange(n), n_groups=cfg.n_groups,
                            d_rope=cfg.d_rope, theta=cfg.rope_theta,
                            latent_rmsnorm=cfg.latent_rmsnorm, eps=cfg.rms_eps)
        c, kr = O.split_rows(rows, cfg.rank, cfg.n_groups, cfg.d_rope)
        t0 = time.perf_counter()
        qn, qr = O.query(x[-1:], w["w_qc"], w["w_qr"], np.array([n - 1]), n_heads=cfg.n_heads,
                         d_nope=cfg.d_nope, d_rope=cfg.d_rope, theta=cfg.rope_theta)
        O.mla_attention(qn, qr, c, kr, w["w_uk"], w["w_uv"], np.array([n - 1]), np.arange(n),
                        np.zeros(1, int), np.zeros(n, int), cfg.softmax_scale, head_chunk=16)
        dt = time.perf_counter() - t0
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    used = cores
    if threadpool_info:
        info = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if info:
            used = min(cores, int(info[0].get("num_threads", cores)))
    return {"value": 1.0 / dt, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"1 of {len(lengths)} sequences: float64 non-absorbed oracle (query, "
                      f"K/V expansion of {n} cached rows for {cfg.n_heads} heads, softmax "
                      f"attention) = 1 decode token, {dt:.2f} s"}


def prefill_alg_flops(cfg, L: int) -> int:
    """Causal absorbed attention over one sequence of L tokens: every (query,
    key <= query, head) pair costs 2(r + G·d_rope) for the score and 2r for P·c."""
    pairs = L * (L + 1) // 2
    return pairs * cfg.n_heads * (2 * cfg.row_width + 2 * cfg.rank)


def prefill_orig_alg_flops(cfg, L: int) -> int:
    """The same attention in the original order: per (query, key <= query, head)
    2(d_nope + d_rope) for the score and 2 d_v for P·v."""
    pairs = L * (L + 1) // 2
    return pairs * cfg.n_heads * (2 * (cfg.d_nope + cfg.d_rope) + 2 * cfg.d_v)


def bench_v4(args, torch, M, I, Hh, cfg):
    """DeepSeek-V4-variant decode at the nanowhale shape: one step = mla_v4_write_cache
    (the new token of each sequence) + mla_v4_query + mla_v4_decode + mla_v4_output
    over `batch` sequences of `context` cached rows (one 512-wide KV head)."""
    import numpy as np
    from oracle import mla_oracle as O
    B, L, D, H = cfg.batch, cfg.context, cfg.head_dim, cfg.n_heads
    dims = M.v4_dims_of(cfg)
    t_setup = time.perf_counter()
    w = I.v4_weights(cfg)
    wd = {k: (torch.from_numpy(v).cuda() if k == "sink" else Hh.to_dev(v, cfg.dtype)) for k, v in w.items()}
    starts = np.arange(B, dtype=np.int64) * L
    cache0 = torch.empty((B * L, D), dtype=torch.bfloat16, device="cuda")
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
    x_new = Hh.to_dev(np.stack([I.x_rows(cfg, b, L - 1, L)[0] for b in range(B)]), cfg.dtype)
    pos_new = torch.full((B,), L - 1, dtype=torch.int32, device="cuda")
    slots_new = torch.from_numpy(starts + L - 1).cuda()
    seq_start = torch.from_numpy(starts).cuda()
    seq_len = torch.full((B,), L, dtype=torch.int32, device="cuda")
    q = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    u = torch.empty((B, cfg.d_model), dtype=torch.bfloat16, device="cuda")
    ws = {op: torch.empty(max(256, M.mla_v4_workspace_size(dims, op, B, B, L)), dtype=torch.uint8, device="cuda")
          for op in (M.MLA_V4_OP_WRITE_CACHE, M.MLA_V4_OP_QUERY, M.MLA_V4_OP_DECODE, M.MLA_V4_OP_OUTPUT)}
    setup_s = time.perf_counter() - t_setup

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

    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms_step, ms_dec = timed(step), timed(decode_only)
    assert torch.isfinite(u.float()).all(), "non-finite V4 output"
    # causal prefill of the first pf_b sequences (their queries from mla_v4_query)
    pf_b = min(32, B)
    x_pf = Hh.to_dev(np.concatenate([I.x_rows(cfg, b, 0, L) for b in range(pf_b)]), cfg.dtype)
    pos_pf = torch.arange(L, dtype=torch.int32, device="cuda").repeat(pf_b)
    q_pf = torch.empty((pf_b * L, H, D), dtype=torch.bfloat16, device="cuda")
    M.mla_v4_query(dims, x_pf, wd["w_qa"], wd["q_gain"], wd["w_qb"], pos_pf, q_pf)
    cu_pf = torch.arange(0, pf_b * L + 1, L, dtype=torch.int64, device="cuda")
    out_pf = torch.empty_like(q_pf)
    ws_pf = torch.empty(max(256, M.mla_v4_workspace_size(dims, M.MLA_V4_OP_PREFILL, pf_b, pf_b * L, L)),
                        dtype=torch.uint8, device="cuda")

    def prefill_only(i):
        M.mla_v4_prefill(dims, q_pf, caches[0], cu_pf, L, wd["sink"], out_pf, workspace=ws_pf)

    steps_keep = args.steps
    args.steps = max(3, min(10, args.steps))
    ms_pf = timed(prefill_only)
    args.steps = steps_keep
    assert torch.isfinite(out_pf.float()).all(), "non-finite V4 prefill output"
    pf_flops = pf_b * L * (L + 1) / 2 * H * 4 * D
    pf_tfs = pf_flops / (ms_pf * 1e-3) / 1e12
    dec_bytes = B * L * D * 2 + 2 * B * H * D * 2
    dec_flops = B * L * H * 4 * D
    gbs = dec_bytes / (ms_dec * 1e-3) / 1e9
    print(f"[bench] v4 decode: step {ms_step * 1e3:.1f} us, mla_v4_decode {ms_dec * 1e3:.1f} us "
          f"({gbs:.0f} GB/s algorithmic); mla_v4_prefill {pf_b}x{L}: {ms_pf:.2f} ms ({pf_tfs:.0f} TFLOP/s) "
          f"(setup {setup_s:.1f} s)", file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle on 32 of the sequences: cache rows, query, attention (float64)
        n_s = 32
        t0 = time.perf_counter()
        for b in range(n_s):
            xb = I.x_rows(cfg, b, 0, L)
            kv = O.v4_cache_rows(xb, w["w_kv"], w["kv_gain"], np.arange(L), d_rope=cfg.d_rope, eps=cfg.rms_eps)
            qq = O.v4_query(xb[-1:], w["w_qa"], w["q_gain"], w["w_qb"], [L - 1], n_heads=H, head_dim=D,
                            d_rope=cfg.d_rope, eps=cfg.rms_eps)
            O.v4_attention(qq, kv, w["sink"], [L - 1], np.arange(L), [0], np.zeros(L, int), cfg.softmax_scale,
                           d_rope=cfg.d_rope)
        dt = time.perf_counter() - t0
        cpu = {"value": round(n_s / dt, 3), "unit": "tokens/s", "cores": host_threads(), "kind": "oracle",
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
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded x ~ N(0,1), weights ~ N(0,1/fan_in), gains 1 + N(0, 0.01), sink N(0,1)",
        "config": {"workload": cfg.name, "batch": B, "context": L, "heads": H, "head_dim": D, "d_rope": cfg.d_rope,
                   "d_model": cfg.d_model, "q_rank": cfg.q_rank, "o_groups": cfg.o_groups, "o_rank": cfg.o_rank,
                   "step": "mla_v4_write_cache + mla_v4_query + mla_v4_decode + mla_v4_output"},
        "roofline": {"bound": "hbm", "kernel": "mla_v4_decode (decode_mfma_kernel<512, 512> + sink/rotation merge)",
                     "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "alg_bytes_per_launch": dec_bytes,
                     "alg_flops_per_launch": dec_flops, "us_per_launch": round(ms_dec * 1e3, 2)},
        "prefill": {"call": "mla_v4_prefill", "sequences": pf_b, "tokens_per_sequence": L,
                    "ms_per_call": round(ms_pf, 4), "tokens_per_s": round(pf_b * L / (ms_pf * 1e-3), 1),
                    "alg_flops_per_call": pf_flops, "achieved_tflops": round(pf_tfs, 1),
                    "mfma_bf16_peak_tflops": MFMA_BF16_PEAK_TFS, "frac": round(pf_tfs / MFMA_BF16_PEAK_TFS, 4),
                    "note": "8 heads fill the 16 MFMA columns as 2 tokens x 8 heads; the PV takes the "
                            "weights as a bf16 hi + lo pair (2 MFMAs), not counted in the algorithmic flops"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def bench_prefill(args, torch, M, I, Hh, cfg):
    """Long causal prefill: one step = mla_write_cache + mla_absorb + mla_prefill over
    the whole sequence (x resident in HBM); the attention kernel is timed alone
    for the MFMA roofline."""
    L = cfg.prefill_len
    layer = Hh.make_layer(cfg)
    dims = layer.dims
    et = torch.bfloat16
    t_setup = time.perf_counter()
    x = torch.empty((L, cfg.d_model), dtype=et, device="cuda")
    for c0 in range(0, L, 8192):
        c1 = min(L, c0 + 8192)
        x[c0:c1] = Hh.raw_to_dev(I.x_rows(cfg, 0, c0, c1, quantized=False), cfg.dtype)
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
    wd = layer.w_dev
    setup_s = time.perf_counter() - t_setup

    def step():
        M.mla_write_cache(dims, x, wd["w_dkv"], wd["w_kr"], pos, slots, cache, workspace=ws_w)
        M.mla_absorb(dims, x, wd["w_qc"], wd["w_qr"], wd["w_uk"], pos, q_lat, q_pe, workspace=ws_a)
        M.mla_prefill(dims, q_lat, q_pe, cache, cu, L, wd["w_uv"], out, workspace=ws_p)

    def attention():
        M.mla_prefill(dims, q_lat, q_pe, cache, cu, L, wd["w_uv"], out, workspace=ws_p)

    # the same prefill in the original order (k_nope and v expanded once per row)
    def step_orig():
        M.mla_write_cache(dims, x, wd["w_dkv"], wd["w_kr"], pos, slots, cache, workspace=ws_w)
        M.mla_query(dims, x, wd["w_qc"], wd["w_qr"], pos, q_nope, q_pe, workspace=ws_a)
        M.mla_prefill_expanded(dims, q_nope, q_pe, cache, cu, L, wd["w_uk"], wd["w_uv"], out, workspace=ws_e)

    def attention_orig():
        M.mla_prefill_expanded(dims, q_nope, q_pe, cache, cu, L, wd["w_uk"], wd["w_uv"], out, workspace=ws_e)

    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, n, w):
        for _ in range(w):
            fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    steps = min(args.steps, 5)
    warm = min(args.warmup, 1)
    ms_step = timed(step, steps, warm)
    ms_attn = timed(attention, steps, warm)
    flops = prefill_alg_flops(cfg, L)
    tflops = flops / (ms_attn * 1e-3) / 1e12
    print(f"[bench] prefill {L}: step {ms_step:.2f} ms, mla_prefill {ms_attn:.2f} ms "
          f"({tflops:.0f} TFLOP/s on the attention) (setup {setup_s:.1f} s)", file=sys.stderr, flush=True)
    assert torch.isfinite(out.float()).all(), "non-finite prefill output"
    ms_step_o = timed(step_orig, steps, warm)
    ms_attn_o = timed(attention_orig, steps, warm)
    flops_o = prefill_orig_alg_flops(cfg, L)
    tflops_o = flops_o / (ms_attn_o * 1e-3) / 1e12
    print(f"[bench] original order: step {ms_step_o:.2f} ms, mla_prefill_expanded {ms_attn_o:.2f} ms "
          f"({tflops_o:.0f} TFLOP/s)", file=sys.stderr, flush=True)
    assert torch.isfinite(out.float()).all(), "non-finite original-order prefill output"
    line = {
        "metric": "MLA absorbed causal prefill tokens/s + % of MFMA roofline, H=16 r=256 L=131072",
        "value": round(L / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded x ~ N(0,1), weights ~ N(0,1/fan_in)",
        "config": {"workload": cfg.name, "tokens": L, "heads": cfg.n_heads, "rank": cfg.rank,
                   "d_rope": cfg.d_rope, "d_model": cfg.d_model,
                   "step": "mla_write_cache + mla_absorb + mla_prefill"},
        "roofline": {"bound": "mfma", "kernel": "mla_prefill (attention + W_UV)",
                     "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFS, 4), "traffic": None,
                     "alg_flops_per_launch": flops, "ms_per_launch": round(ms_attn, 3)},
        "original_order": {
            "step": "mla_write_cache + mla_query + mla_prefill_expanded",
            "tokens_per_s": round(L / (ms_step_o * 1e-3), 1), "ms_per_step": round(ms_step_o, 3),
            "kernel": "mla_prefill_expanded (K/V expansion + attention)",
            "achieved": round(tflops_o, 1), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
            "frac": round(tflops_o / MFMA_BF16_PEAK_TFS, 4), "alg_flops_per_launch": flops_o,
            "ms_per_launch": round(ms_attn_o, 3)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}); the decode "
              "path is measured on one GPU's share only.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import head_latent_attention_kv_amd as M
    import mla_inputs as I
    from tests import harness as Hh

    M.load()
    torch.cuda.set_device(0)
    if args.workload in I.V4_CONFIGS:
        return bench_v4(args, torch, M, I, Hh, I.V4_CONFIGS[args.workload])
    cfg = I.CONFIGS[args.workload]
    if cfg.mode == "prefill":
        return bench_prefill(args, torch, M, I, Hh, cfg)
    if cfg.mode != "decode":
        raise SystemExit(f"no benchmark for workload mode {cfg.mode!r}")
    threads = args.threads or min(16, host_threads())
    lengths = I.context_lengths(cfg)
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)
    B = len(lengths)
    t_setup = time.perf_counter()
    layer = Hh.make_layer(cfg)
    cache0 = build_cache(torch, M, I, layer, cfg, lengths, starts, threads)
    cache_bytes = cache0.numel() * cache0.element_size()
    n_copies = max(2, math.ceil(512e6 / cache_bytes) + 1)
    caches = [cache0] + [cache0.clone() for _ in range(n_copies - 1)]
    # the new token of each sequence (position n-1): its x, position and slot
    x_new = np.stack([I.x_rows(cfg, b, int(n) - 1, int(n)) [0] for b, n in enumerate(lengths)])
    x_new_d = Hh.to_dev(x_new, cfg.dtype)
    pos_new = torch.from_numpy((lengths - 1).astype(np.int32)).cuda()
    slots_new = torch.from_numpy(starts + lengths - 1).cuda()
    seq_start = torch.from_numpy(starts).cuda()
    seq_len = torch.from_numpy(lengths.astype(np.int32)).cuda()
    max_len = int(lengths.max())
    et = torch.bfloat16
    q_lat = torch.empty((B, cfg.n_heads, cfg.rank), dtype=et, device="cuda")
    q_pe = torch.empty((B, cfg.n_heads, cfg.d_rope), dtype=et, device="cuda")
    out = torch.empty((B, cfg.n_heads, cfg.d_v), dtype=et, device="cuda")
    dims = layer.dims
    ws_w = torch.empty(M.mla_workspace_size(dims, M.MLA_OP_WRITE_CACHE, 0, B, 0), dtype=torch.uint8, device="cuda")
    ws_a = torch.empty(M.mla_workspace_size(dims, M.MLA_OP_ABSORB, 0, B, 0), dtype=torch.uint8, device="cuda")
    ws_d = torch.empty(M.mla_workspace_size(dims, M.MLA_OP_DECODE, B, 0, max_len), dtype=torch.uint8, device="cuda")
    wd = layer.w_dev
    setup_s = time.perf_counter() - t_setup

    def step(i):
        c = caches[i % n_copies]
        M.mla_write_cache(dims, x_new_d, wd["w_dkv"], wd["w_kr"], pos_new, slots_new, c, workspace=ws_w)
        M.mla_absorb(dims, x_new_d, wd["w_qc"], wd["w_qr"], wd["w_uk"], pos_new, q_lat, q_pe, workspace=ws_a)
        M.mla_decode(dims, q_lat, q_pe, c, seq_start, seq_len, max_len, wd["w_uv"], out, workspace=ws_d)

    def decode_only(i):
        M.mla_decode(dims, q_lat, q_pe, caches[i % n_copies], seq_start, seq_len, max_len, wd["w_uv"],
                     out, workspace=ws_d)

    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    print(f"[bench] {args.steps} steps: {ms_step * 1e3:.1f} us/step (setup {setup_s:.1f} s)",
          file=sys.stderr, flush=True)

    # the whole decode call (attention, then the split merge folded into W_UV)
    for i in range(args.warmup):
        decode_only(i)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        decode_only(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_dec = e0.elapsed_time(e1) / args.steps

    # the dominant kernel alone: the split attention (mla_decode_partials launches
    # exactly that kernel, with mla_decode's split plan), HIP events on its stream
    n_split = M.mla_decode_splits(dims, B, max_len)
    part_o = torch.empty((B, n_split, cfg.n_heads, cfg.rank), dtype=et, device="cuda")
    part_ml = torch.empty((B, n_split, cfg.n_heads, 2), dtype=torch.float32, device="cuda")

    def attention_only(i):
        M.mla_decode_partials(dims, q_lat, q_pe, caches[i % n_copies], seq_start, seq_len, max_len, n_split,
                              part_o, part_ml)

    for i in range(args.warmup):
        attention_only(i)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        attention_only(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_att = e0.elapsed_time(e1) / args.steps
    alg_bytes = attention_alg_bytes(cfg, lengths)
    achieved = alg_bytes / (ms_att * 1e-3) / 1e9
    traffic = measured_traffic()
    print(f"[bench] decode call: {ms_dec * 1e3:.1f} us; attention kernel ({n_split} splits): "
          f"{ms_att * 1e3:.1f} us, {achieved:.0f} GB/s algorithmic", file=sys.stderr, flush=True)

    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all(), "non-finite decode output"

    # beyond the attention: the low-rank query path (DeepSeek-V2's 1536-wide query
    # factorisation) in place of [W_QC | W_QR], and the output projection W_o
    q_rank = I.Q_LORA_RANK
    lw = {k: Hh.to_dev(v, cfg.dtype) for k, v in I.lowrank_query_weights(cfg, q_rank).items()}
    w_o = Hh.to_dev(I.output_weight(cfg), cfg.dtype)
    u = torch.empty((B, cfg.d_model), dtype=et, device="cuda")
    ws_l = torch.empty(max(256, M.mla_lowrank_workspace_size(dims, q_rank, B)), dtype=torch.uint8, device="cuda")
    ws_o = torch.empty(max(256, M.mla_workspace_size(dims, M.MLA_OP_OUTPUT, 0, B, 0)), dtype=torch.uint8,
                       device="cuda")

    def lowrank_only(i):
        M.mla_absorb_lowrank(dims, q_rank, x_new_d, lw["w_qa"], lw["q_gain"], lw["w_qb"], wd["w_uk"], pos_new,
                             q_lat, q_pe, workspace=ws_l)

    def output_only(i):
        M.mla_output(dims, out, w_o, u, workspace=ws_o)

    def layer_step(i):
        c = caches[i % n_copies]
        M.mla_write_cache(dims, x_new_d, wd["w_dkv"], wd["w_kr"], pos_new, slots_new, c, workspace=ws_w)
        lowrank_only(i)
        M.mla_decode(dims, q_lat, q_pe, c, seq_start, seq_len, max_len, wd["w_uv"], out, workspace=ws_d)
        output_only(i)

    def timed(fn):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms_lr, ms_out, ms_layer = timed(lowrank_only), timed(output_only), timed(layer_step)
    assert torch.isfinite(u.float()).all(), "non-finite output projection"
    lr_bytes = 2 * (q_rank * cfg.d_model + cfg.n_heads * (cfg.d_nope + cfg.d_rope) * q_rank +
                    cfg.n_heads * cfg.d_nope * cfg.rank + q_rank)
    wo_bytes = 2 * cfg.d_model * cfg.n_heads * cfg.d_v
    print(f"[bench] low-rank query {ms_lr * 1e3:.1f} us, output projection {ms_out * 1e3:.1f} us, "
          f"layer step {ms_layer * 1e3:.1f} us", file=sys.stderr, flush=True)
    beyond = {
        "lowrank_query": {"call": "mla_absorb_lowrank", "q_rank": q_rank, "us": round(ms_lr * 1e3, 2),
                          "weight_bytes": lr_bytes,
                          "hbm_frac": round(lr_bytes / (ms_lr * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "output_projection": {"call": "mla_output", "us": round(ms_out * 1e3, 2), "weight_bytes": wo_bytes,
                              "hbm_frac": round(wo_bytes / (ms_out * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "layer_step": {"step": "mla_write_cache + mla_absorb_lowrank + mla_decode + mla_output",
                       "us": round(ms_layer * 1e3, 2), "tokens_per_s": round(B / (ms_layer * 1e-3), 1)},
    }

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, I, lengths)
        print(f"[bench] cpu oracle: {cpu['sample']}", file=sys.stderr, flush=True)

    tokens_per_s = B / (ms_step * 1e-3)
    line = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded x ~ N(0,1), weights ~ N(0,1/fan_in)",
        "config": {"workload": cfg.name, "batch": B, "context": int(max_len), "heads": cfg.n_heads,
                   "rank": cfg.rank, "d_rope": cfg.d_rope, "d_model": cfg.d_model,
                   "step": "mla_write_cache + mla_absorb + mla_decode"},
        "roofline": {"bound": "hbm", "kernel": "decode_wide_kernel (split attention over the latent cache)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": (round(traffic / (ms_att * 1e-3) / 1e9, 1) if traffic else None),
                     "traffic_bytes_per_launch": traffic,
                     "alg_bytes_per_launch": alg_bytes,
                     "alg_flops_per_launch": attention_alg_flops(cfg, lengths),
                     "mfma_frac": round(attention_alg_flops(cfg, lengths) / (ms_att * 1e-3) / 1e12
                                        / MFMA_BF16_PEAK_TFS, 4),
                     "us_per_launch": round(ms_att * 1e3, 2)},
        "decode_call": {"us": round(ms_dec * 1e3, 2), "alg_bytes": decode_alg_bytes(cfg, lengths),
                        "alg_flops": decode_alg_flops(cfg, lengths),
                        "hbm_frac": round(decode_alg_bytes(cfg, lengths) / (ms_dec * 1e-3) / 1e9
                                          / HBM_PEAK_GBS, 4)},
        "beyond_attention": beyond,
        "cpu_baseline": cpu,
    }
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


if __name__ == "__main__":
    main()
