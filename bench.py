"""Benchmark: MLA absorbed decode (all four C-ABI calls) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

A step is one pass of the whole path -- absorb_q, decode, merge (when split), out_proj --
over one batch of a seeded synthetic DeepSeek-V2-shaped latent cache.  The cache and the
two weight matrices are held in several device copies ("layers") used round-robin, so a
step's inputs come from HBM rather than from the 256 MB on-chip Infinity Cache, as when
consecutive layers of a model run.  Inputs are resident on the device before timing.

Prints one JSON line: throughput in cached latent tokens per second over the whole step,
the decode kernel's roofline fraction (HIP-event timing inside the timed region), and the
CPU oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MLA decode cached-latent-tokens/s on 1 GPU; % of HBM BW and bf16 MFMA peak"
UNIT = "cached-latent-tokens/s"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
ROW_BYTES = 1152               # one cached latent row [c_KV 512 ; k_R 64] in bf16
FLOP_PER_ROW_HEAD = 2 * 576 + 2 * 512   # score + weighted sum, per (row, query head)
MALL_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "mla_latent_kv_20_amd", "csrc", f)
                  for f in ("decode_bf16.hip", "mla_common.h")]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per decode launch from the committed counter summary, if still current."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    rec = t.get(workload)
    if not rec or rec.get("kernel_hash") != kernel_hash():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, budget_s: float):
    """Time the oracle's defining (materialized K/V) form on a bounded sample of the workload."""
    import oracle as O
    from mla_latent_kv_20_amd import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        threads = os.cpu_count() or 1
    b = 0
    lo, hi = int(w.offsets[b]), int(w.offsets[b + 1])
    rows = np.arange(lo, hi)
    a = dict(c_kv=W.to_f64(w.c_kv[rows], w.dtype), k_r=W.to_f64(w.k_r[rows], w.dtype),
             offsets=np.array([0, hi - lo], np.int64),
             q_c=W.to_f64(w.q_c[:w.q_per_seq], w.dtype), q_r=W.to_f64(w.q_r[:w.q_per_seq], w.dtype),
             w_uk=w.f64("w_uk"), w_uv=w.f64("w_uv"), q_per_seq=w.q_per_seq)
    heads_done, t0 = 0, time.perf_counter()
    # heads one at a time until the budget is spent (at least one head)
    while heads_done < w.n_h:
        sub = dict(a, q_c=a["q_c"][:, heads_done:heads_done + 1], q_r=a["q_r"][:, heads_done:heads_done + 1],
                   w_uk=a["w_uk"][heads_done:heads_done + 1], w_uv=a["w_uv"][heads_done:heads_done + 1])
        O.naive_decode(**sub)
        heads_done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    cached = (hi - lo) - (w.q_per_seq if w.note == "appended" else 0)
    value = cached * (heads_done / w.n_h) / dt
    return {"value": value, "unit": UNIT, "cores": int(threads), "kind": "oracle",
            "sample": f"sequence 0 ({hi - lo} rows), {heads_done} of {w.n_h} heads, naive fp64 "
                      f"form (materialized k^C, v^C); {dt:.1f} s; tokens/s scaled by the head fraction"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--config", default="dsv2_b32_t4096")
    ap.add_argument("--copies", type=int, default=0, help="layer copies (0: enough to exceed 2x MALL)")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--split-rows", type=int, default=0)
    ap.add_argument("--partials", choices=["auto", "f32", "f16"], default="auto",
                    help="storage of split results (auto: fp16 when there is a merge)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the decode shards by sequence with no exchange; see the design notes).", file=sys.stderr)
        sys.exit(2)

    import torch
    from mla_latent_kv_20_amd import binding as B
    from mla_latent_kv_20_amd import device as D
    from mla_latent_kv_20_amd import workloads as W

    if not os.path.exists(B.LIB_PATH):
        from mla_latent_kv_20_amd import build
        build.build()
    B.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")

    w = W.make_config(args.config)
    S = args.num_splits or w.num_splits
    R = args.split_rows or w.split_rows
    d = B.dims(w.n_h, w.d_h, w.d_c, w.d_r, B.MLA_BF16 if w.dtype == W.BF16 else B.MLA_F32)
    esz = 2 if w.dtype == W.BF16 else 4
    layer_bytes = w.rows * (w.d_c + w.d_r) * esz + 2 * w.n_h * w.d_h * w.d_c * esz
    copies = args.copies or max(2, math.ceil(2 * MALL_BYTES / layer_bytes))
    print(f"bench: {args.config} rows={w.rows} splits={S} split_rows={R} copies={copies}",
          file=sys.stderr, flush=True)

    base = D.to_device(w, dev)
    layers = [base] + [dict(base, cache=base["cache"].clone(), w_uk=base["w_uk"].clone(),
                            w_uv=base["w_uv"].clone()) for _ in range(copies - 1)]
    n_q = w.n_q
    part = B.default_partial_dtype(d, S) if args.partials == "auto" else \
        {"f32": B.MLA_F32, "f16": B.MLA_F16}[args.partials]
    bufs = dict(q_abs=torch.empty((n_q, w.n_h, w.d_c + w.d_r), dtype=base["q_c"].dtype, device=dev),
                o_part=torch.empty((S, n_q, w.n_h, w.d_c), dtype=B._torch_dtype(part), device=dev),
                lse_part=torch.empty((S, n_q, w.n_h), dtype=torch.float32, device=dev),
                o_lat=torch.empty((n_q, w.n_h, w.d_c), dtype=torch.float32, device=dev),
                lse=torch.empty((n_q, w.n_h), dtype=torch.float32, device=dev),
                o_c=torch.empty((n_q, w.n_h, w.d_h), dtype=base["q_c"].dtype, device=dev))

    def step(i, ev=None):
        L = layers[i % copies]
        if ev is not None:
            ev[0].record()
        qa = B.absorb_q(d, L["q_c"], L["q_r"], L["w_uk"], bufs["q_abs"])
        if ev is not None:
            ev[1].record()
        op, lp = B.decode(d, qa, L["cache"][:, :w.d_c], L["cache"][:, w.d_c:], L["offsets"], w.batch,
                          w.q_per_seq, S, R, bufs["o_part"], bufs["lse_part"])
        if ev is not None:
            ev[2].record()
        if S > 1 or part != B.MLA_F32:
            o_lat, _ = B.merge_splits(d, op, lp, bufs["o_lat"], bufs["lse"])
        else:
            o_lat = op[0]
        if ev is not None:
            ev[3].record()
        B.out_proj(d, o_lat, L["w_uv"], bufs["o_c"])
        if ev is not None:
            ev[4].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    K = args.steps
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    names = ["absorb_q", "decode", "merge", "out_proj"]
    per = {n: np.array([events[i][j].elapsed_time(events[i][j + 1]) for i in range(K)])
           for j, n in enumerate(names)}
    step_ms = np.array([events[i][0].elapsed_time(events[i][4]) for i in range(K)])
    span_ms = events[0][0].elapsed_time(events[K - 1][4])
    ms_per_step = span_ms / K
    cached = w.cached_rows()
    value = cached / (ms_per_step * 1e-3)

    dec_ms = float(per["decode"].mean())
    dec_bytes = cached * ROW_BYTES + (w.rows - cached) * ROW_BYTES
    flops = float(FLOP_PER_ROW_HEAD) * w.n_h * sum(
        (int(L) - w.q_per_seq + r + 1) for L in w.lengths for r in range(w.q_per_seq))
    intensity = flops / dec_bytes
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if intensity < ridge:
        achieved = dec_bytes / (dec_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    else:
        achieved = flops / (dec_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    roof["traffic"] = measured_traffic(args.config)
    roof["kernel"] = "mla_decode_bf16_kernel"
    roof["algorithmic_bytes_per_launch"] = dec_bytes
    roof["algorithmic_flop_per_launch"] = flops

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": UNIT, "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if w.dtype == W.BF16 else "f32",
        "data": "synthetic (seeded Gaussian latent cache, DeepSeek-V2 attention dims, random weights)",
        "config": {"workload": args.config, "batch": w.batch, "seq_len": int(w.lengths.max()),
                   "cached_rows": cached, "q_per_seq": w.q_per_seq, "n_h": w.n_h, "d_h": w.d_h,
                   "d_c": w.d_c, "d_r": w.d_r, "num_splits": S, "split_rows": R, "layer_copies": copies,
                   "partials": {B.MLA_F32: "f32", B.MLA_F16: "f16"}[part]},
        "roofline": roof,
        "kernels_ms": {n: round(float(v.mean()), 5) for n, v in per.items()},
        "decode_merge_tokens_per_s": round(cached / ((per["decode"].mean() + per["merge"].mean()) * 1e-3), 1),
        "step_ms_p10_p50_p90": [round(float(np.percentile(step_ms, q)), 5) for q in (10, 50, 90)],
        "mfma_frac_decode": round(flops / (dec_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "wall_ms_per_step": round(wall * 1e3 / K, 5),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
