"""Benchmark: MLA absorbed decode (all four C-ABI calls) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

A step is one pass of the whole path -- absorb_q, decode, then the split merge and the value
projection (one fused call by default; --unfused runs merge_splits and out_proj) -- over one batch of a seeded synthetic DeepSeek-V2-shaped latent cache.  The cache and the
two weight matrices are held in several device copies ("layers") used round-robin, so a
step's inputs come from HBM rather than from the 256 MB on-chip Infinity Cache, as when
consecutive layers of a model run.  One replayed HIP graph holds 60 steps, one per layer of
the 60-layer model, as a serving loop captures a whole decode step.  Inputs are resident on
the device before timing.

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
# prefill workloads (no cached rows: T_q = T_k, causal) count the prompt tokens instead
PREFILL_METRIC = "MLA prefill tokens/s on 1 GPU (absorbed form, causal); % of bf16 MFMA peak"
PREFILL_UNIT = "prefill-tokens/s"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
ROW_BYTES = 1152               # one cached latent row [c_KV 512 ; k_R 64] in bf16
FLOP_PER_ROW_HEAD = 2 * 576 + 2 * 512   # score + weighted sum, per (row, query head)
MALL_BYTES = 256 << 20
MODEL_LAYERS = 60              # DeepSeek-V2's layers: the steps (or launches) one replayed graph holds
D_MODEL = 5120                 # DeepSeek-V2 hidden width: input of the decode prologue
D_CQ = 1536                    # DeepSeek-V2 compressed query width (W^UQ's input)
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


def host_facts():
    """The host the CPU baseline ran on: usable cores, CPU model, BLAS pool size."""
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):  # pragma: no cover - non-Linux
        affinity = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        blas = affinity
    return {"affinity_cores": int(affinity), "cpu_model": model, "blas_threads": int(blas)}


def cpu_baseline(w, budget_s: float):
    """Time the CPU oracle on the workload, in its two forms.

    - Naive (the pages' definition: materialized K/V per head), on a bounded sample: sequences
      in order, each head by head, until the time budget is spent; the rate is cached rows
      covered (a partly done sequence counts by its head fraction) per second.  This is `value`.
    - Absorbed (q_abs against the latent rows, split partials, merge, W^UV), over the whole
      workload, reported beside it.
    """
    import oracle as O
    from mla_latent_kv_20_amd import workloads as W
    facts = host_facts()
    w_uk, w_uv = w.f64("w_uk"), w.f64("w_uv")
    appended = w.q_per_seq if w.note == "appended" else 0
    covered, seqs, heads_last, t0 = 0.0, 0, 0, time.perf_counter()
    for b in range(w.batch):
        lo, hi = int(w.offsets[b]), int(w.offsets[b + 1])
        qs = slice(b * w.q_per_seq, (b + 1) * w.q_per_seq)
        c_kv, k_r = W.to_f64(w.c_kv[lo:hi], w.dtype), W.to_f64(w.k_r[lo:hi], w.dtype)
        q_c, q_r = W.to_f64(w.q_c[qs], w.dtype), W.to_f64(w.q_r[qs], w.dtype)
        heads = 0
        while heads < w.n_h:
            h = slice(heads, heads + 1)
            O.naive_decode(c_kv=c_kv, k_r=k_r, offsets=np.array([0, hi - lo], np.int64), q_c=q_c[:, h],
                           q_r=q_r[:, h], w_uk=w_uk[h], w_uv=w_uv[h], q_per_seq=w.q_per_seq)
            heads += 1
            if time.perf_counter() - t0 > budget_s:
                break
        covered += (hi - lo - appended if w.cached_rows() else w.q_per_seq) * heads / w.n_h
        seqs, heads_last = b + 1, heads
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    unit = UNIT if w.cached_rows() else PREFILL_UNIT
    total = float(w.cached_rows() if w.cached_rows() else w.n_q)
    # the absorbed form over every sequence (one at a time: bounded host memory)
    t1 = time.perf_counter()
    for b in range(w.batch):
        lo, hi = int(w.offsets[b]), int(w.offsets[b + 1])
        qs = slice(b * w.q_per_seq, (b + 1) * w.q_per_seq)
        O.absorbed_decode(c_kv=W.to_f64(w.c_kv[lo:hi], w.dtype), k_r=W.to_f64(w.k_r[lo:hi], w.dtype),
                          offsets=np.array([0, hi - lo], np.int64), q_c=W.to_f64(w.q_c[qs], w.dtype),
                          q_r=W.to_f64(w.q_r[qs], w.dtype), w_uk=w_uk, w_uv=w_uv, q_per_seq=w.q_per_seq,
                          num_splits=w.num_splits, split_rows=w.split_rows)
    dt_abs = time.perf_counter() - t1
    return {"value": covered / dt, "unit": unit, "cores": min(facts["blas_threads"], facts["affinity_cores"]),
            "kind": "oracle",
            "sample": f"sequences 0..{seqs - 1} of {w.batch} in order ({heads_last} of {w.n_h} heads of "
                      f"the last), naive fp64 form (materialized k^C, v^C), {covered:.0f} "
                      f"{'cached rows' if w.cached_rows() else 'prompt tokens'} "
                      f"in {dt:.1f} s; tokens/s over that sample",
            "absorbed": {"value": total / dt_abs, "unit": unit, "seconds": round(dt_abs, 2),
                         "sample": "the whole workload, absorbed fp64 form (q_abs against the latent rows, "
                                   "split partials, merge, W^UV), one sequence at a time"},
            **facts}


def measured_peaks(B, torch):
    """Achievable rates measured beside the published peaks: back-to-back bf16 MFMAs on every
    SIMD, a streaming read of 1 GiB (4x the Infinity Cache) in the decode's load form, and a
    plain 512 MiB device copy (read + write bytes).  Medians of 5 launches each."""
    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return sorted(ts)[len(ts) // 2]
    buf, flop = B.calib_mfma(4000)
    t_mfma = timed(lambda: B.calib_mfma(4000, buf))
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    rout, nread = B.calib_read(src, 256)
    t_read = timed(lambda: B.calib_read(src, 256, rout))
    half = src[: 512 << 20]
    dst = torch.empty_like(half)
    t_copy = timed(lambda: dst.copy_(half))
    del src, dst
    return {"mfma_bf16_TFLOPs": round(flop / t_mfma / 1e12, 1),
            "hbm_read_GBs": round(nread / t_read / 1e9, 1),
            "copy_GBs": round(2 * (512 << 20) / t_copy / 1e9, 1),
            "how": "bf16 MFMA 32x32x16, 4 chains per wave, 1024 workgroups; streaming read of 1 GiB by 256 "
                   "workgroups in 36 KiB direct-to-LDS tiles; 512 MiB device copy counted as read + write"}


def copy_calibration(mib: int, reps: int) -> None:
    """A plain device copy of known size, to scale HBM byte counters read under a profiler."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "reps": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--config", default="dsv2_b32_t4096")
    ap.add_argument("--copies", type=int, default=0, help="layer copies (0: enough to exceed 2x MALL)")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--split-rows", type=int, default=0)
    ap.add_argument("--plan", choices=["config", "auto"], default="config",
                    help="split plan: the workload's own, or mla_plan_splits on its lengths (auto)")
    ap.add_argument("--partials", choices=["auto", "f32", "f16"], default="auto",
                    help="storage of split results (auto: fp16 when there is a merge)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of graph replay")
    ap.add_argument("--unfused", action="store_true",
                    help="step with mla_merge_splits + mla_out_proj instead of mla_merge_out_proj")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the decode shards by sequence with no exchange; see the design notes).", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration, 5)
        return

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
    d = B.dims(w.n_h, w.d_h, w.d_c, w.d_r, B.MLA_BF16 if w.dtype == W.BF16 else B.MLA_F32)
    S, R = (B.plan_splits(d, w.offsets, w.batch, w.q_per_seq) if args.plan == "auto"
            else (w.num_splits, w.split_rows))
    S = args.num_splits or S
    R = args.split_rows or R
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

    fused = not args.unfused

    def step(i):
        L = layers[i % copies]
        qa = B.absorb_q(d, L["q_c"], L["q_r"], L["w_uk"], bufs["q_abs"])
        op, lp = B.decode(d, qa, L["cache"][:, :w.d_c], L["cache"][:, w.d_c:], L["offsets"], w.batch,
                          w.q_per_seq, S, R, bufs["o_part"], bufs["lse_part"])
        if S == 1 and part == B.MLA_F32:        # one fp32 split: the decode's output is final
            B.out_proj(d, op[0], L["w_uv"], bufs["o_c"])
            return
        if fused:
            B.merge_out_proj(d, op, lp, L["w_uv"], bufs["o_c"], bufs["lse"], None)
            return
        if S > 1 or part != B.MLA_F32:
            o_lat, _ = B.merge_splits(d, op, lp, bufs["o_lat"], bufs["lse"])
        else:
            o_lat = op[0]
        B.out_proj(d, o_lat, L["w_uv"], bufs["o_c"])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps

    # Whole-step throughput: one HIP graph holds MODEL_LAYERS steps, one per layer of the
    # model (a serving loop captures a model's layers), cycling over the layer copies, and is
    # replayed; a second graph holds the K % n_graph remaining steps, so exactly K steps are
    # timed.
    n_graph = copies * max(1, math.ceil(MODEL_LAYERS / copies))
    if not args.no_graph:
        def capture(n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for c in range(n):
                    step(c)
            return g
        g_all = capture(n_graph)
        g_rest = capture(K % n_graph) if K % n_graph else None
        for i in range(max(1, args.warmup // n_graph)):
            g_all.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        g0.record()
        for i in range(K // n_graph):
            g_all.replay()
        if g_rest is not None:
            g_rest.replay()
        g1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        graph_ms = g0.elapsed_time(g1) / K

    if args.no_graph:
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        g0.record()
        for i in range(K):
            step(i)
        g1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        graph_ms = g0.elapsed_time(g1) / K
    ms_per_step = graph_ms
    cached = w.cached_rows()
    prefill = cached == 0
    tokens = w.n_q if prefill else cached          # the unit of every rate below
    value = tokens / (ms_per_step * 1e-3)

    # Each kernel alone: launches over the layer copies captured as one HIP graph and replayed,
    # so the mean is GPU time per launch (dispatch gaps included, no host launch cost).  The
    # weight-only kernels cycle over enough weight copies to exceed twice the MALL, as their
    # weights would come from HBM in a model's step.  The decode's mean is the roofline's
    # duration.
    w_bytes = w.n_h * w.d_h * w.d_c * esz
    wcopies = max(copies, math.ceil(2 * MALL_BYTES / w_bytes))
    w_uk_set = [L["w_uk"] for L in layers] + [base["w_uk"].clone() for _ in range(wcopies - copies)]
    w_uv_set = [L["w_uv"] for L in layers] + [base["w_uv"].clone() for _ in range(wcopies - copies)]
    calls = {
        "absorb_q": (wcopies, lambda j: B.absorb_q(d, base["q_c"], base["q_r"], w_uk_set[j], bufs["q_abs"])),
        "decode": (copies, lambda j: B.decode(d, bufs["q_abs"], layers[j]["cache"][:, :w.d_c],
                                              layers[j]["cache"][:, w.d_c:], layers[j]["offsets"], w.batch,
                                              w.q_per_seq, S, R, bufs["o_part"], bufs["lse_part"])),
        "merge": (1, lambda j: B.merge_splits(d, bufs["o_part"], bufs["lse_part"], bufs["o_lat"], bufs["lse"]))
        if (S > 1 or part != B.MLA_F32) else None,
        "out_proj": (wcopies, lambda j: B.out_proj(d, bufs["o_lat"], w_uv_set[j], bufs["o_c"])),
        "merge_out_proj": (wcopies, lambda j: B.merge_out_proj(d, bufs["o_part"], bufs["lse_part"], w_uv_set[j],
                                                                bufs["o_c"], bufs["lse"], None))
        if d.dtype == B.MLA_BF16 else None,
    }
    # Decode prologue (one new token per query, DeepSeek-V2 hidden width): the new rows go to
    # a buffer of their own so that the measured caches stay as drawn.
    prologue = d.dtype == B.MLA_BF16 and (w.d_c + w.d_r) % 32 == 0
    if prologue:
        pw_bytes = (w.d_c + w.d_r) * D_MODEL * esz
        pcopies = math.ceil(2 * MALL_BYTES / pw_bytes)
        gen = torch.Generator(device=dev).manual_seed(7)
        h_new = (torch.randn((n_q, D_MODEL), generator=gen, device=dev)).to(base["q_c"].dtype)
        w_down = [(torch.randn((w.d_c + w.d_r, D_MODEL), generator=gen, device=dev) / math.sqrt(D_MODEL))
                  .to(base["q_c"].dtype) for _ in range(pcopies)]
        pos_new = torch.from_numpy(np.diff(w.offsets).astype(np.int64)).to(dev).repeat_interleave(w.q_per_seq)
        new_rows = torch.empty((n_q, w.d_c + w.d_r), dtype=base["q_c"].dtype, device=dev)
        dst_new = torch.arange(n_q, dtype=torch.int64, device=dev)
        ws_new = torch.empty(max(1, B.kv_append_workspace_bytes(d, n_q)), dtype=torch.uint8, device=dev)
        calls["kv_append"] = (pcopies, lambda j: B.kv_append(d, h_new, w_down[j][:w.d_c], w_down[j][w.d_c:],
                                                              pos_new, dst_new, new_rows, workspace=ws_new))
        calls["absorb_q_rope"] = (wcopies, lambda j: B.absorb_q_rope(d, base["q_c"], base["q_r"], w_uk_set[j],
                                                                      pos_new, bufs["q_abs"]))
    # Quantized cache (E4M3 codes, one scale per row): each layer copy's cache quantized into
    # code buffers of its own, enough of them to exceed twice the MALL; the decode alone and
    # the step absorb_q, decode_fp8, merge_out_proj.
    fp8 = d.dtype == B.MLA_BF16 and w.d_c == 512 and w.d_r == 64 and w.n_h % 32 == 0
    if fp8:
        code_bytes = w.rows * (w.d_c + w.d_r + 4)
        fcopies = max(copies, math.ceil(2 * MALL_BYTES / code_bytes))
        fp8_sets = [B.quantize_rows_fp8(d, layers[j % copies]["cache"]) for j in range(fcopies)]
        torch.cuda.synchronize()

        def fp8_decode(j):
            return B.decode_fp8(d, bufs["q_abs"], fp8_sets[j][0], fp8_sets[j][1], base["offsets"], w.batch,
                                w.q_per_seq, S, R, bufs["o_part"], bufs["lse_part"])

        def fp8_step(j):
            L = layers[j % copies]
            qa = B.absorb_q(d, L["q_c"], L["q_r"], L["w_uk"], bufs["q_abs"])
            op, lp = B.decode_fp8(d, qa, fp8_sets[j][0], fp8_sets[j][1], L["offsets"], w.batch, w.q_per_seq,
                                  S, R, bufs["o_part"], bufs["lse_part"])
            if S == 1 and part == B.MLA_F32:
                B.out_proj(d, op[0], L["w_uv"], bufs["o_c"])
            else:
                B.merge_out_proj(d, op, lp, L["w_uv"], bufs["o_c"], bufs["lse"], None)

        calls["decode_fp8"] = (fcopies, fp8_decode)
        calls["step_fp8"] = (fcopies, fp8_step)
    # Weight folding (c^Q -> absorbed query, o_lat -> block output), unfolded against folded,
    # at DeepSeek-V2's d_cq and d_model; each weight cycles over enough copies to exceed twice
    # the MALL.
    fold = d.dtype == B.MLA_BF16 and w.d_c % 128 == 0 and (w.n_h * w.d_h) % 128 == 0
    if fold:
        gen = torch.Generator(device=dev).manual_seed(11)
        bf16 = base["q_c"].dtype

        def randw(shape, fan):
            return (torch.randn(shape, generator=gen, device=dev) / math.sqrt(fan)).to(bf16)

        def copies_for(nbytes):
            return max(1, math.ceil(2 * MALL_BYTES / nbytes))

        c_q = torch.randn((n_q, D_CQ), generator=gen, device=dev).to(bf16)
        ucop = copies_for(w.n_h * w.d_h * D_CQ * esz)
        w_uq_set = [randw((w.n_h, w.d_h, D_CQ), D_CQ) for _ in range(ucop)]
        gcop = copies_for(w.n_h * w.d_c * D_CQ * esz)
        g_set = [B.fold_q(d, w_uq_set[j % ucop], base["w_uk"]) for j in range(gcop)]
        ocop = copies_for(D_MODEL * w.n_h * w.d_h * esz)
        w_o_set = [randw((D_MODEL, w.n_h * w.d_h), w.n_h * w.d_h) for _ in range(ocop)]
        fcop = copies_for(D_MODEL * w.n_h * w.d_c * esz)
        wf_set = [B.fold_o(d, w_o_set[j % ocop], base["w_uv"]) for j in range(fcop)]
        torch.cuda.synchronize()
        q_c_buf = torch.empty((n_q, w.n_h, w.d_h), dtype=bf16, device=dev)
        u_buf = torch.empty((n_q, D_MODEL), dtype=bf16, device=dev)
        pws = torch.empty(max(1, B.proj_workspace_bytes(d, n_q, D_MODEL, D_CQ)), dtype=torch.uint8, device=dev)
        calls["q_up"] = (ucop, lambda j: B.q_up(d, c_q, w_uq_set[j], q_c_buf, pws))
        calls["absorb_q_folded"] = (gcop, lambda j: B.absorb_q_folded(d, c_q, g_set[j], base["q_r"], bufs["q_abs"]))
        calls["o_proj"] = (ocop, lambda j: B.o_proj(d, bufs["o_c"], w_o_set[j], u_buf, pws))
        calls["out_folded"] = (fcop, lambda j: B.out_folded(d, bufs["o_lat"], wf_set[j], u_buf, pws))
    per = {}
    for name, item in calls.items():
        if item is None:
            continue
        n, fn = item
        for j in range(n):
            fn(j)
        torch.cuda.synchronize()
        # At least MODEL_LAYERS launches per replay (each copy equally often): the gap between
        # two replays is then shared by that many launches, as in the whole-step graph.
        m = n * max(1, math.ceil(MODEL_LAYERS / n))
        reps = max(1, K // m)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if args.no_graph:                  # eager launches (counter runs): host cost may show
            e0.record()
            for _ in range(reps):
                for j in range(m):
                    fn(j % n)
            e1.record()
        else:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for j in range(m):
                    fn(j % n)
            g.replay()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
        torch.cuda.synchronize()
        per[name] = e0.elapsed_time(e1) / (reps * m)

    # Spread of the step time: a separate pass of replays of the all-layers graph, one event
    # between replays (the headline above is timed without them).
    spread = None
    if not args.no_graph:
        n_rep = max(5, min(50, K // n_graph))
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_rep + 1)]
        evs[0].record()
        for r in range(n_rep):
            g_all.replay()
            evs[r + 1].record()
        torch.cuda.synchronize()
        st = sorted(evs[r].elapsed_time(evs[r + 1]) * 1e3 / n_graph for r in range(n_rep))
        pick = lambda q: round(st[min(n_rep - 1, int(round(q * (n_rep - 1))))], 2)
        spread = {"replays": n_rep, "steps_per_replay": n_graph, "p10_us": pick(0.1), "median_us": pick(0.5),
                  "p90_us": pick(0.9)}

    # The decode with its cache resident in the Infinity Cache: every launch reads the first
    # copy (reported beside the cold figure, never as it).
    warm_ms = None
    if not args.no_graph and w.rows * ROW_BYTES <= MALL_BYTES * 3 // 4:
        _, fn = calls["decode"]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(copies):
                fn(0)
        g.replay()
        torch.cuda.synchronize()
        reps = max(1, K // copies)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        warm_ms = e0.elapsed_time(e1) / (reps * copies)

    dec_ms = per["decode"]
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
    peaks = measured_peaks(B, torch)
    mpk = peaks["hbm_read_GBs"] if roof["bound"] == "hbm" else peaks["mfma_bf16_TFLOPs"]
    roof["measured_peak"] = mpk
    roof["frac_of_measured"] = round(roof["achieved"] / mpk, 4)
    roof["traffic"] = measured_traffic(args.config)
    roof["kernel"] = "mla_decode_bf16_kernel"
    roof["algorithmic_bytes_per_launch"] = dec_bytes
    roof["algorithmic_flop_per_launch"] = flops

    out = {
        "metric": PREFILL_METRIC if prefill else METRIC, "value": round(value, 1),
        "unit": PREFILL_UNIT if prefill else UNIT, "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if w.dtype == W.BF16 else "f32",
        "data": "synthetic (seeded Gaussian latent cache, DeepSeek-V2 attention dims, random weights)",
        "config": {"workload": args.config, "batch": w.batch, "seq_len": int(w.lengths.max()),
                   "cached_rows": cached, "q_per_seq": w.q_per_seq, "n_h": w.n_h, "d_h": w.d_h,
                   "d_c": w.d_c, "d_r": w.d_r, "num_splits": S, "split_rows": R, "plan": args.plan, "layer_copies": copies,
                   "partials": {B.MLA_F32: "f32", B.MLA_F16: "f16"}[part]},
        "roofline": roof,
        "kernels_ms_mean": {n: round(v, 5) for n, v in per.items()},
        "prologue": ({"kv_append": {"n_new": n_q, "d_model": D_MODEL,
                                    "algorithmic_bytes": (w.d_c + w.d_r) * D_MODEL * esz + n_q * D_MODEL * esz
                                    + n_q * (w.d_c + w.d_r) * esz + 16 * n_q,
                                    "GB_per_s": round(((w.d_c + w.d_r) * D_MODEL * esz + n_q * D_MODEL * esz
                                                       + n_q * (w.d_c + w.d_r) * esz + 16 * n_q)
                                                      / (per["kv_append"] * 1e-3) / 1e9, 1)},
                      "absorb_q_rope_ms": round(per["absorb_q_rope"], 5)} if prologue else None),
        "fp8_cache": (fp8_summary(w, per, flops, tokens, fcopies) if fp8 else None),
        "folding": (fold_summary(w, per, esz) if fold else None),
        "decode_merge_tokens_per_s": round(tokens / ((dec_ms + per.get("merge", 0.0)) * 1e-3), 1),
        "timing": (f"hip graph replay ({n_graph} steps per graph, one per model layer, cycling over {copies} layer copies)"
                   if not args.no_graph else "eager launches"),
        "step_calls": ("absorb_q, decode, out_proj (one fp32 split: no merge)" if S == 1 and part == B.MLA_F32
                       else "absorb_q, decode, merge_out_proj" if fused else "absorb_q, decode, merge_splits, out_proj"),
        "mfma_frac_decode": round(flops / (dec_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "measured_peaks": peaks,
        "wall_ms_per_step": round(wall * 1e3 / K, 5),
        "step_spread": spread,
        "decode_warm_ms": round(warm_ms, 5) if warm_ms is not None else None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def fold_summary(w, per, esz):
    """Unfolded against folded weights, per step, from c^Q and from o_lat."""
    uq = w.n_h * w.d_h * D_CQ * esz
    uk = w.n_h * w.d_h * w.d_c * esz
    g = w.n_h * w.d_c * D_CQ * esz
    wo = D_MODEL * w.n_h * w.d_h * esz
    wf = D_MODEL * w.n_h * w.d_c * esz
    q_unf = per["q_up"] + per["absorb_q"]
    o_unf = per["out_proj"] + per["o_proj"]
    return {"d_cq": D_CQ, "d_model": D_MODEL,
            "query": {"unfolded_ms": round(q_unf, 5), "q_up_ms": round(per["q_up"], 5),
                      "absorb_q_ms": round(per["absorb_q"], 5), "folded_ms": round(per["absorb_q_folded"], 5),
                      "unfolded_weight_bytes": uq + uk, "folded_weight_bytes": g,
                      "folded_GB_per_s": round(g / (per["absorb_q_folded"] * 1e-3) / 1e9, 1)},
            "output": {"unfolded_ms": round(o_unf, 5), "out_proj_ms": round(per["out_proj"], 5),
                       "o_proj_ms": round(per["o_proj"], 5), "folded_ms": round(per["out_folded"], 5),
                       "unfolded_weight_bytes": uk + wo, "folded_weight_bytes": wf,
                       "folded_GB_per_s": round(wf / (per["out_folded"] * 1e-3) / 1e9, 1)}}


def fp8_summary(w, per, flops, cached, fcopies):
    """The quantized-cache decode: E4M3 codes (576 B) and a 4-byte scale per row."""
    ms = per["decode_fp8"]
    nbytes = w.rows * (w.d_c + w.d_r + 4) + w.n_q * w.n_h * (w.d_c + w.d_r) * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    tfs = flops / (ms * 1e-3) / 1e12
    return {"format": "e4m3 codes + fp32 scale per row", "code_copies": fcopies,
            "decode_ms": round(ms, 5), "step_ms": round(per["step_fp8"], 5),
            "step_tokens_per_s": round(cached / (per["step_fp8"] * 1e-3), 1),
            "algorithmic_bytes_per_launch": nbytes, "GB_per_s": round(gbs, 1),
            "hbm_frac": round(gbs / PEAK_HBM_GBS, 4), "TFLOP_per_s": round(tfs, 1),
            "mfma_frac": round(tfs / PEAK_BF16_TFLOPS, 4),
            "bound": "mfma" if flops / nbytes > PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9) else "hbm"}


if __name__ == "__main__":
    main()
