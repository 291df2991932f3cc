"""Benchmark of the block-scaled fp8 small-M GEMM on one MI355X.

Default workload (one JSON line on stdout): the wo_a decode/verify shape at 6 rows, G=2 groups of
[1024 x 4096] e4m3 weights with 32x32 exponent blocks, bf16 activations [6, 8192], bf16 output
[6, 2, 1024], the built-in split-K plan. A step is one GEMM call on one weight copy; the calls
cycle through enough distinct weight copies (>= 512 MiB, twice the 256 MiB Infinity Cache) that
every call streams its weights from HBM. The timed calls are captured once in a HIP graph and
replayed (as the pages time their kernels), between a synchronize and HIP events on both sides.

value = effective weight-stream GB/s = (e4m3 bytes + exponent bytes) / time per call.
roofline.achieved = algorithmic bytes (weights + exponents + X + Y) / time per call.
The time per call is the timed graph replay (HIP events on the launch stream around it) divided
by the number of calls in it: the average launch duration, gaps between launches included, which
rocprofv3's average kernel duration for the same command matches within a few percent. HIP events
around single eager calls are also reported; they include host launch gaps.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--m M]
       [--no-cpu-baseline] [--all FILE]
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "us/call and effective weight-stream GB/s (% of HBM peak), M=6 block-fp8 GEMM"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
COLD_BYTES = 512 << 20
# The pages' own figure for this workload (other hardware, context): on GB10 the twin path ran
# 43 wo_a layers at 6 rows in 2.20 ms, i.e. 51.2 us/call, about 164 GB/s of weight stream.
PAGES_GBS = 8_396_800 / (2.20e-3 / 43) / 1e9

WORKLOADS = {
    # name: (G, N, K, default M, exponent byte range, out dtype, description)
    "wo_a": (2, 1024, 4096, 6, (115, 125), "bf16",
             "wo_a small-batch decode: X bf16 [M, 2*4096], W e4m3 [2,1024,4096] + u8 exponents [2,32,128]"),
    "wo_a_mid": (2, 1024, 4096, 64, (115, 125), "bf16",
                 "wo_a mid path: X bf16 [M, 2*4096], W e4m3 [2,1024,4096] + u8 exponents [2,32,128]"),
    "wo_a_tp3": (4, 1024, 4096, 6, (115, 123), "bf16",
                 "wo_a padded-TP3 shard: X bf16 [M, 4*4096], W e4m3 [4,1024,4096] + u8 exponents [4,32,128]"),
    "shared_down": (1, 5120, 576, 6, (117, 123), "bf16",
                    "shared-expert down_proj: X bf16 [M, 576], W e4m3 [5120, 576] + u8 exponents [160, 18]"),
    "shared_down_pad": (1, 5120, 640, 6, (117, 123), "bf16",
                        "shared-expert down_proj, K zero-padded 576->640"),
    "lm_head": (1, 32768, 5120, 128, (118, 122), "f32",
                "draft LM head: X bf16 [M, 5120], W e4m3 [32768, 5120] + u8 exponents [1024, 160], fp32 logits"),
    "main_proj": (1, 1280, 5120, 16, (115, 125), "bf16",
                  "draft main_proj shard (row-scale twin): X bf16 [M, 5120], W e4m3 [1280, 5120] + u8 exponents "
                  "per row and 32 columns [1280, 160]"),
}
ROW_SCALE_WORKLOADS = {"main_proj"}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--workload", default="wo_a", choices=sorted(WORKLOADS))
    p.add_argument("--m", type=int, default=None)
    p.add_argument("--split-k", type=int, default=0)
    p.add_argument("--path", default="bf16", choices=["bf16", "mx", "mxfp8"],
                   help="bf16: the exact twin GEMM (default); mx: the fp8 x fp8 GEMM on MXFP8 activations; "
                        "mxfp8: the exact twin GEMM with the MXFP8 output epilogue")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--all", default=None, help="also time every workload and row count; write JSON lines here")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB, 20 times (counter calibration)")
    return p.parse_args()


def algorithmic_bytes(M, G, N, K, out_bytes, row_scales=False):
    w = G * N * K
    e = G * N * (K // 32) if row_scales else G * (N // 32) * (K // 32)
    return w, e, M * G * K * 2, M * G * N * out_bytes


def make_copies(torch, B, G, N, K, elo, ehi, n_copies, seed, row_scales=False):
    """Seeded synthetic weight copies on the device: e4m3 codes uniform over the finite codes,
    exponent bytes uniform in [elo, ehi] (one per 32x32 block, or per row and 32 columns)."""
    erows = N if row_scales else N // 32
    import synthetic as S
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    table = torch.from_numpy(S.FINITE_E4M3_CODES).cuda()
    qs, es = [], []
    for i in range(n_copies):
        idx = torch.randint(0, table.numel(), (G, N, K), generator=gen, device="cuda", dtype=torch.int32)
        qs.append(table[idx])
        es.append(torch.randint(elo, ehi + 1, (G, erows, K // 32), generator=gen, device="cuda",
                                dtype=torch.int32).to(torch.uint8))
        del idx
    return qs, es


def graph_us(torch, fn, steps):
    """Average time per call of `steps` calls of fn(i) captured in one HIP graph and replayed
    between HIP events on the replay stream (the first replay uploads the graph, untimed)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for i in range(steps):
                fn(i)
    torch.cuda.current_stream().wait_stream(side)
    graph.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    graph.replay()
    t1.record()
    torch.cuda.synchronize()
    del graph
    return 1e3 * t0.elapsed_time(t1) / steps


def time_workload(name, M, steps, warmup, split_k=0, path="bf16"):
    """path "bf16": the exact twin GEMM (bsfp8_gemm). path "mx": the fp8 x fp8 GEMM
    (bsfp8_gemm_mx) on activations quantized once before the timed region; the quantizer is timed
    on its own and reported as quantize_us. path "mxfp8": the twin GEMM with the MXFP8 output
    epilogue (bsfp8_gemm_mxfp8: GEMM + fused sum-and-quantise kernel per call)."""
    import torch
    import block_scaled_fp8_skinny_amd as B
    import synthetic as S

    G, N, K, _, (elo, ehi), out, desc = WORKLOADS[name]
    row_scales = name in ROW_SCALE_WORKLOADS
    out_bytes = 4 if out == "f32" else 2
    w_b, e_b, x_b, y_b = algorithmic_bytes(M, G, N, K, out_bytes, row_scales)
    if path == "mx":
        x_b = M * G * K + M * G * K // 32             # e4m3 codes + scale bytes
    if path == "mxfp8":
        y_b = M * G * N + M * G * N // 32             # e4m3 codes + scale bytes of the output
    copy_bytes = w_b + e_b
    n_copies = max(4, min(steps, math.ceil(COLD_BYTES / copy_bytes)))
    qs, es = make_copies(torch, B, G, N, K, elo, ehi, n_copies, seed=7000 + M, row_scales=row_scales)
    x = torch.from_numpy(S.bf16_normal(S.rng(7100 + M), (M, G * K)).view("int16")).view(torch.bfloat16).cuda()
    if row_scales:
        ws = B.workspace_row32(M, G, N, K, split_k)
    else:
        ws = B.workspace(M, G, N, K, split_k) if path == "bf16" else None
    y = torch.empty((M, G, N), dtype=torch.float32 if out == "f32" else torch.bfloat16, device="cuda")
    quant_us = None
    if path == "mx":
        xq, xs = B.bsfp8_quantize_mx(x)
        plan = {"mx_cfg": B.bsfp8_mx_plan(M, G, N), **B.bsfp8_mx_config_info(B.bsfp8_mx_plan(M, G, N))}

        def call(i):
            B.bsfp8_gemm_mx(xq, xs, qs[i % n_copies], es[i % n_copies], out=y, out_dtype=out)

        for i in range(20):
            B.bsfp8_quantize_mx(x, xq=xq, xs=xs)
        quant_us = graph_us(torch, lambda i: B.bsfp8_quantize_mx(x, xq=xq, xs=xs), min(steps, 1000))
    elif row_scales:
        plan = {"row_scale_twin": True}

        def call(i):
            B.bsfp8_gemm_row32(x, qs[i % n_copies], es[i % n_copies], split_k=split_k, ws=ws, out=y, out_dtype=out)
    elif path == "mxfp8":
        plan = B.bsfp8_plan_info(M, G, N, K, split_k, path=3)
        ws = B.workspace_mxfp8(M, G, N, K, split_k)
        yq = torch.empty((M, G * N), dtype=torch.uint8, device="cuda")
        ys = torch.empty((M, G * N // 32), dtype=torch.uint8, device="cuda")

        def call(i):
            B.bsfp8_gemm_mxfp8(x, qs[i % n_copies], es[i % n_copies], split_k=split_k, ws=ws, yq=yq, ys=ys)
    else:
        plan = B.bsfp8_plan_info(M, G, N, K, split_k)

        def call(i):
            B.bsfp8_gemm(x, qs[i % n_copies], es[i % n_copies], split_k=split_k, ws=ws, out=y, out_dtype=out)

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()

    # (1) kernel duration: HIP events around each call on the launch stream
    stream = torch.cuda.current_stream()
    n_ev = min(steps, 1000)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_ev)]
    for i in range(n_ev):
        evs[2 * i].record(stream)
        call(i)
        evs[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    kern_ms = sorted(evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(n_ev))
    kern_us_mean = 1e3 * sum(kern_ms) / n_ev
    kern_us_median = 1e3 * kern_ms[n_ev // 2]

    # (2) wall time per call: all `steps` calls captured in one graph, replayed once
    wall_us = graph_us(torch, call, steps)
    wall_ms = wall_us * steps / 1e3
    res = dict(workload=name, path=path, desc=desc, M=M, G=G, N=N, K=K, out=out, plan=plan, copies=n_copies,
               copy_bytes=copy_bytes, wall_us_per_call=wall_us, kernel_us_mean=kern_us_mean,
               kernel_us_median=kern_us_median, weight_stream_gbs_wall=copy_bytes / (wall_us * 1e3),
               algorithmic_bytes=w_b + e_b + x_b + y_b, flops=2 * M * G * N * K,
               algorithmic_gbs=(w_b + e_b + x_b + y_b) / (wall_us * 1e3),
               tflops=2 * M * G * N * K / (wall_us * 1e6), wall_ms_total=wall_ms, quantize_us=quant_us)
    del qs, es
    torch.cuda.empty_cache()
    return res


def time_make_twin(n_layers=43, G=4, R=1024, D=4096, elo=115, ehi=123):
    """The twin encoder at the padded-TP3 layer shape: n_layers distinct bf16 weights [G, R, D],
    each exactly e4m3 x 2^e per 32x32 block (e = byte - 127 in [elo, ehi], built on the device
    from seeded codes by bsfp8_dequant), encoded once each by bsfp8_make_twin (a synchronous
    prepare call: it allocates and clears an 8-byte counter, runs the encoder and reads the
    verdict back). Reported: the GPU span between HIP events around each call on its stream, and
    the host wall time per call."""
    import torch
    import block_scaled_fp8_skinny_amd as B
    qs, es = make_copies(torch, B, G, R, D, elo, ehi, n_layers, seed=7500)
    ws = [B.bsfp8_dequant(qs[i], es[i]) for i in range(n_layers)]
    del qs, es
    for i in range(3):
        B.bsfp8_make_twin(ws[i])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_layers)]
    accepted = 0
    t0 = time.perf_counter()
    for i in range(n_layers):
        evs[2 * i].record(stream)
        t = B.bsfp8_make_twin(ws[i])
        evs[2 * i + 1].record(stream)
        accepted += int(t.accepted)
    torch.cuda.synchronize()
    wall_us = 1e6 * (time.perf_counter() - t0) / n_layers
    spans = sorted(1e3 * evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(n_layers))
    gpu_us = sum(spans) / n_layers
    nbytes = G * R * D * 2 + G * R * D + 2 * G * (R // 32) * (D // 32)   # read bf16, write codes, exps, ok
    del ws
    torch.cuda.empty_cache()
    return dict(workload="twin_tp3", path="make_twin", desc=f"make_twin of {n_layers} exact bf16 layers [{G},{R},{D}]",
                G=G, N=R, K=D, layers=n_layers, accepted=accepted, gpu_span_us_per_layer=gpu_us,
                gpu_span_us_median=spans[n_layers // 2], wall_us_per_layer=wall_us, bytes_per_layer=nbytes,
                algorithmic_gbs=nbytes / (gpu_us * 1e3), pct_hbm_peak=100 * nbytes / (gpu_us * 1e3) / HBM_PEAK_GBS)


def cpu_baseline(name, M, seconds):
    """The oracle as it stands, timed on this host on a bounded sample of the same workload:
    whole GEMM calls on weight copies of the real shape until `seconds` have passed."""
    import numpy as np
    import oracle
    import synthetic as S
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    G, N, K, _, (elo, ehi), out, _ = WORKLOADS[name]
    r = S.rng(9000 + M)
    x = S.bf16_normal(r, (M, G * K))
    calls, t_total = 0, 0.0
    while t_total < seconds:
        q = S.e4m3_codes(r, (G, N, K))
        e = S.exponent_bytes(r, (G, N // 32, K // 32), elo, ehi)
        t0 = time.perf_counter()
        oracle.gemm(x, G, N, K, q, e, out="f32" if out == "f32" else "bf16")
        t_total += time.perf_counter() - t0
        calls += 1
    copy_bytes = G * N * K + G * (N // 32) * (K // 32)
    gbs = copy_bytes * calls / t_total / 1e9
    return {"value": gbs, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "us_per_call": 1e6 * t_total / calls,
            "sample": f"{calls} oracle.gemm calls (float64) on distinct weight copies of the same "
                      f"shape (M={M}, G={G}, N={N}, K={K}), {t_total:.1f} s of CPU time, "
                      f"BLAS threads={threads}, os.cpu_count()={os.cpu_count()}"}


def gemm_source_sha256():
    """Hash of the sources the bf16 GEMM kernels are built from (gemm.hip and device.h)."""
    h = hashlib.sha256()
    for f in ("gemm.hip", "device.h"):
        with open(os.path.join(ROOT, "block_scaled_fp8_skinny_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_from_profile(name, M):
    """HBM bytes per launch from the committed rocprofv3 counter summary, when it was taken on
    the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}_m{M}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    sha = gemm_source_sha256()
    if rec.get("gemm_source_sha256") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(20):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 20}), flush=True)
        return
    M = args.m or WORKLOADS[args.workload][3]
    r = time_workload(args.workload, M, args.steps, args.warmup, args.split_k, path=args.path)
    G, N, K = r["G"], r["N"], r["K"]
    line = {
        "metric": METRIC,
        "value": round(r["weight_stream_gbs_wall"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["wall_us_per_call"] / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (round(r["weight_stream_gbs_wall"] / PAGES_GBS, 2)
                        if args.workload == "wo_a" and M == 6 and args.path == "bf16" else None),
        "dtype": "fp8" if args.path == "mx" else "bf16",
        "data": "synthetic",
        "config": {"workload": r["desc"] + f"; M={M}" + {"mx": "; fp8 x fp8 path (MXFP8 activations)",
                                                          "mxfp8": "; MXFP8 output epilogue"}.get(args.path, ""),
                   "path": args.path, "M": M, "G": G, "N": N, "K": K,
                   "weight_copies": r["copies"], "copy_bytes": r["copy_bytes"], "plan": r["plan"]},
        "us_per_call": round(r["wall_us_per_call"], 3),
        "quantize_us_per_call": round(r["quantize_us"], 3) if r["quantize_us"] is not None else None,
        "pct_hbm_peak": round(100 * r["weight_stream_gbs_wall"] / HBM_PEAK_GBS, 1),
        "eager_event_us_per_call_mean": round(r["kernel_us_mean"], 3),
        "eager_event_us_per_call_median": round(r["kernel_us_median"], 3),
        "roofline": {"bound": "hbm", "achieved": round(r["algorithmic_gbs"], 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(r["algorithmic_gbs"] / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profile(args.workload, M) if args.path == "bf16" else None,
                     "algorithmic_bytes_per_launch": r["algorithmic_bytes"]},
        "baseline_ref": "pages (GB10, other hardware): twin path 2.20 ms / 43 layers = 51.2 us/call at M=6",
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.workload, M, args.cpu_seconds)
    if args.all:
        rows = []
        for name, ms in (("shared_down", [6]), ("shared_down_pad", [6]), ("wo_a", [2, 4, 6, 8]),
                         ("wo_a_mid", [16, 32, 64, 128, 192]), ("wo_a_tp3", [2, 6, 8]),
                         ("lm_head", [16, 64, 128])):
            for m in ms:
                st = 400 if name == "lm_head" else 2000
                rr = time_workload(name, m, st, 50)
                rows.append(rr)
                print(json.dumps(rr), file=sys.stderr, flush=True)
        # the twin encoder at the padded-TP3 layer shape
        rr = time_make_twin()
        rows.append(rr)
        print(json.dumps(rr), file=sys.stderr, flush=True)
        # the row-scale twin (one exponent per row and 32 columns) at its page's shape
        for m in (1, 6, 16):
            rr = time_workload("main_proj", m, 2000, 50)
            rows.append(rr)
            print(json.dumps(rr), file=sys.stderr, flush=True)
        # the MXFP8 output epilogue (GEMM + fused sum-and-quantise kernel)
        for name, ms in (("wo_a", [2, 6, 8]), ("wo_a_mid", [16, 64, 192])):
            for m in ms:
                rr = time_workload(name, m, 2000, 50, path="mxfp8")
                rows.append(rr)
                print(json.dumps(rr), file=sys.stderr, flush=True)
        # the fp8 x fp8 path (MXFP8 activations) on the same weights
        for name, ms in (("wo_a", [6]), ("wo_a_mid", [16, 64, 128, 192]), ("lm_head", [16, 64, 128])):
            for m in ms:
                st = 400 if name == "lm_head" else 2000
                rr = time_workload(name, m, st, 50, path="mx")
                rows.append(rr)
                print(json.dumps(rr), file=sys.stderr, flush=True)
        with open(args.all, "w") as f:
            for rr in rows:
                f.write(json.dumps(rr) + "\n")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
