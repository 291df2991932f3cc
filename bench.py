"""Benchmark of the block-scaled fp8 small-M GEMM on one MI355X.

Headline (the `value` of the JSON line): the wo_a decode/verify shape at 6 rows, G=2 groups of
[1024 x 4096] e4m3 weights with 32x32 exponent blocks, bf16 activations [6, 8192], bf16 output
[6, 2, 1024], the built-in plan.

Protocol (page "recipes/docker-images/mia-tp4/adapter/shared_pad_k.py", MEASUREMENT: distinct
weight copies so that the cache is cold, captured graphs, interleaved rounds):
  * every configuration draws C distinct seeded weight copies whose codes and exponent bytes
    together hold at least 512 MiB (twice the 256 MiB Infinity Cache), whatever --steps says;
  * a step is one GEMM call on each of the C copies, in order (the pages' ms/step over their 43
    layers), captured once in a HIP graph;
  * activations are cold too: call i of a step reads activation copy i (the same values), as a
    layer reads the previous kernel's output rather than a buffer left in L2 by the call before;
  * rounds: every configuration's step graph, and the plain-read floor graphs, replayed in turn
    between HIP events on the replay stream (the headline: exactly --steps steps per round, each
    timed region bracketed by synchronisation); at least 5 rounds; each figure is the median over
    rounds;
  * the plain-read floor of each weight set: the same graph with the GEMM replaced by a kernel
    that only reads the copy's bytes with the GEMM's load shape (bsfp8_read_floor), and a bare
    launch (the same kernel reading nothing); and per configuration the read + write floor, the
    same reads followed by a write of that configuration's output bytes; for every unsplit row
    also the data-movement floor (floor_xrw): the same, with every floor
    workgroup also reading a slab of the bytes a workgroup of the plan reads beyond its share of
    the weights (its activation rows, K wide, and the weight rows other m-blocks read again),
    spread over the steps of its weight share.

Per call: us_per_call = step time / C (gaps between launches included, as a graph replays them).
value = weight-stream GB/s = (e4m3 bytes + exponent bytes) / us_per_call. roofline.achieved =
algorithmic bytes (weights + exponents + X + Y) / us_per_call, as a fraction of 8 TB/s.
Every configuration named by the workloads gets such an entry in "configs", with the floor, the
roofline fraction, the MFMA rate and the CPU oracle's time (all host threads and one thread);
so do the twin encoder (make_twin) and the standalone dequantisation (bsfp8_dequant) per
[4, 1024, 4096] layer.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--rounds R] [--no-cpu-baseline]
       [--headline-only] [--workload NAME --m M [--path P] [--split-k S]] [--extra FILE]
"""
import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "us/call and effective weight-stream GB/s (% of HBM peak), M=6 block-fp8 GEMM"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_FP8_PEAK_TFLOPS = 5000.0
COLD_BYTES = 512 << 20
FLOOR_WGS = 256
# The pages' own figure for the headline workload (other hardware, context): on GB10 the twin
# path ran 43 wo_a layers at 6 rows in 2.20 ms, i.e. 51.2 us/call, about 164 GB/s of weight stream.
PAGES_GBS = 8_396_800 / (2.20e-3 / 43) / 1e9

WORKLOADS = {
    # name: (G, N, K, default M, exponent byte range, out dtype, description)
    "wo_a": (2, 1024, 4096, 6, (115, 125), "bf16",
             "wo_a small-batch decode: X bf16 [M, 2*4096], W e4m3 [2,1024,4096] + u8 exponents [2,32,128]"),
    "wo_a_mid": (2, 1024, 4096, 64, (115, 125), "bf16",
                 "wo_a mid path: X bf16 [M, 2*4096], W e4m3 [2,1024,4096] + u8 exponents [2,32,128]"),
    "wo_a_tp3": (4, 1024, 4096, 6, (115, 123), "bf16",
                 "wo_a padded-TP3 shard: X bf16 [M, 4*4096], W e4m3 [4,1024,4096] + u8 exponents [4,32,128] "
                 "(the twins of 43 exact bf16 layers)"),
    "shared_down": (1, 5120, 576, 6, (117, 123), "bf16",
                    "shared-expert down_proj: X bf16 [M, 576], W e4m3 [5120, 576] + u8 exponents [160, 18]"),
    "shared_down_pad": (1, 5120, 640, 6, (117, 123), "bf16",
                        "shared-expert down_proj, K zero-padded 576->640 (zero codes, exponent byte 127)"),
    "lm_head": (1, 32768, 5120, 128, (118, 122), "f32",
                "draft LM head: X bf16 [M, 5120], W e4m3 [32768, 5120] + u8 exponents [1024, 160], fp32 logits"),
    "main_proj": (1, 1280, 5120, 16, (115, 125), "bf16",
                  "draft main_proj shard (row-scale twin): X bf16 [M, 5120], W e4m3 [1280, 5120] + u8 exponents "
                  "per row and 32 columns [1280, 160]"),
}
ROW_SCALE_WORKLOADS = {"main_proj"}
WEIGHT_SET = {"wo_a": "wo_a", "wo_a_mid": "wo_a", "wo_a_tp3": "wo_a_tp3", "shared_down": "shared_down",
              "shared_down_pad": "shared_down_pad", "lm_head": "lm_head", "main_proj": "main_proj"}

# The configurations of the workloads: (label, workload, M, split_k)
DEFAULT_CONFIGS = (
    [("d1", "shared_down", 6, 0), ("d1", "shared_down_pad", 6, 0)]
    + [("d2", "wo_a", m, 0) for m in (2, 4, 6, 8)]
    + [("d2 split", "wo_a", m, 8) for m in (2, 4, 6, 8)]
    + [("d3", "wo_a_mid", m, 0) for m in (16, 32, 64, 128, 192)]
    + [("d3 split", "wo_a_mid", 16, 4), ("d3 split", "wo_a_mid", 32, 2)]
    + [("d4", "wo_a_tp3", m, 0) for m in (2, 6, 8)]
    + [("d5", "lm_head", m, 0) for m in (16, 64, 128)]
)
HEADLINE = ("d2", "wo_a", 6, 0)
TWIN_LAYERS = 43


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20, help="steps of the headline per timed round")
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--rounds", type=int, default=7)
    p.add_argument("--reps", type=int, default=8, help="steps per timed round of the other configurations")
    p.add_argument("--headline-only", action="store_true")
    p.add_argument("--workload", default=None, choices=sorted(WORKLOADS))
    p.add_argument("--m", type=int, default=None)
    p.add_argument("--split-k", type=int, default=0)
    p.add_argument("--path", default="bf16", choices=["bf16", "mx", "mxfp8"],
                   help="bf16: the exact twin GEMM (default); mx: the fp8 x fp8 GEMM on MXFP8 activations; "
                        "mxfp8: the exact twin GEMM with the MXFP8 output epilogue")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=8.0, help="CPU time per leg of the headline's baseline")
    p.add_argument("--extra", default=None, help="also time the fp8 x fp8 path, the MXFP8 epilogue and the "
                                                 "row-scale twin; write their entries as JSON lines here")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB, 20 times (counter calibration)")
    return p.parse_args()


# ------------------------------------------------------------------------------------------------
# inputs
# ------------------------------------------------------------------------------------------------
def shape_of(name):
    G, N, K = WORKLOADS[name][:3]
    erows = N if name in ROW_SCALE_WORKLOADS else N // 32
    return G, N, K, erows


def copy_nbytes(name):
    G, N, K, erows = shape_of(name)
    return G * N * K + G * erows * (K // 32)


class WeightSet:
    """C distinct weight copies, each one device buffer [codes | exponent bytes] (so that the
    floor kernel reads exactly the bytes a GEMM call streams), with q and e views into it."""

    def __init__(self, torch, name, bufs):
        G, N, K, erows = shape_of(name)
        self.name, self.bufs = name, bufs
        nq = G * N * K
        self.q = [b[:nq].view(G, N, K) for b in bufs]
        self.e = [b[nq:nq + G * erows * (K // 32)].view(G, erows, K // 32) for b in bufs]
        self.copy_bytes = copy_nbytes(name)

    def __len__(self):
        return len(self.bufs)


def n_copies_for(name):
    return max(4, math.ceil(COLD_BYTES / copy_nbytes(name)))


def random_weight_set(torch, name, seed, n=None):
    """Seeded codes uniform over the finite e4m3 codes and exponent bytes uniform in the
    workload's range, drawn on the device."""
    import synthetic as S
    G, N, K, erows = shape_of(name)
    elo, ehi = WORKLOADS[name][4]
    n = n or n_copies_for(name)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    table = torch.from_numpy(S.FINITE_E4M3_CODES).cuda()
    nq = G * N * K
    bufs = []
    for _ in range(n):
        b = torch.empty(copy_nbytes(name), dtype=torch.uint8, device="cuda")
        idx = torch.randint(0, table.numel(), (nq,), generator=gen, device="cuda", dtype=torch.int32)
        b[:nq] = table[idx]
        b[nq:] = torch.randint(elo, ehi + 1, (G * erows * (K // 32),), generator=gen, device="cuda",
                               dtype=torch.int32).to(torch.uint8)
        bufs.append(b)
        del idx
    return WeightSet(torch, name, bufs)


def padded_weight_set(torch, B, src, name):
    """The copies of src zero-padded along K (zero codes, exponent byte 127) by the library."""
    G, N, K, erows = shape_of(name)
    nq = G * N * K
    bufs = []
    for q, e in zip(src.q, src.e):
        qp, ep = B.bsfp8_pad_k_weight(q, e, K)
        b = torch.empty(copy_nbytes(name), dtype=torch.uint8, device="cuda")
        b[:nq] = qp.reshape(-1)
        b[nq:] = ep.reshape(-1)
        bufs.append(b)
    return WeightSet(torch, name, bufs)


def twin_weight_set(torch, B, seed, n_layers=TWIN_LAYERS, reps=5):
    """The padded-TP3 twin workload: n_layers exact bf16 layers [4, 1024, 4096] (each 32x32 block
    e4m3 * 2^e, e - 127 in [115, 123] - 127, rebuilt from seeded codes by bsfp8_dequant), encoded by
    bsfp8_make_twin (each call timed, `reps` rounds), whose twins are the GEMM's weight copies, and by
    bsfp8_make_twin_async in one graph over all layers (`reps` timed replays: the encoder's rate)."""
    name = "wo_a_tp3"
    src = random_weight_set(torch, name, seed, n=n_layers)
    layers = [B.bsfp8_dequant(q, e) for q, e in zip(src.q, src.e)]
    G, N, K, erows = shape_of(name)
    nq = G * N * K
    for w in layers[:3]:
        B.bsfp8_make_twin(w)                        # warm-up
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    round_means, accepted, twins = [], 0, None
    for rd in range(reps):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_layers)]
        out = []
        for i, w in enumerate(layers):
            evs[2 * i].record(stream)
            t = B.bsfp8_make_twin(w)
            evs[2 * i + 1].record(stream)
            out.append(t)
        torch.cuda.synchronize()
        round_means.append(1e3 * sum(evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(n_layers)) / n_layers)
        if twins is None:
            twins = out
            accepted = sum(int(t.accepted) for t in out)
    bufs = []
    for t, q0, e0 in zip(twins, src.q, src.e):
        b = torch.empty(copy_nbytes(name), dtype=torch.uint8, device="cuda")
        b[:nq] = t.q.reshape(-1)
        b[nq:] = t.e.reshape(-1)
        bufs.append(b)
    same = all(torch.equal(t.q, q0) and torch.equal(t.e, e0) for t, q0, e0 in zip(twins, src.q, src.e))
    nbytes = G * N * K * 2 + G * N * K + 2 * G * (N // 32) * (K // 32)   # read bf16; write codes, exps, ok
    sync_us = statistics.median(round_means)
    # the encoder itself: bsfp8_make_twin_async (no allocation, no synchronisation) on every layer
    # in one graph, each into its own twin buffers and inexact-block counter, `reps` timed replays
    aq = [torch.empty_like(t.q) for t in twins]
    ae = [torch.empty_like(t.e) for t in twins]
    aok = [torch.empty_like(t.ok) for t in twins]
    cnt = torch.zeros(n_layers, dtype=torch.int64, device="cuda")
    ga = capture(torch, lambda i: B.bsfp8_make_twin_async(layers[i], cnt[i:i + 1], aq[i], ae[i], aok[i]), n_layers)
    ga.replay()
    torch.cuda.synchronize()
    async_same = (int(cnt.count_nonzero().item()) == n_layers - accepted and
                  all(torch.equal(a, t.q) and torch.equal(b, t.e) for a, b, t in zip(aq, ae, twins)))
    tw_rounds = []
    for rd in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        ga.replay()
        b.record(stream)
        torch.cuda.synchronize()
        tw_rounds.append(1e3 * a.elapsed_time(b) / n_layers)
    us = statistics.median(tw_rounds)
    del ga, aq, ae, aok
    # the standalone dequantisation (the twin back to bf16, into the layers' own buffers, so every
    # call reads and writes its own cold copy): one graph of n_layers calls, `reps` timed replays
    g = capture(torch, lambda i: B.bsfp8_dequant(twins[i].q, twins[i].e, out=layers[i]), n_layers)
    g.replay()
    torch.cuda.synchronize()
    dq_rounds = []
    for rd in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        dq_rounds.append(1e3 * a.elapsed_time(b) / n_layers)
    dq_bytes = G * N * K + G * (N // 32) * (K // 32) + G * N * K * 2     # read codes, exps; write bf16
    dq_us = statistics.median(dq_rounds)
    # its read + write floor: the floor kernel reading each twin copy and writing the layer's bytes
    sink = torch.empty(FLOOR_WGS, dtype=torch.int32, device="cuda")
    gf = capture(torch, lambda i: B.bsfp8_read_floor(bufs[i], nwg=FLOOR_WGS, sink=sink,
                                                     out=layers[i].view(torch.uint8).reshape(-1)), n_layers)
    gf.replay()
    torch.cuda.synchronize()
    fl_rounds = []
    for rd in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        gf.replay()
        b.record(stream)
        torch.cuda.synchronize()
        fl_rounds.append(1e3 * a.elapsed_time(b) / n_layers)
    fl_us = statistics.median(fl_rounds)
    dequant_entry = {
        "label": "f1 dequant", "workload": "wo_a_tp3", "path": "dequant",
        "desc": f"bsfp8_dequant of {n_layers} twins [{G},{N},{K}] to bf16, each into its own layer buffer "
                f"(one graph of {n_layers} calls)",
        "layers": n_layers, "us_per_layer": round(dq_us, 3),
        "us_per_layer_rounds": [round(v, 3) for v in dq_rounds], "bytes_per_layer": dq_bytes,
        "floor_rw_us_per_layer": round(fl_us, 3), "floor_rw_frac": round(fl_us / dq_us, 4),
        "roofline": {"bound": "hbm", "achieved": round(dq_bytes / (dq_us * 1e3), 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dq_bytes / (dq_us * 1e3) / HBM_PEAK_GBS, 4)},
    }
    del g, gf
    twin_entry = {
        "label": "d4 make_twin", "workload": "wo_a_tp3", "path": "make_twin",
        "desc": f"twin encoder on {n_layers} exact bf16 layers [{G},{N},{K}]: bsfp8_make_twin_async, one graph "
                f"of {n_layers} calls, each into its own buffers and counter; sync_call_us_per_layer = the "
                f"synchronous bsfp8_make_twin (counter allocated and cleared, encoder, verdict read back), "
                f"GPU span per call",
        "layers": n_layers, "accepted": accepted, "twins_equal_source": bool(same),
        "async_equals_sync": bool(async_same),
        "us_per_layer": us, "us_per_layer_rounds": [round(v, 3) for v in tw_rounds], "bytes_per_layer": nbytes,
        "sync_call_us_per_layer": round(sync_us, 3), "sync_call_us_per_layer_rounds": round_means,
        "algorithmic_gbs": nbytes / (us * 1e3),
        "roofline": {"bound": "hbm", "achieved": round(nbytes / (us * 1e3), 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(nbytes / (us * 1e3) / HBM_PEAK_GBS, 4)},
    }
    del layers, src
    return WeightSet(torch, name, bufs), [twin_entry, dequant_entry]


def activations(torch, M, G, K, seed):
    import synthetic as S
    return torch.from_numpy(S.bf16_normal(S.rng(seed), (M, G * K)).view("int16")).view(torch.bfloat16).cuda()


# ------------------------------------------------------------------------------------------------
# graphs and rounds
# ------------------------------------------------------------------------------------------------
def capture(torch, fn, n_calls):
    """One HIP graph of fn(0), fn(1), ..., fn(n_calls - 1), captured on a side stream."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for i in range(n_calls):
                fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return graph


def time_replays(torch, graph, reps):
    """Milliseconds for `reps` replays of graph, between HIP events on the replay stream, with the
    device synchronised before and after."""
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(s)
    for _ in range(reps):
        graph.replay()
    t1.record(s)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1)


class Timed:
    """A step graph (n_calls calls) and its per-round times."""

    def __init__(self, key, graph, n_calls, reps):
        self.key, self.graph, self.n_calls, self.reps = key, graph, n_calls, reps
        self.round_us = []              # per-call microseconds, one per round

    def run_round(self, torch):
        ms = time_replays(torch, self.graph, self.reps)
        self.round_us.append(1e3 * ms / (self.reps * self.n_calls))
        return ms

    @property
    def us(self):
        return statistics.median(self.round_us)

    @property
    def spread(self):
        return (max(self.round_us) - min(self.round_us)) / self.us if self.round_us else 0.0


# ------------------------------------------------------------------------------------------------
# configurations
# ------------------------------------------------------------------------------------------------
def algorithmic_bytes(name, M, path="bf16"):
    G, N, K, erows = shape_of(name)
    out_bytes = 4 if WORKLOADS[name][5] == "f32" else 2
    w, e = G * N * K, G * erows * (K // 32)
    x = M * G * K * 2
    y = M * G * N * out_bytes
    if path == "mx":
        x = M * G * K + M * G * K // 32
    if path == "mxfp8":
        y = M * G * N + M * G * N // 32
    return w, e, x, y


def make_call(torch, B, ws_set, name, M, split_k, path, xs, out):
    """The per-call function over the copies of ws_set (call i reads weight copy i and activation
    copy i of xs), its plan report and its buffers."""
    G, N, K, _ = shape_of(name)
    od = WORKLOADS[name][5]
    C, X = len(ws_set), len(xs)
    if path == "mx":
        xm = [B.bsfp8_quantize_mx(x) for x in xs]
        plan = {"mx_cfg": B.bsfp8_mx_plan(M, G, N), **B.bsfp8_mx_config_info(B.bsfp8_mx_plan(M, G, N))}
        return (lambda i: B.bsfp8_gemm_mx(xm[i % X][0], xm[i % X][1], ws_set.q[i % C], ws_set.e[i % C], out=out,
                                          out_dtype=od)), plan
    if name in ROW_SCALE_WORKLOADS:
        ws = B.workspace_row32(M, G, N, K, split_k)
        return (lambda i: B.bsfp8_gemm_row32(xs[i % X], ws_set.q[i % C], ws_set.e[i % C], split_k=split_k, ws=ws,
                                             out=out, out_dtype=od)), {"row_scale_twin": True}
    if path == "mxfp8":
        plan = B.bsfp8_plan_info(M, G, N, K, split_k, path=3)
        ws = B.workspace_mxfp8(M, G, N, K, split_k)
        yq = torch.empty((M, G * N), dtype=torch.uint8, device="cuda")
        ys = torch.empty((M, G * N // 32), dtype=torch.uint8, device="cuda")
        return (lambda i: B.bsfp8_gemm_mxfp8(xs[i % X], ws_set.q[i % C], ws_set.e[i % C], split_k=split_k, ws=ws,
                                             yq=yq, ys=ys)), plan
    plan = B.bsfp8_plan_info(M, G, N, K, split_k)
    ws = B.workspace(M, G, N, K, split_k)
    return (lambda i: B.bsfp8_gemm(xs[i % X], ws_set.q[i % C], ws_set.e[i % C], split_k=split_k, ws=ws, out=out,
                                   out_dtype=od)), plan


def entry_for(label, name, M, split_k, path, plan, t, ws_set, floor_t, launch_t, floor_rw_t=None, floor_xrw_t=None):
    G, N, K, erows = shape_of(name)
    w, e, x, y = algorithmic_bytes(name, M, path)
    us = t.us
    alg = w + e + x + y
    flops = 2 * M * G * N * K
    pages = G * N * K + G * N * K // 32
    peak = MFMA_FP8_PEAK_TFLOPS if path == "mx" else MFMA_BF16_PEAK_TFLOPS
    ent = {
        "label": label, "workload": name, "desc": WORKLOADS[name][6], "M": M, "G": G, "N": N, "K": K, "path": path,
        "split_k": split_k, "plan": plan, "copies": len(ws_set), "copy_bytes": ws_set.copy_bytes,
        "us_per_call": round(us, 3), "us_per_call_rounds": [round(v, 3) for v in t.round_us],
        "round_spread": round(t.spread, 4),
        "weight_stream_gbs": round((w + e) / (us * 1e3), 1),
        "pages_convention_gbs": round(pages / (us * 1e3), 1),
        "algorithmic_bytes": alg,
        "roofline": {"bound": "hbm", "achieved": round(alg / (us * 1e3), 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(alg / (us * 1e3) / HBM_PEAK_GBS, 4)},
        "tflops": round(flops / (us * 1e6), 2),
        "mfma_frac": round(flops / (us * 1e6) / peak, 4),
    }
    if floor_t is not None:
        ent["floor_us_per_call"] = round(floor_t.us, 3)
        ent["floor_frac"] = round(floor_t.us / us, 4)
        ent["launch_us_per_call"] = round(launch_t.us, 3)
    if floor_rw_t is not None:
        ent["floor_rw_us_per_call"] = round(floor_rw_t.us, 3)
        ent["floor_rw_frac"] = round(floor_rw_t.us / us, 4)
    if floor_xrw_t is not None:
        ent["floor_xrw_us_per_call"] = round(floor_xrw_t.us, 3)
        ent["floor_xrw_frac"] = round(floor_xrw_t.us / us, 4)
    return ent


# ------------------------------------------------------------------------------------------------
# the CPU oracle as a baseline
# ------------------------------------------------------------------------------------------------
def cpu_info():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "usable_cpus": usable}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return None


def _oracle_leg(fn, seconds, min_calls=1):
    calls, t_total = 0, 0.0
    while calls < min_calls or t_total < seconds:
        t0 = time.perf_counter()
        fn()
        t_total += time.perf_counter() - t0
        calls += 1
    return calls, t_total


def cpu_baseline(name, M, seconds, n_rows=None):
    """The oracle as it stands (oracle.gemm, float64 NumPy) timed on this host on a bounded sample
    of the workload: whole calls of the real shape (or, for the LM head, n_rows of its vocabulary
    rows per call, scaled to the full call), until `seconds` have passed, once with every BLAS
    thread and once with one. Returns the baseline in the headline's unit (GB/s of weight stream)
    and microseconds per call."""
    import numpy as np
    import oracle
    import synthetic as S
    try:
        from threadpoolctl import threadpool_limits
    except Exception:
        threadpool_limits = None
    G, N, K, erows = shape_of(name)
    elo, ehi = WORKLOADS[name][4]
    out = "f32" if WORKLOADS[name][5] == "f32" else "bf16"
    rows = n_rows or N
    r = S.rng(9000 + M)
    x = S.bf16_normal(r, (M, G * K))
    q = S.e4m3_codes(r, (G, rows, K))
    e = S.exponent_bytes(r, (G, rows // 32, K // 32), elo, ehi)
    fn = lambda: oracle.gemm(x, G, rows, K, q, e, out=out)
    scale = N / rows
    copy_bytes = copy_nbytes(name)
    res = {}
    for leg, limit in (("all_threads", None), ("one_thread", 1)):
        if limit is not None and threadpool_limits is None:
            continue
        if limit is None:
            calls, t = _oracle_leg(fn, seconds)
            threads = blas_threads()
        else:
            with threadpool_limits(limits=1):
                calls, t = _oracle_leg(fn, seconds)
            threads = 1
        us = 1e6 * t / calls * scale
        res[leg] = {"us_per_call": round(us, 1), "gbs": copy_bytes / (us * 1e3), "threads": threads, "calls": calls,
                    "cpu_seconds": round(t, 2)}
    a = res["all_threads"]
    sample = (f"{a['calls']} oracle.gemm calls (float64 NumPy) on one seeded weight of the shape "
              f"(M={M}, G={G}, N={rows}{f' of {N} rows, time scaled by {scale:g}' if rows != N else ''}, K={K}), "
              f"{a['cpu_seconds']} s with {a['threads']} BLAS threads")
    if "one_thread" in res:
        o = res["one_thread"]
        sample += f"; {o['calls']} calls, {o['cpu_seconds']} s with one thread"
    return {"value": a["gbs"], "unit": "GB/s", "cores": a["threads"], "kind": "oracle",
            "us_per_call": a["us_per_call"], "sample": sample,
            "one_thread": res.get("one_thread"), **cpu_info()}


def cpu_twin_baseline(seconds):
    """oracle.make_twin on one group [1, 1024, 4096] of the padded-TP3 layer, scaled to the layer."""
    import oracle
    import synthetic as S
    src = S.twin_source(7600, G=1, R=1024, D=4096)
    w = oracle.dequant_bf16(src["q"], src["e"])
    calls, t = _oracle_leg(lambda: oracle.make_twin(w), seconds)
    us = 1e6 * t / calls * 4
    return {"us_per_layer": round(us, 1), "kind": "oracle", "threads": 1,
            "sample": f"{calls} oracle.make_twin calls on one group [1,1024,4096] of a layer, {t:.2f} s, "
                      f"scaled by 4 to the [4,1024,4096] layer (NumPy elementwise work, one thread)"}


def cpu_dequant_baseline(seconds):
    """oracle.dequant_bf16 on one group [1, 1024, 4096] of the padded-TP3 layer, scaled to the layer."""
    import oracle
    import synthetic as S
    src = S.twin_source(7700, G=1, R=1024, D=4096)
    calls, t = _oracle_leg(lambda: oracle.dequant_bf16(src["q"], src["e"]), seconds)
    us = 1e6 * t / calls * 4
    return {"us_per_layer": round(us, 1), "kind": "oracle", "threads": 1,
            "sample": f"{calls} oracle.dequant_bf16 calls on one group [1,1024,4096] of a layer, {t:.2f} s, "
                      f"scaled by 4 to the [4,1024,4096] layer (NumPy elementwise work)"}


# ------------------------------------------------------------------------------------------------
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
    if rec.get("gemm_source_sha256") != gemm_source_sha256():
        return None
    return rec.get("hbm_bytes_per_launch")


def run(args):
    import torch
    import block_scaled_fp8_skinny_amd as B

    t_start = time.perf_counter()
    if args.workload:
        M = args.m or WORKLOADS[args.workload][3]
        configs = [("single", args.workload, M, args.split_k)]
        headline = configs[0]
        path = args.path
    elif args.headline_only:
        configs = [HEADLINE]
        headline = HEADLINE
        path = "bf16"
    else:
        configs = list(DEFAULT_CONFIGS)
        headline = HEADLINE
        path = "bf16"

    # weight sets
    sets, prep_entries = {}, None
    needed = {WEIGHT_SET[c[1]] for c in configs}
    seeds = {"wo_a": 7000, "shared_down": 7200, "lm_head": 7300, "main_proj": 7400}
    for ws_name in sorted(needed):
        if ws_name == "shared_down_pad":
            continue
        if ws_name == "wo_a_tp3":
            sets[ws_name], prep_entries = twin_weight_set(torch, B, 7500, reps=max(3, args.rounds))
        else:
            sets[ws_name] = random_weight_set(torch, ws_name, seeds[ws_name])
    if "shared_down_pad" in needed:
        if "shared_down" not in sets:
            sets["shared_down"] = random_weight_set(torch, "shared_down", seeds["shared_down"])
        sets["shared_down_pad"] = padded_weight_set(torch, B, sets["shared_down"], "shared_down_pad")
    torch.cuda.synchronize()

    # step graphs
    timed, meta = [], []
    keep = []                                       # buffers the graphs address (a graph does not keep
                                                    # them alive, and every capture empties the cache)
    for (label, name, M, split_k) in configs:
        G, N, K, _ = shape_of(name)
        ws_set = sets[WEIGHT_SET[name]]
        # one activation copy per weight copy: a layer's input is the previous kernel's output, not
        # a buffer left in L2 by the call before (with one shared copy, 96 KB of activations stayed
        # in L2 across calls or not depending on where the allocator put them: 4.09 or 4.22 us)
        C = len(ws_set)
        x0 = activations(torch, M, G, K, 7100 + M)
        xs = [x0] + [x0.clone() for _ in range(C - 1)]
        od = torch.float32 if WORKLOADS[name][5] == "f32" else torch.bfloat16
        out = torch.empty((M, G, N), dtype=od, device="cuda")
        fn, plan = make_call(torch, B, ws_set, name, M, split_k, path, xs, out)
        for i in range(C):                          # eager warm-up over every copy
            fn(i)
        torch.cuda.synchronize()
        g = capture(torch, fn, C)
        reps = args.steps if (label, name, M, split_k) == headline else args.reps
        timed.append(Timed((label, name, M, split_k), g, C, reps))
        meta.append((label, name, M, split_k, plan, ws_set))
        keep.append((xs, out, fn))                  # fn holds the workspace the graph writes
    # plain-read floors and a bare launch over each weight set's copies
    floors = {}
    sink = torch.empty(FLOOR_WGS, dtype=torch.int32, device="cuda")
    for ws_name in sorted({WEIGHT_SET[c[1]] for c in configs}):
        ws_set = sets[ws_name]
        C = len(ws_set)
        gf = capture(torch, lambda i, s=ws_set: B.bsfp8_read_floor(s.bufs[i], nwg=FLOOR_WGS, sink=sink), C)
        gl = capture(torch, lambda i, s=ws_set: B.bsfp8_read_floor(s.bufs[i], nbytes=0, nwg=FLOOR_WGS, sink=sink), C)
        floors[ws_name] = (Timed(("floor", ws_name), gf, C, args.reps), Timed(("launch", ws_name), gl, C, args.reps))
    # read + write floors: the same reads, then a configuration's output bytes written (a kernel
    # that stores pays for its writes and their completion at its end)
    rw_floors = {}
    for (label, name, M, split_k) in configs:
        ws_name = WEIGHT_SET[name]
        ob = (algorithmic_bytes(name, M, path)[3] + 15) // 16 * 16
        if (ws_name, ob) in rw_floors:
            continue
        ws_set = sets[ws_name]
        yb = torch.empty(ob, dtype=torch.uint8, device="cuda")
        keep.append(yb)
        g = capture(torch, lambda i, s=ws_set, yb=yb: B.bsfp8_read_floor(s.bufs[i], nwg=FLOOR_WGS, sink=sink, out=yb),
                    len(ws_set))
        rw_floors[(ws_name, ob)] = Timed(("floor_rw", ws_name, ob), g, len(ws_set), args.reps)
    # ... and, for every unsplit row, the data-movement floor: the same, with each
    # floor workgroup also reading a slab of the bytes a workgroup of the plan reads beyond its
    # share of the weights (the activation rows of its m-block, K wide, and the weight rows that
    # the plan's other m-blocks read again), spread over the 256 floor workgroups; those bytes are
    # cache-resident after their first reads in a call, as the activations and re-read weights
    # are, and every call reads its own slab copy, as every GEMM call its own activations. The
    # slab loads are spread over the steps of the weight share (each step's before its weight
    # loads, as the GEMMs issue each chunk's activations before its weights): with one step (every
    # shape below the LM head) that is the slab first, and on the LM head's 640 KB shares it was
    # 0.6-1.2 us faster than the slab first
    def slab_of(name, M, plan):
        G, N, K, _ = shape_of(name)
        rows = min(plan["BM"], M) if plan["mblocks"] == 1 else plan["BM"]
        per = (rows * K * 2 * plan["workgroups"] + (plan["mblocks"] - 1) * G * N * K) // FLOOR_WGS
        return (per + 15) // 16 * 16, G * plan["mblocks"]
    xrw_floors, xkeys = {}, []
    for (label, name, M, split_k, plan, ws_set) in meta:
        xkeys.append(None)
        if split_k or path != "bf16" or name in ROW_SCALE_WORKLOADS or "BM" not in plan:
            continue
        ob = (algorithmic_bytes(name, M, path)[3] + 15) // 16 * 16
        sb, groups = slab_of(name, M, plan)
        key = (WEIGHT_SET[name], ob, sb, groups)
        xkeys[-1] = key
        if key in xrw_floors:
            continue
        yb = torch.empty(ob, dtype=torch.uint8, device="cuda")
        slabs = [torch.zeros(groups * sb, dtype=torch.uint8, device="cuda") for _ in range(len(ws_set))]
        keep.extend([yb, slabs])
        g = capture(torch, lambda i, s=ws_set, yb=yb, sl=slabs, gr=groups: B.bsfp8_read_floor(
            s.bufs[i], nwg=FLOOR_WGS, sink=sink, out=yb, slab=sl[i], slab_groups=gr, interleave=True), len(ws_set))
        xrw_floors[key] = Timed(("floor_xrw",) + key, g, len(ws_set), args.reps)
    every = (timed + [t for pair in floors.values() for t in pair] + list(rw_floors.values()) +
             list(xrw_floors.values()))

    # warm-up replays, then interleaved rounds
    for t in every:
        for _ in range(args.warmup if t.key == headline else 1):
            t.graph.replay()
    torch.cuda.synchronize()
    for rd in range(args.rounds):
        for t in every:
            t.run_round(torch)
        print(f"round {rd + 1}/{args.rounds} done", file=sys.stderr, flush=True)
    gpu_s = time.perf_counter() - t_start

    entries = []
    for t, (label, name, M, split_k, plan, ws_set), xkey in zip(timed, meta, xkeys):
        ft, lt = floors[WEIGHT_SET[name]]
        ob = (algorithmic_bytes(name, M, path)[3] + 15) // 16 * 16
        rwt = rw_floors[(WEIGHT_SET[name], ob)]
        xrwt = xrw_floors.get(xkey) if xkey else None
        entries.append(entry_for(label, name, M, split_k, path, plan, t, ws_set, ft, lt, rwt, xrwt))
    floor_summary = {k: {"copy_bytes": sets[k].copy_bytes, "copies": len(sets[k]),
                         "read_us_per_call": round(f.us, 3), "read_gbs": round(sets[k].copy_bytes / (f.us * 1e3), 1),
                         "launch_us_per_call": round(l.us, 3), "workgroups": FLOOR_WGS}
                     for k, (f, l) in floors.items()}

    # CPU baselines (the oracle; rank 0 at N=1)
    hl_index = configs.index(headline)
    if not args.no_cpu_baseline:
        for ent, (label, name, M, split_k, plan, ws_set) in zip(entries, meta):
            if name in ROW_SCALE_WORKLOADS or path != "bf16":
                continue
            is_head = (label, name, M, split_k) == headline
            secs = args.cpu_seconds if is_head else 0.5
            rows = 2048 if name == "lm_head" else None
            if split_k and not is_head:             # same oracle call as the built-in plan's entry
                continue
            ent["cpu_baseline"] = cpu_baseline(name, M, secs, n_rows=rows)
        if prep_entries is not None:
            prep_entries[0]["cpu_baseline"] = cpu_twin_baseline(2.0)
            prep_entries[1]["cpu_baseline"] = cpu_dequant_baseline(1.0)

    head = entries[hl_index]
    name, M = headline[1], headline[2]
    G, N, K, _ = shape_of(name)
    line = {
        "metric": METRIC,
        "value": head["weight_stream_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": timed[hl_index].us * timed[hl_index].n_calls / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (round(head["weight_stream_gbs"] / PAGES_GBS, 2)
                        if (name, M, path) == ("wo_a", 6, "bf16") else None),
        "dtype": "fp8" if path == "mx" else "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOADS[name][6] + f"; M={M}", "path": path, "M": M, "G": G, "N": N, "K": K,
                   "split_k": headline[3], "plan": head["plan"], "weight_copies": head["copies"],
                   "copy_bytes": head["copy_bytes"], "calls_per_step": head["copies"],
                   "rounds": args.rounds, "statistic": "median over interleaved rounds"},
        "us_per_call": head["us_per_call"],
        "us_per_call_rounds": head["us_per_call_rounds"],
        "pct_hbm_peak": round(100 * head["weight_stream_gbs"] / HBM_PEAK_GBS, 1),
        "floor_us_per_call": head.get("floor_us_per_call"),
        "floor_frac": head.get("floor_frac"),
        "floor_rw_us_per_call": head.get("floor_rw_us_per_call"),
        "floor_rw_frac": head.get("floor_rw_frac"),
        "floor_xrw_us_per_call": head.get("floor_xrw_us_per_call"),
        "floor_xrw_frac": head.get("floor_xrw_frac"),
        "roofline": dict(head["roofline"], traffic=traffic_from_profile(name, M) if path == "bf16" else None,
                         algorithmic_bytes_per_launch=head["algorithmic_bytes"]),
        "baseline_ref": "pages (GB10, other hardware): twin path 2.20 ms / 43 layers = 51.2 us/call at M=6",
    }
    if "cpu_baseline" in head:
        line["cpu_baseline"] = head["cpu_baseline"]
    if len(entries) > 1 or prep_entries is not None:
        line["configs"] = entries + (prep_entries or [])
        line["floors"] = floor_summary
    line["timing"] = {"gpu_setup_and_rounds_s": round(gpu_s, 1), "total_s": round(time.perf_counter() - t_start, 1)}
    return line


def run_extra(args, path_out):
    """The next-step paths on the same protocol: fp8 x fp8 (MXFP8 activations), the MXFP8 output
    epilogue, the row-scale twin. One JSON line per entry."""
    rows = []
    for path, cases in (("mx", [("wo_a", 6), ("wo_a_mid", 64), ("wo_a_mid", 192), ("lm_head", 16), ("lm_head", 128)]),
                        ("mxfp8", [("wo_a", 6), ("wo_a_mid", 64), ("wo_a_mid", 192)]),
                        ("bf16", [("main_proj", 1), ("main_proj", 6), ("main_proj", 16)])):
        for name, M in cases:
            a = argparse.Namespace(**vars(args))
            a.workload, a.m, a.path, a.split_k, a.no_cpu_baseline = name, M, path, 0, True
            ln = run(a)
            rows.append({"path": path, "workload": name, "M": M, "us_per_call": ln["us_per_call"],
                         "weight_stream_gbs": ln["value"], "roofline": ln["roofline"],
                         "floor_frac": ln["floor_frac"], "plan": ln["config"]["plan"]})
            print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
    with open(path_out, "w") as f:
        for r in rows:
            f.write(json.dumps(r) + "\n")


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
    line = run(args)
    if args.extra:
        run_extra(args, args.extra)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
