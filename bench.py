"""Benchmark of the LLM.int8() mixed-precision matmul on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only prefill|decode]
                    [--no-cpu-baseline] [--sweep]

A step is one full int8_mixed_matmul call (outlier detection, isolation,
row-wise quantization, int8 MFMA matmul, dequantization and the 16-bit
outlier matmul) on a weight converted to Int8 beforehand (the conversion runs
once at load time and is timed separately).  Inputs are seeded synthetic
tensors already resident in HBM.

Headline (`value`): int8-mixed matmul TOPS = 2*T*K*N / t_step on the
prefill 175B-class FFN up-projection, X fp16 [2048,12288] with 7 planted
outlier dimensions, W fp16 [12288,49152], tau = 6.  Also reported: weight
GB/s = (K*N + 4*N) / t_step on the decode FFN up-projection X [8,8192],
W [8192,28672], with 8 rotating weight copies so that no call finds its
weight in the 256 MB last-level cache.

Per-kernel durations come from HIP events recorded on the stream the
library launches on, inside the timed loop; the roofline objects divide
the algorithmic work of one launch by that duration.  The CPU baseline is
the test oracle (plain C, on the host's cores) timed on a row sample of
the prefill workload.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, published
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, published
DECODE_ROTATE = 8
# decode graphs hold this many passes over the rotating weight copies (32
# calls per replay), as one decode step of a model holds many matmuls in one
# graph; with one pass (8 calls) the replay launch added ~4 us per call
DECODE_PASSES = 4
CALLS_PER_REPLAY = DECODE_ROTATE * DECODE_PASSES
CPU_THREADS = 16             # host-core share of one GPU on an 8-GPU host
CPU_TARGET_S = 15.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--only", choices=["prefill", "decode", "down"], default=None,
                   help="one workload only (down: the down-projection context timing, for "
                        "profiling runs)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-variants", action="store_true",
                   help="skip the memory-halved and bf16 variants and the down-projection "
                        "context timing (profiling runs that should see only the headline "
                        "kernels)")
    p.add_argument("--sweep", action="store_true",
                   help="instead of the headline run: the four projections of a 175B-class "
                        "block at T=4096 with 0, 8, 64 and 256 planted outlier dimensions "
                        "(time against the outlier count); prints one JSON line")
    p.add_argument("--no-sweep", action="store_true",
                   help="skip the outlier-count sweep of the 175B-class block projections that "
                        "the default run reports under other_configs")
    p.add_argument("--no-ceilings", action="store_true",
                   help="skip the measured-ceiling kernels (bare int8 MFMA loop, HBM stream read)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 1 GiB device-to-device copy (a kernel of known "
                        "traffic, for scaling the HBM byte counters)")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def src_digest(names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "int8_mixed_precision_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(profile_name: str, digest: str, key: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary
    (profiles/*.md, 'key: value' lines), if it was taken on the kernel
    source as it is now (else None)."""
    path = os.path.join(ROOT, "profiles", profile_name)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.strip().startswith("- "):
                k, v = line.strip()[2:].split(":", 1)
                vals[k.strip().strip("`")] = v.strip().strip("`")
    if vals.get("kernel_src_sha") != digest or key not in vals:
        return None
    return float(vals[key])


PREWARM_S = 0.3


def prewarm(torch, body, seconds=PREWARM_S):
    """Untimed calls for `seconds` of wall time before the warmup steps: the
    GPU's clocks ramp up over tens of milliseconds after idle time (host-side
    input generation), and a few warmup steps alone leave the first timed
    loop of a run measurably slower than later ones."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for i in range(4):
            body(i, None)
        torch.cuda.synchronize()


def timed_loop(torch, steps, warmup, body, nev=3):
    """Runs body(i, evs) warmup + steps times; returns the wall time of the
    timed steps (synchronized on both sides) and the event lists (nev events
    per step)."""
    for i in range(warmup):
        body(i, None)
    torch.cuda.synchronize()
    evs = []
    t0 = time.perf_counter()
    for i in range(steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(nev)] if nev else None
        body(i, e)
        evs.append(e)
    torch.cuda.synchronize()
    return time.perf_counter() - t0, evs


def prefill_variants(torch, mm, w, X, W16, Wq, sw, ws, Y, steps, warmup):
    """The memory-halved and bf16 variants of the prefill step and the
    fp32/bf16 checkpoint conversion, on the same inputs."""
    T, K, N = w.T, w.K, w.N
    ops = 2.0 * T * K * N
    # The memory-halved variant (no 16-bit weight: outlier rows recovered
    # from the Int8 weight) and the bf16 variant (the same values rounded to
    # bf16, weight converted from the bf16 checkpoint) are timed alternated
    # call by call with the fp16 call, so all three see the same clocks
    # (timed one after another, later loops ran at lower clocks).
    Xb, Wb = X.to(torch.bfloat16), W16.to(torch.bfloat16)
    Wqb, swb, _ = mm.quantize_checkpoint(Wb)
    Yb = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")

    def call_f16():
        mm.mixed_matmul(X, Wq, sw, W16, w.tau, workspace=ws, out=Y)

    def call_halved():
        mm.quantize_activations(X, N, w.tau, ws)
        mm.matmul_prepared(ws, T, K, Wq, sw, None, out=Y)

    def call_bf16():
        mm.mixed_matmul(Xb, Wqb, swb, Wb, w.tau, workspace=ws, out=Yb)

    calls = (("f16", call_f16), ("halved", call_halved), ("bf16", call_bf16))
    log(f"prefill variants (fp16, memory-halved, bf16 alternated): {warmup} warmup + {steps} "
        "timed rounds")
    for _ in range(max(1, warmup)):
        for _, c in calls:
            c()
    prewarm(torch, lambda i, e: [c() for _, c in calls])
    evs = {name: [] for name, _ in calls}
    for _ in range(steps):
        for name, c in calls:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            c()
            b.record()
            evs[name].append((a, b))
    torch.cuda.synchronize()
    call_ms = {name: float(np.mean([a.elapsed_time(b) for a, b in v])) for name, v in evs.items()}
    # weight conversion from fp32 and bf16 checkpoints
    conv = {}
    W32 = W16.float()
    for tag, Wc in (("bf16", Wb), ("f32", W32)):
        mm.quantize_checkpoint(Wc)
        torch.cuda.synchronize()
        ca, cb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ca.record()
        for _ in range(3):
            mm.quantize_checkpoint(Wc)
        cb.record()
        torch.cuda.synchronize()
        ms = ca.elapsed_time(cb) / 3
        conv[tag] = {"ms": round(ms, 4),
                     "GB/s": round((Wc.element_size() * K * N + K * N + 4.0 * N) /
                                   (ms * 1e-3) / 1e9, 1)}
    del W32, Xb, Wb, Wqb, swb, Yb
    return {"halved_tops": ops / (call_ms["halved"] * 1e-3) / 1e12,
            "halved_ms_per_step": call_ms["halved"],
            "bf16_tops": ops / (call_ms["bf16"] * 1e-3) / 1e12, "bf16_ms_per_step": call_ms["bf16"],
            "alternated_f16_ms": call_ms["f16"], "convert": conv}


def bench_prefill(torch, mm, synth, steps, warmup, variants=True):
    w = synth.WORKLOADS["up"]
    T, K, N = w.T, w.K, w.N
    log(f"prefill: generating X [{T},{K}], W [{K},{N}]")
    X = torch.from_numpy(synth.make_x(w, threads=CPU_THREADS)).cuda()
    Wh = synth.make_w(w, threads=CPU_THREADS)
    W16 = torch.from_numpy(Wh).cuda()
    del Wh
    Wq = torch.empty(mm.weight_bytes(K, N), dtype=torch.int8, device="cuda")
    sw = torch.empty(N, dtype=torch.float32, device="cuda")
    # weight conversion (once per weight), timed on its own
    for _ in range(2):
        mm.quantize_weight(W16, out=(Wq, sw))
    torch.cuda.synchronize()
    qa, qb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    qa.record()
    for _ in range(5):
        mm.quantize_weight(W16, out=(Wq, sw))
    qb.record()
    torch.cuda.synchronize()
    q_ms = qa.elapsed_time(qb) / 5

    ws = mm.new_workspace(T, K, N)
    Y = torch.empty((T, N), dtype=torch.float16, device="cuda")

    def step(i, e):
        # int8_mixed_matmul == quantize_activations + matmul_prepared (same
        # kernels, same stream); the split lets two events bracket the
        # matmul.  No event goes before the activation pass: an event
        # recorded right after the previous step's matmul cost ~7.7 us per
        # step on the GPU (0.918 against 0.911 ms per step, one box,
        # alternated; 0.907 ms with no events at all), time the call itself
        # does not take.
        mm.quantize_activations(X, N, w.tau, ws)
        if e is not None:
            e[0].record()
        mm.matmul_prepared(ws, T, K, Wq, sw, W16, out=Y)
        if e is not None:
            e[1].record()

    log(f"prefill: {PREWARM_S} s prewarm, {warmup} warmup + {steps} timed steps")
    prewarm(torch, step)
    wall, evs = timed_loop(torch, steps, warmup, step, nev=2)
    # activation pass: from the previous step's matmul end to this step's
    # matmul start (the two kernels and the launch gaps around them)
    act_ms = (float(np.mean([evs[i - 1][1].elapsed_time(evs[i][0]) for i in range(1, len(evs))]))
              if len(evs) > 1 else None)
    gemm_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    extra = prefill_variants(torch, mm, w, X, W16, Wq, sw, ws, Y, steps, warmup) if variants else {}
    # the outlier count of this X (one debug call, outside the timed loop)
    dbg = mm.mixed_matmul_debug(X, Wq, sw, W16, w.tau)
    o = int(dbg["count"][0])
    if variants:
        ours = lambda: mm.matmul_prepared(ws, T, K, Wq, sw, W16, out=Y)
        # the converted weight as a plain [N,K] matrix (panels of 256 rows,
        # k-tiles of 64 columns; both divide this workload's N and K)
        wq_rows = Wq.view(N // 256, K // 64, 256, 64).permute(0, 2, 1, 3).reshape(N, K)
        extra["vendor_int8_gemm"] = vendor_int8_gemm(torch, dbg["xq"], wq_rows, steps, warmup,
                                                     ours)
        del wq_rows
    del dbg
    ops = 2.0 * T * K * N
    ms_step = wall * 1e3 / steps
    return {
        "T": T, "K": K, "N": N, "tau": w.tau, "o": o, "ms_per_step": ms_step,
        "tops": ops * steps / wall / 1e12,
        "activation_ms": act_ms, "gemm_ms": gemm_ms,
        "gemm_tops": ops / (gemm_ms * 1e-3) / 1e12,
        "quantize_weight_ms": q_ms,
        "quantize_weight_gbs": (2.0 * K * N + K * N + 4.0 * N) / (q_ms * 1e-3) / 1e9,
        **extra,
    }


def vendor_int8_gemm(torch, xq, wq, steps, warmup, ours):
    """Context for the roofline: the vendor library's int8 GEMM (hipBLASLt
    through torch._int_mm) on the same Xq [T,K] and Wq [N,K], int32 out - the
    int8 product alone, without dequantization, outlier product or fp16 Y -
    alternated step by step with this library's whole matmul (`ours`, the
    prepared entry point) so that both see the same clocks."""
    T, K = xq.shape
    N = wq.shape[0]
    b = wq.t()

    def step(i, e):
        if e is not None:
            e[0].record()
        torch._int_mm(xq, b)
        if e is not None:
            e[1].record()
        ours()
        if e is not None:
            e[2].record()

    try:
        prewarm(torch, step)
        _, evs = timed_loop(torch, steps, warmup, step)
    except RuntimeError as err:   # no int8 GEMM in this torch build
        return {"note": f"unavailable: {str(err)[:80]}"}
    ms = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    ours_ms = float(np.median([e[1].elapsed_time(e[2]) for e in evs]))
    return {"note": "torch._int_mm (hipBLASLt) on the same int8 operands, int32 out; alternated "
                    "with this library's whole matmul (dequantization, outlier product, fp16 Y)",
            "ms": round(ms, 4), "TOPS": round(2.0 * T * K * N / (ms * 1e-3) / 1e12, 1),
            "ours_ms": round(ours_ms, 4)}


def bench_down(torch, mm, synth, steps, warmup):
    """The prefill FFN down-projection workload (T=2048, K=49152, N=12288,
    Laplace activations with planted and natural outliers): whole
    int8_mixed_matmul calls on a pre-converted weight.  Context next to the
    headline; 384 output tiles make 1.5 rounds on 256 CUs, which the matmul
    runs as 768 half-K units."""
    w = synth.WORKLOADS["down"]
    T, K, N = w.T, w.K, w.N
    log(f"down: generating X [{T},{K}], W [{K},{N}]")
    X = torch.from_numpy(synth.make_x(w, threads=CPU_THREADS)).cuda()
    W16 = torch.from_numpy(synth.make_w(w, threads=CPU_THREADS)).cuda()
    Wq, sw = mm.quantize_weight(W16)
    ws = mm.new_workspace(T, K, N)
    Y = torch.empty((T, N), dtype=torch.float16, device="cuda")

    def step(i, e):
        mm.mixed_matmul(X, Wq, sw, W16, w.tau, workspace=ws, out=Y)

    log(f"down: {PREWARM_S} s prewarm, {warmup} warmup + {steps} timed steps")
    prewarm(torch, step)
    # wall time only: no events between the calls (an event recorded after
    # a matmul costs the GPU several microseconds)
    wall, _ = timed_loop(torch, steps, warmup, step, nev=0)
    dbg = mm.mixed_matmul_debug(X, Wq, sw, W16, w.tau)
    o = int(dbg["count"][0])
    del dbg, X, W16, Wq, sw, ws, Y
    torch.cuda.empty_cache()
    return {"T": T, "K": K, "N": N, "tau": w.tau, "outlier_dims": o,
            "ms_per_call": round(wall * 1e3 / steps, 4),
            "TOPS": round(2.0 * T * K * N * steps / wall / 1e12, 2)}


def decode_batched(torch, mm, synth, w, sets, rounds, warmup, rows=(32, 128)):
    """Batched decode on the decode workload's weights: T = 32 and 128 rows of
    activations with the same recipe, whole calls from a HIP graph over the
    rotating weight copies (the streaming matmul kernels).  Context only."""
    out = []
    K, N = w.K, w.N
    for T in rows:
        X = torch.from_numpy(synth.make_x(w, T=T, threads=CPU_THREADS)).cuda()
        ws = mm.new_workspace(T, K, N)
        Y = torch.empty((T, N), dtype=torch.float16, device="cuda")

        def one_round():
            for Wq, sw, W16 in sets:
                mm.mixed_matmul(X, Wq, sw, W16, w.tau, workspace=ws, out=Y)

        one_round()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(DECODE_PASSES):
                one_round()
        torch.cuda.synchronize()

        def step(i, e):
            if e is not None:
                e[0].record()
            graph.replay()
            if e is not None:
                e[1].record()

        prewarm(torch, step)
        wall, _ = timed_loop(torch, rounds, max(1, warmup // CALLS_PER_REPLAY + 1), step)
        calls = rounds * CALLS_PER_REPLAY
        out.append({"T": T, "us_per_call": round(wall * 1e6 / calls, 2),
                    "weight_GB/s": round(K * N * calls / wall / 1e9, 1),
                    "TOPS": round(2.0 * T * K * N * calls / wall / 1e12, 1)})
        del graph, X, ws, Y
        torch.cuda.empty_cache()
    return out


def decode_variants(torch, mm, w, X, sets, ws, Y, rounds, warmup):
    """The memory-halved and bf16 variants of the decode call (graph replays
    over the same rotating weight copies)."""
    T, K, N = w.T, w.K, w.N
    steps = rounds * CALLS_PER_REPLAY
    wbytes = K * N + 4.0 * N
    # the memory-halved variant: no 16-bit weight passed at all
    def one_round_halved():
        for Wq, sw, _ in sets:
            mm.mixed_matmul(X, Wq, sw, None, w.tau, workspace=ws, out=Y)

    one_round_halved()
    torch.cuda.synchronize()
    graph_h = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph_h):
        for _ in range(DECODE_PASSES):
            one_round_halved()
    torch.cuda.synchronize()

    def step_halved(i, e):
        if e is not None:
            e[0].record()
        graph_h.replay()
        if e is not None:
            e[1].record()
            e[2].record()

    log(f"decode, memory-halved: {rounds} timed graph replays")
    wall_h, evs_h = timed_loop(torch, rounds, max(1, warmup // CALLS_PER_REPLAY + 1), step_halved)
    call_h_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs_h])) / CALLS_PER_REPLAY

    # the bf16 variant: bf16 X and W16 (the same values rounded), weight
    # copies converted from the bf16 checkpoint
    Xb = X.to(torch.bfloat16)
    sets_b = []
    for _, _, W16 in sets:
        Wb = W16.to(torch.bfloat16)
        Wqb, swb, _ = mm.quantize_checkpoint(Wb)
        sets_b.append((Wqb, swb, Wb))
    Yb = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")

    def one_round_bf16():
        for Wq, sw, Wb in sets_b:
            mm.mixed_matmul(Xb, Wq, sw, Wb, w.tau, workspace=ws, out=Yb)

    one_round_bf16()
    torch.cuda.synchronize()
    graph_b = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph_b):
        for _ in range(DECODE_PASSES):
            one_round_bf16()
    torch.cuda.synchronize()

    def step_bf16(i, e):
        if e is not None:
            e[0].record()
        graph_b.replay()
        if e is not None:
            e[1].record()
            e[2].record()

    log(f"decode, bf16 variant: {rounds} timed graph replays")
    wall_b, evs_b = timed_loop(torch, rounds, max(1, warmup // CALLS_PER_REPLAY + 1), step_bf16)
    call_b_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs_b])) / CALLS_PER_REPLAY
    del sets_b, graph_b
    # warm: the same weight copy in every call (235 MB, which the 256 MB
    # last-level cache can hold) - context next to the cold metric
    Wq0, sw0, W160 = sets[0]

    def one_round_warm():
        for _ in range(DECODE_ROTATE):
            mm.mixed_matmul(X, Wq0, sw0, W160, w.tau, workspace=ws, out=Y)

    one_round_warm()
    torch.cuda.synchronize()
    graph_w = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph_w):
        for _ in range(DECODE_PASSES):
            one_round_warm()
    torch.cuda.synchronize()

    def step_warm(i, e):
        if e is not None:
            e[0].record()
        graph_w.replay()
        if e is not None:
            e[1].record()

    log(f"decode, warm weight: {rounds} timed graph replays")
    prewarm(torch, step_warm)
    wall_w, _ = timed_loop(torch, rounds, max(1, warmup // CALLS_PER_REPLAY + 1), step_warm)
    del graph_w
    return {"halved_weight_gbs": wbytes * steps / wall_h / 1e9, "halved_call_ms": call_h_ms,
            "bf16_weight_gbs": wbytes * steps / wall_b / 1e9, "bf16_call_ms": call_b_ms,
            "warm_weight_gbs": wbytes * steps / wall_w / 1e9, "warm_call_ms": wall_w * 1e3 / steps}


def bench_decode(torch, mm, synth, steps, warmup, variants=True):
    w = synth.WORKLOADS["dec"]
    T, K, N = w.T, w.K, w.N
    log(f"decode: generating X [{T},{K}], W [{K},{N}], {DECODE_ROTATE} weight copies")
    X = torch.from_numpy(synth.make_x(w, threads=CPU_THREADS)).cuda()
    W16_0 = torch.from_numpy(synth.make_w(w, threads=CPU_THREADS)).cuda()
    Wq0, sw0 = mm.quantize_weight(W16_0)
    sets = [(Wq0, sw0, W16_0)]
    for _ in range(DECODE_ROTATE - 1):
        sets.append((Wq0.clone(), sw0.clone(), W16_0.clone()))
    ws = mm.new_workspace(T, K, N)
    Y = torch.empty((T, N), dtype=torch.float16, device="cuda")

    # A decode call is tens of microseconds of GPU work, less than the Python
    # binding takes to issue it, so the steps are launched from a HIP graph
    # (one replay = DECODE_PASSES passes over the DECODE_ROTATE weight
    # copies), as a serving loop would.  The graph holds only the library's
    # own kernel launches.
    def one_round():
        for Wq, sw, W16 in sets:
            mm.mixed_matmul(X, Wq, sw, W16, w.tau, workspace=ws, out=Y)

    one_round()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(DECODE_PASSES):
            one_round()
    torch.cuda.synchronize()
    rounds = max(2, (steps + CALLS_PER_REPLAY - 1) // CALLS_PER_REPLAY)
    steps = rounds * CALLS_PER_REPLAY

    def step(i, e):
        if e is not None:
            e[0].record()
        graph.replay()
        if e is not None:
            e[1].record()

    log(f"decode: {PREWARM_S} s prewarm, {warmup} warmup + {rounds} timed graph replays of "
        f"{CALLS_PER_REPLAY} calls")
    prewarm(torch, step)
    wall, evs = timed_loop(torch, rounds, max(1, warmup // CALLS_PER_REPLAY + 1), step, nev=2)
    call_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) / CALLS_PER_REPLAY

    extra = decode_variants(torch, mm, w, X, sets, ws, Y, rounds, warmup) if variants else {}
    if variants:
        log("decode: batched rows (32, 128)")
        extra["batched"] = decode_batched(torch, mm, synth, w, sets, rounds, warmup)
    dbg = mm.mixed_matmul_debug(X, Wq0, sw0, W16_0, w.tau)
    o = int(dbg["count"][0])
    wbytes = K * N + 4.0 * N
    alg_bytes = 2.0 * T * K + K * N + 4.0 * N + 2.0 * o * N + 2.0 * T * N
    return {
        "T": T, "K": K, "N": N, "tau": w.tau, "o": o, "ms_per_step": wall * 1e3 / steps,
        "steps": steps, "weight_gbs": wbytes * steps / wall / 1e9, "call_ms": call_ms,
        "alg_bytes": alg_bytes, "alg_gbs": alg_bytes / (call_ms * 1e-3) / 1e9,
        **extra,
    }


def bench_sweep(torch, mm, synth, steps, warmup, prewarm_s):
    """Every sweep workload: the full call (activation pass + matmul, both
    timed by events on the library's stream), with and without the 16-bit
    weight.  Inputs are generated per workload and freed after it."""
    rows = []
    for name, w in synth.WORKLOADS.items():
        if not name.startswith("sweep_"):
            continue
        T, K, N = w.T, w.K, w.N
        log(f"sweep {name}: T={T} K={K} N={N}, {w.n_dims} planted dims")
        X = torch.from_numpy(synth.make_x(w, threads=CPU_THREADS)).cuda()
        W16 = torch.from_numpy(synth.make_w(w, threads=CPU_THREADS)).cuda()
        Wq, sw = mm.quantize_weight(W16)
        ws = mm.new_workspace(T, K, N)
        Y = torch.empty((T, N), dtype=torch.float16, device="cuda")
        res = {"workload": name, "T": T, "K": K, "N": N, "planted": w.n_dims}
        for tag, w16 in (("", W16), ("halved_", None)):
            def step(i, e, w16=w16):
                if e is not None:
                    e[0].record()
                mm.quantize_activations(X, N, w.tau, ws)
                if e is not None:
                    e[1].record()
                mm.matmul_prepared(ws, T, K, Wq, sw, w16, out=Y)
                if e is not None:
                    e[2].record()
            prewarm(torch, step, prewarm_s)
            wall, evs = timed_loop(torch, steps, warmup, step)
            act = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
            gemm = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
            res[tag + "ms"] = round(wall * 1e3 / steps, 4)
            res[tag + "TOPS"] = round(2.0 * T * K * N * steps / wall / 1e12, 1)
            res[tag + "activation_ms"] = round(act, 4)
            res[tag + "gemm_ms"] = round(gemm, 4)
        dbg = mm.mixed_matmul_debug(X, Wq, sw, W16, w.tau)
        res["o"] = int(dbg["count"][0])
        rows.append(res)
        log(f"sweep {name}: o={res['o']}, {res['ms']:.3f} ms ({res['TOPS']} TOPS), "
            f"memory-halved {res['halved_ms']:.3f} ms")
        del X, W16, Wq, sw, ws, Y, dbg
        torch.cuda.empty_cache()
    return rows


def measured_ceilings(torch):
    """What this chip delivers, measured in the same run: a bare int8 MFMA
    loop (independent accumulators, no memory traffic) and a coalesced
    stream read of 2 GiB, each with the shader clock it ran at (libceiling,
    built beside the library)."""
    import ctypes
    path = os.path.join(ROOT, "int8_mixed_precision_amd", "libceiling.so")
    lib = ctypes.CDLL(path)
    vp, ci, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.ceiling_mfma_i8.argtypes = [ci, ci, ci, vp, vp, vp]
    lib.ceiling_stream.argtypes = [vp, i64, ci, ci, vp, vp, vp]
    ops_iter = lib.ceiling_mfma_ops_per_iter()
    stream = lambda: vp(torch.cuda.current_stream().cuda_stream)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    out = {}

    def timed(launch, clk, reps=5):
        for _ in range(2):
            launch()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            launch()
        b.record()
        torch.cuda.synchronize()
        c = clk.view(-1, 2).cpu().numpy().astype(np.float64)
        ghz = float(np.mean(c[:, 0] / (c[:, 1] / 100e6)) / 1e9)
        return a.elapsed_time(b) / reps, ghz

    # two instruction forms on pseudo-random operands; the better one is
    # the ceiling (the part is power limited: the form and the operand
    # bits decide the clock it holds)
    grid, iters = 1024, 2000         # 4 workgroups of 8 waves per CU, ~4 ms per launch
    forms = {0: "v_mfma_i32_32x32x32_i8", 1: "v_mfma_i32_16x16x64_i8"}
    mf = []
    for form, name in forms.items():
        clk = torch.zeros(2 * grid, dtype=torch.int64, device="cuda")
        rc = []
        ms, ghz = timed(lambda: rc.append(lib.ceiling_mfma_i8(form, grid, iters, vp(sink.data_ptr()),
                                                               vp(clk.data_ptr()), stream())), clk)
        if any(rc):
            raise RuntimeError(f"ceiling_mfma_i8 form {form}: status {max(rc)}")
        ops = grid * 8 * iters * float(ops_iter)
        mf.append({"TOPS": round(ops / (ms * 1e-3) / 1e12, 1), "clock_GHz": round(ghz, 3),
                   "kernel": f"back-to-back {name} on pseudo-random operands, no memory traffic"})
    out["mfma_i8"] = dict(max(mf, key=lambda r: r["TOPS"]), all=mf)
    nbytes = 2 << 30
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    # (variant, grid): grid-stride 16 loads x 256 lanes on 256 workgroups;
    # grid-stride 32 x 256 on 512; partitioned 16 x 512 on 256 and 1024;
    # partitioned 16 x 256 on 2048 (the best shapes of a sweep; the best of
    # them in this run is the ceiling)
    shapes = [(0, 256), (1, 512), (2, 256), (2, 1024), (3, 2048)]
    names = {0: "grid-stride, 16 loads x 256 lanes", 1: "grid-stride, 32 loads x 256 lanes",
             2: "partitioned, 16 loads x 512 lanes", 3: "partitioned, 16 loads x 256 lanes"}
    runs = []
    for variant, grid in shapes:
        clk = torch.zeros(2 * grid, dtype=torch.int64, device="cuda")
        rc = []
        ms, ghz = timed(lambda: rc.append(lib.ceiling_stream(vp(buf.data_ptr()), nbytes, grid, variant,
                                                             vp(sink.data_ptr()), vp(clk.data_ptr()),
                                                             stream())), clk)
        if any(rc):
            raise RuntimeError(f"ceiling_stream variant {variant} grid {grid}: status {max(rc)}")
        runs.append({"GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1), "clock_GHz": round(ghz, 3),
                     "order": names[variant], "workgroups": grid})
    best = max(runs, key=lambda r: r["GB/s"])
    out["hbm_read"] = {**best, "kernel": "coalesced 16-byte loads over 2 GiB (best of the shapes tried)",
                       "all": [{k: r[k] for k in ("GB/s", "order", "workgroups")} for r in runs]}
    del buf
    torch.cuda.empty_cache()
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_stages(oracle, X, Wq, sw, W16, tau, rows, threads):
    """Seconds per oracle step (the steps as the pages order them) on the
    listed rows; detection and isolation always see every row."""
    t = {}
    t0 = time.perf_counter()
    flag = oracle.detect(X, tau)
    t["detect"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    idx = oracle.compact(flag)
    t["isolate"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    xq, sx = oracle.quantize_rows(X, flag, rows=rows)
    t["quantize_x"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    acc = oracle.int8_gemm(xq, Wq, threads=threads)
    t["int8_gemm"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.output(acc, sx, sw, X, W16, idx, rows=rows, threads=threads)
    t["dequant_and_outliers"] = time.perf_counter() - t0
    return t


def cpu_baseline(synth):
    """The oracle, as it is, on the host's cores: per-step times at one
    thread and at CPU_THREADS threads (the host-core share of one GPU) for
    the tiny and decode workloads in full and for a row sample of the
    prefill up-projection; value = the up-projection's TOPS with the
    per-row steps extrapolated from the sample to all rows."""
    import oracle
    res = {"kind": "oracle", "unit": "TOPS", "cores": CPU_THREADS,
           "nproc": os.cpu_count(), "cpu_model": cpu_model()}
    stages = {}
    for name in ("tiny", "dec"):
        w = synth.WORKLOADS[name]
        X, W = synth.make_x(w, threads=CPU_THREADS), synth.make_w(w, threads=CPU_THREADS)
        Wq, sw = oracle.quantize_weight(W, threads=CPU_THREADS)
        for th in (1, CPU_THREADS):
            st = oracle_stages(oracle, X, Wq, sw, W, w.tau, None, th)
            stages[f"{name}_{th}t"] = {k: round(v, 6) for k, v in st.items()}
        del X, W, Wq
    w = synth.WORKLOADS["up"]
    T, K, N = w.T, w.K, w.N
    X = synth.make_x(w, threads=CPU_THREADS)
    W = synth.make_w(w, threads=CPU_THREADS)
    Wq, sw = oracle.quantize_weight(W, threads=CPU_THREADS)
    one = np.linspace(0, T - 1, 4).astype(np.int64)
    st1 = oracle_stages(oracle, X, Wq, sw, W, w.tau, one, 1)
    # size the all-core sample to about CPU_TARGET_S from the one-thread rate
    per_row_1t = (st1["quantize_x"] + st1["int8_gemm"] + st1["dequant_and_outliers"]) / len(one)
    rows = int(min(T, max(CPU_THREADS, CPU_TARGET_S * CPU_THREADS * 0.8 / max(per_row_1t, 1e-6))))
    rows -= rows % CPU_THREADS
    sample = np.linspace(0, T - 1, rows).astype(np.int64)
    stn = oracle_stages(oracle, X, Wq, sw, W, w.tau, sample, CPU_THREADS)
    stages[f"up_1t_{len(one)}rows"] = {k: round(v, 6) for k, v in st1.items()}
    stages[f"up_{CPU_THREADS}t_{rows}rows"] = {k: round(v, 6) for k, v in stn.items()}
    per_row = (stn["quantize_x"] + stn["int8_gemm"] + stn["dequant_and_outliers"]) / rows
    whole = stn["detect"] + stn["isolate"] + per_row * T
    res.update({
        "value": round(2.0 * T * K * N / whole / 1e12, 4),
        "sample": f"prefill up-projection: detection and isolation over all {T} rows, the "
                  f"per-row steps on {rows} of {T} rows at {CPU_THREADS} threads, extrapolated "
                  f"to {T} rows ({whole:.1f} s for the whole call); weight conversion untimed",
        "stages_s": stages,
        "note": "stages_s: seconds per oracle step (detect, isolate, quantize_x, int8_gemm, "
                "dequant_and_outliers); <config>_<threads>t, tiny and dec in full; the "
                "oracle runs detect, isolate and quantize_x on one thread whatever the "
                "thread count, int8_gemm and dequant_and_outliers on the threads given",
    })
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              "(sharding over several GPUs is described, not implemented)", file=sys.stderr)
        sys.exit(2)
    import torch

    import int8_mixed_precision_amd as mm
    import synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("copy calibration: 3 copies of 1 GiB")

    if args.sweep:
        rows = bench_sweep(torch, mm, synth, args.steps, args.warmup, PREWARM_S / 2)
        print(json.dumps({"metric": "int8-mixed matmul time vs outlier count, 175B-class "
                                    "block projections at T=4096", "unit": "ms",
                          "steps": args.steps, "warmup": args.warmup, "data": "synthetic",
                          "results": rows}), flush=True)
        return

    pre = dec = None
    if args.only in (None, "prefill"):
        pre = bench_prefill(torch, mm, synth, args.steps, args.warmup, not args.no_variants)
        log(f"prefill: {pre['tops']:.1f} TOPS ({pre['ms_per_step']:.3f} ms/step), "
            f"gemm {pre['gemm_ms']:.3f} ms, activation pass "
            + (f"{pre['activation_ms']:.3f} ms" if pre["activation_ms"] is not None else "n/a (one step)")
            + (f"; memory-halved {pre['halved_tops']:.1f} TOPS, bf16 {pre['bf16_tops']:.1f} TOPS"
               if "halved_tops" in pre else ""))
        torch.cuda.empty_cache()
    down = None
    if (args.only is None and not args.no_variants) or args.only == "down":
        down = bench_down(torch, mm, synth, args.steps, args.warmup)
        log(f"down: {down['TOPS']:.1f} TOPS ({down['ms_per_call']:.3f} ms/call, o = {down['outlier_dims']})")
    if args.only in (None, "decode"):
        dec = bench_decode(torch, mm, synth, args.steps, args.warmup, not args.no_variants)
        log(f"decode: {dec['weight_gbs']:.1f} GB/s weight ({dec['call_ms'] * 1e3:.1f} us/call)"
            + (f"; memory-halved {dec['halved_weight_gbs']:.1f} GB/s "
               f"({dec['halved_call_ms'] * 1e3:.1f} us/call), bf16 {dec['bf16_weight_gbs']:.1f} GB/s "
               f"({dec['bf16_call_ms'] * 1e3:.1f} us/call)" if "halved_weight_gbs" in dec else ""))

    sweep = None
    if args.only is None and not args.no_variants and not args.no_sweep:
        log("sweep: 175B-class block projections at T=4096, 0/8/64/256 planted outlier dims")
        sweep = bench_sweep(torch, mm, synth, 5, 2, 0.05)
    ceil = None
    if not args.no_ceilings:
        log("measured ceilings: bare int8 MFMA loop, 2 GiB stream read")
        ceil = measured_ceilings(torch)

    gemm_digest = src_digest(["k_gemm.hip", "common.hpp"])
    decode_digest = src_digest(["k_decode.hip", "common.hpp"])
    out = {
        "metric": "int8-mixed matmul TOPS @ T=2048 K=12288 N=49152; weight GB/s @ T=8",
        "higher_is_better": True, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "scaling": "weak", "vs_baseline": None, "dtype": "i8", "data": "synthetic",
    }
    if pre is not None:
        ach = pre["gemm_tops"]
        out.update({
            "value": round(pre["tops"], 2), "unit": "TOPS",
            "ms_per_step": round(pre["ms_per_step"], 4),
            "config": {"workload": "prefill 175B-class FFN up-projection (LLM.int8() matmul, "
                                   "W pre-converted to Int8)",
                       "T": pre["T"], "K": pre["K"], "N": pre["N"], "tau": pre["tau"],
                       "outlier_dims": pre["o"],
                       "fraction_8bit": round((pre["K"] - pre["o"]) / pre["K"], 6)},
            "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_INT8_TOPS,
                         "unit": "TFLOP/s", "frac": round(ach / PEAK_INT8_TOPS, 4),
                         "traffic": measured_traffic("gemm_i8_prefill_up_traffic.md",
                                                     gemm_digest, "hbm_bytes_per_launch"),
                         "kernel": "k_gemm_i8_big (int8 MFMA + fused dequant/fp16 outlier epilogue)",
                         "work": "2*T*K*N int8 ops per launch", "ms": round(pre["gemm_ms"], 4)},
            # activation_pass: previous matmul end to this matmul start (the
            # two activation kernels and the launch gaps around them)
            "stages_ms": {"activation_pass": (round(pre["activation_ms"], 4)
                                              if pre["activation_ms"] is not None else None),
                          "gemm": round(pre["gemm_ms"], 4)},
            "quantize_weight": {"ms": round(pre["quantize_weight_ms"], 4),
                                "GB/s": round(pre["quantize_weight_gbs"], 1),
                                "bytes": "one read of W (2KN, or 4KN for fp32) + KN + 4N "
                                         "written"},
        })
        if "halved_tops" in pre:
            alt = ("timed call by call alternated with the fp16 call (fp16 "
                   f"{pre['alternated_f16_ms']:.4f} ms per call in the same loop)")
            out["memory_halved"] = {"note": "W16 not passed: outlier rows recovered from the "
                                            "Int8 weight (same X, W, tau); " + alt,
                                    "TOPS": round(pre["halved_tops"], 2),
                                    "ms_per_step": round(pre["halved_ms_per_step"], 4)}
            out["bf16_variant"] = {"note": "X, W16, Y bfloat16 (the same values rounded to "
                                           "bf16); whole int8_mixed_matmul_bf16 calls; " + alt,
                                   "TOPS": round(pre["bf16_tops"], 2),
                                   "ms_per_step": round(pre["bf16_ms_per_step"], 4)}
            out["quantize_weight"]["from_bf16"] = pre["convert"]["bf16"]
            out["quantize_weight"]["from_f32"] = pre["convert"]["f32"]
            # weight bytes the matmul needs: Int8 + scales against the 16-bit
            # weight (memory-halved variant), or plus the 16-bit copy
            K, N = pre["K"], pre["N"]
            out["memory_halved"]["weight_memory_ratio"] = round((K * N + 4.0 * N) / (2.0 * K * N), 4)
        if "vendor_int8_gemm" in pre:
            out["roofline"]["vendor_int8_gemm"] = pre["vendor_int8_gemm"]
        if ceil is not None:
            m = ceil["mfma_i8"]["TOPS"]
            out["roofline"]["measured_peak"] = {"value": m, "unit": "TFLOP/s",
                                                **{k: v for k, v in ceil["mfma_i8"].items() if k != "all"}}
            out["roofline"]["frac_of_measured"] = round(ach / m, 4)
    if dec is not None:
        d = {"metric": "weight GB/s @ T=8", "value": round(dec["weight_gbs"], 1), "unit": "GB/s",
             "ms_per_step": round(dec["ms_per_step"], 5), "steps": dec["steps"],
             "launch": f"HIP graph replays of {CALLS_PER_REPLAY} calls ({DECODE_PASSES} passes over "
                       f"the {DECODE_ROTATE} rotating weight copies)",
             "config": {"workload": "decode FFN up-projection, W pre-converted to Int8, "
                                    f"{DECODE_ROTATE} rotating weight copies",
                        "T": dec["T"], "K": dec["K"], "N": dec["N"], "tau": dec["tau"],
                        "outlier_dims": dec["o"]},
             "roofline": {"bound": "hbm", "achieved": round(dec["alg_gbs"], 1),
                          "peak": PEAK_HBM_GBS, "unit": "GB/s",
                          "frac": round(dec["alg_gbs"] / PEAK_HBM_GBS, 4),
                          "traffic": measured_traffic("decode_dec_traffic.md", decode_digest, "hbm_bytes_per_launch"),
                          "kernel": "k_decode (the whole int8_mixed_matmul call)",
                          "work": "2TK + KN + 4N + 2oN + 2TN bytes per call",
                          "ms": round(dec["call_ms"], 5)}}
        if "halved_weight_gbs" in dec:
            d["memory_halved"] = {"note": "W16 not passed: outlier rows recovered from the "
                                          "Int8 weight",
                                  "weight GB/s": round(dec["halved_weight_gbs"], 1),
                                  "call_ms": round(dec["halved_call_ms"], 5)}
            d["bf16_variant"] = {"note": "X, W16, Y bfloat16",
                                 "weight GB/s": round(dec["bf16_weight_gbs"], 1),
                                 "call_ms": round(dec["bf16_call_ms"], 5)}
            d["warm"] = {"note": "one weight copy in every call (cache resident); the metric "
                                 "rotates 8 copies",
                         "weight GB/s": round(dec["warm_weight_gbs"], 1),
                         "call_ms": round(dec["warm_call_ms"], 5)}
        if ceil is not None:
            m = ceil["hbm_read"]["GB/s"]
            d["roofline"]["measured_peak"] = {"value": m, "unit": "GB/s",
                                              **{k: v for k, v in ceil["hbm_read"].items() if k != "all"}}
            d["roofline"]["frac_of_measured"] = round(dec["alg_gbs"] / m, 4)
        if pre is None:
            out.update({"value": d["value"], "unit": "GB/s", "ms_per_step": d["ms_per_step"],
                        "config": d["config"], "roofline": d["roofline"]})
        else:
            out["decode"] = d
    if down is not None:
        out["other_configs"] = {"down": {
            "workload": "prefill FFN down-projection (whole int8_mixed_matmul calls, W "
                        "pre-converted to Int8)", **down}}
    if dec is not None and "batched" in dec:
        out.setdefault("other_configs", {})["batched_decode"] = {
            "workload": "decode FFN up-projection weights (K=8192, N=28672, 8 rotating copies) "
                        "with 32 and 128 activation rows, whole calls from a HIP graph",
            "results": dec["batched"]}
    if sweep is not None:
        out.setdefault("other_configs", {})["sweep_175b_block"] = {
            "workload": "175B-class block projections (QKV 12288->36864, out 12288->12288, up "
                        "12288->49152, down 49152->12288) at T=4096 with 0, 8, 64 and 256 planted "
                        "outlier dims; whole calls with and without W16 (memory-halved), "
                        "5 timed steps each",
            "results": sweep}
    if ceil is not None:
        out["measured_ceilings"] = ceil
    if not args.no_cpu_baseline and pre is not None:
        log("cpu baseline: oracle steps at 1 and all threads")
        out["cpu_baseline"] = cpu_baseline(synth)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
