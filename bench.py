"""Benchmark of the packed low-bit BitLinear hot path on one MI355X.

Headline workload (one "step"): an i2_s BitLinear decode step of a
30-layer, hidden-2560 BitNet-2B-like stack at M = 1 with fp32 activations --
per layer Q, K, V, O (2560 x 2560), up and gate (6912 x 2560) and down
(2560 x 6912), each with its own synthetic activation (Q/K/V share one,
up/gate share one).  The 210 products of a step run as one prepared batch
(two launches: activation digit planes + product).  The metric is effective
weight bandwidth: packed bytes read per step (codes plus the 4-byte tail
scale of each matrix, 594.7 MB, more than twice the 256 MiB Infinity Cache)
divided by the step time.

The JSON line also carries the roofline of the dominant kernel (the batched
product, timed live with HIP events on its stream; its HBM traffic is taken
from the committed rocprofv3 counter summary when that summary was made from
the current kernel source, and the rate of a read-only streaming kernel as
the practical bound), the CPU oracle on the whole step (its rows split over
every host core, and on one core; the median of three runs each), and
extras: single-call per-matrix GEMV times (fp32 and int8 activations), the
same step with the fused epilogues and as dependent per-layer batches, the
TQ2_0 small-batch GEMV, the W1A8 products of hidden 5120 (single calls, a
plain bf16 matmul of the same shapes as context, and prepared batches of 12
decoder layers), the int8 prefill GEMM with i2_s, TQ2_0 and W1 weights (TOPS
against the int8 matrix-core peak) and the one-shot bf16 layer.

The second half of the metric, the i2_s int8 prefill GEMM at M = 512, is
reported as "roofline_gemm": the GEMM kernel timed the same way (back-to-back
launches between HIP events), int8 TOPS against the dense int8 peak, with its
HBM traffic and matrix-core busy fraction from its own committed counter
summary when that matches the current source.

"roofline_w1a8" reports the W1A8 LM head (248320 x 5120, G = 128, M = 1) the
same way, whole calls over rotating weight copies.

Warm-up is by time as well as by count: after the W warm-up steps the step
keeps running until at least 80 ms of continuous work have passed
(reported as "warmup_settle_ms"), because after an idle period (the host
builds 595 MB of synthetic weights before the timing) the step takes about
20 ms to reach its steady time, and a timed window inside that ramp reads up
to 10% slow.  The other lines (GEMM, W1A8, extras) run their own calls for
at least 60 ms before timing (settle()), since some follow the CPU oracle
leg.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extras]
       python bench.py --gemm-only      (the GEMM roofline alone)
       python bench.py --w1-only        (the W1A8 LM-head line alone)
       python bench.py --copy-probe     (a plain 256 MiB device copy, to
                                         calibrate rocprofv3 byte counters)
"""
import hashlib
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 matrix cores, published (POP/s x 1000)
LAYERS = 30
HIDDEN, FFN = 2560, 6912
# dominant kernel of a step: i2_s, M = 1, fp4 digit planes on the fp4 matrix cores
KERNEL = "f4_batch_kernel<1, false, 1>"
KERNEL_SOURCES = ["binary_bit_weight_amd/csrc/gemv_fp4.hip", "binary_bit_weight_amd/csrc/common.h"]
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "f4_batch_i2s_m1_decode30_counters.md")
# the other half of the metric: the i2_s int8 prefill GEMM at M = 512
GEMM_KERNEL = "gemm_i8_i2s_kernel"
GEMM_SOURCES = ["binary_bit_weight_amd/csrc/gemm_i8.hip", "binary_bit_weight_amd/csrc/common.h"]
GEMM_SUMMARY = os.path.join(ROOT, "profiles", "gemm_i8_i2s_m512_counters.md")
GEMM_SHAPES = [(6912, 2560), (2560, 6912)]    # (N, K) at M = 512; the first is the roofline line
# W1A8 (binary weights, int8 activations): the LM head at hidden 5120, G = 128
W1_KERNEL = "w1_stream_kernel"
W1_SOURCES = ["binary_bit_weight_amd/csrc/gemv_w1.hip", "binary_bit_weight_amd/csrc/common.h"]
W1_SUMMARY = os.path.join(ROOT, "profiles", "w1_stream_lm_head_m1_counters.md")
W1_HEAD = (248320, 5120, 128)
COPY_PROBE_BYTES = 256 << 20
ROLES = [("q", HIDDEN, HIDDEN, 0), ("k", HIDDEN, HIDDEN, 0), ("v", HIDDEN, HIDDEN, 0), ("o", HIDDEN, HIDDEN, 1),
         ("up", FFN, HIDDEN, 2), ("gate", FFN, HIDDEN, 2), ("down", HIDDEN, FFN, 3)]   # (name, N, K, x slot)


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_sha(sources=None):
    h = hashlib.sha256()
    for f in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def summary_values(path, sources):
    """The 'key: value' lines of a committed counter summary, or {} when it is
    missing or was taken from another version of the kernel source."""
    try:
        kv = {}
        with open(path) as fh:
            for line in fh:
                if ":" in line and line.startswith("- "):
                    k, v = line[2:].split(":", 1)
                    kv[k.strip()] = v.strip().strip("`")
        return kv if kv.get("kernel_source_sha256_16") == kernel_source_sha(sources) else {}
    except OSError:
        return {}


def profiled_traffic():
    """HBM bytes per launch of KERNEL from the committed counter summary, or
    None when it is missing or stale."""
    try:
        return int(summary_values(TRAFFIC_SUMMARY, KERNEL_SOURCES)["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_probe():
    """A plain device-to-device copy of COPY_PROBE_BYTES, five times: run under
    rocprofv3 --pmc FETCH_SIZE (or WRITE_SIZE) to learn how many counter KiB
    one byte of known traffic reads as."""
    import torch
    src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device="cuda").fill_(7)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": COPY_PROBE_BYTES, "copies": 5}), flush=True)


def build_decode_step(L, synth, torch, dev):
    """Seven distinct packed matrices (one per role, seeds 201..207), each
    copied to LAYERS distinct device buffers; activations N(0,1) per layer
    and slot."""
    packed = {}
    for i, (name, N, K, _) in enumerate(ROLES):
        w = synth.ternary(201 + i, N, K)
        scale = float(synth.uniform_f32(211 + i, 1, 0.01, 0.1)[0])
        packed[name] = (L.ll_pack_i2s(w, scale), N, K)
    items, weight_bytes, keep = [], 0, []
    for layer in range(LAYERS):
        xs = [torch.from_numpy(synth.normal_f32(1000 + 4 * layer + s, 1, HIDDEN if s != 3 else FFN)).to(dev)
              for s in range(4)]
        keep.append(xs)
        for name, N, K, slot in ROLES:
            p, _, _ = packed[name]
            W = L.upload_i2s(p, N, K, dev)
            y = torch.empty((1, N), dtype=torch.float32, device=dev)
            items.append((W, xs[slot], None, y))
            weight_bytes += p.size
    return packed, items, weight_bytes


_W1_HOST = {}


def w1_weights(L, synth, seed, N, K, G):
    """Sign bits and fp16 group mean-abs scales of dense N(0, 0.02) rows
    (generated in 4096-row chunks, converted by ll_w1_from_dense); built once
    per (seed, N, K, G) and process."""
    key = (seed, N, K, G)
    if key in _W1_HOST:
        return _W1_HOST[key]
    bits = np.empty((N, K // 32), np.uint32)
    scales = np.empty((N, K // G), np.uint16)
    for c in range((N + synth.CHUNK_ROWS - 1) // synth.CHUNK_ROWS):
        r0 = c * synth.CHUNK_ROWS
        rows = min(synth.CHUNK_ROWS, N - r0)
        bits[r0:r0 + rows], scales[r0:r0 + rows] = L.ll_w1_from_dense(synth.dense_chunk(seed, K, c, rows), G)
    _W1_HOST[key] = (bits, scales)
    return bits, scales


def settle(torch, fn, seconds=0.06):
    """Runs fn(i) in batches of 20 calls until `seconds` of wall time have
    passed: after an idle period the GPU clocks need about 20 ms of
    continuous work to reach their steady state."""
    t0, i = time.perf_counter(), 0
    while True:
        for _ in range(20):
            fn(i)
            i += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return


def time_graph(torch, call, copies, calls, stream):
    """GPU time of one call: `calls` calls (call(i, stream) with i cycling
    over `copies` weight copies) captured in one HIP graph and replayed, so
    the host's per-call cost stays out of the figure."""
    for i in range(copies):
        call(i, None)                               # warm-up; sets per-kernel launch attributes
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            call(i % copies, None)
    settle(torch, lambda i: g.replay())
    ms = time_events(torch, g.replay, 3, stream)
    del g
    return ms / calls


def time_events(torch, fn, reps, stream):
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for _ in range(reps):
        fn()
    e.record(stream)
    e.synchronize()
    return s.elapsed_time(e) / reps


def cpu_baseline(oracle, packed, items):
    """The oracle (fp64, decoding every weight from the packed bytes) on the
    whole decode step the GPU leg runs -- its 210 products on their own
    activations -- single-threaded and with its rows split over every host
    core (oracle.cores()); the median of three runs of each."""
    xs = [x.cpu().numpy() for (_, x, _, _) in items]
    nbytes = sum(packed[name][0].size for _ in range(LAYERS) for (name, _, _, _) in ROLES)

    def run(threads):
        t0 = time.perf_counter()
        for layer in range(LAYERS):
            for r, (name, N, K, _) in enumerate(ROLES):
                oracle.i2s_gemv_f32(packed[name][0], N, K, xs[len(ROLES) * layer + r], threads=threads)
        return time.perf_counter() - t0

    cores = oracle.cores()
    one = sorted(run(1) for _ in range(3))[1]
    allc = sorted(run(cores) for _ in range(3))[1]
    return {"value": round(nbytes / allc / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": "the whole 30-layer decode step (210 i2_s GEMVs, %.1f MB, the GPU leg's activations), "
                      "median of 3 runs: %.2f s on %d host threads" % (nbytes / 1e6, allc, cores),
            "single_thread": {"value": round(nbytes / one / 1e9, 4), "unit": "GB/s", "cores": 1,
                              "seconds": round(one, 3)}}


def stream_probe(L, torch, dev, stream, nbytes=1 << 30):
    """Plain streaming read of a 1 GiB device buffer (ll_probe_stream_read),
    timed with HIP events: the read rate the weight-streaming kernels are
    compared with."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(3)
    blocks = 256 * 8
    sink = torch.empty(blocks, dtype=torch.int32, device=dev)
    settle(torch, lambda i: L.ll_probe_stream_read(buf, sink, blocks, stream))
    ms = time_events(torch, lambda: L.ll_probe_stream_read(buf, sink, blocks, stream), 20, stream)
    del buf
    torch.cuda.empty_cache()
    return {"GB_s": round(nbytes / (ms * 1e-3) / 1e9, 1), "bytes": nbytes, "ms": round(ms, 4)}


def dependent_decode_step(L, torch, items, weight_bytes, steps, stream):
    """The same 30 layers with the products of a layer grouped as a real
    decode orders them: Q/K/V (one activation), O, up/gate (one activation),
    down -- 120 prepared batches run one after another (2 launches each),
    captured in one HIP graph.  Each batch waits for the one before, as a
    layer's input waits for the previous layer's output."""
    plans = []
    for layer in range(LAYERS):
        it = items[len(ROLES) * layer: len(ROLES) * (layer + 1)]
        for group in ([0, 1, 2], [3], [4, 5], [6]):
            plans.append(L.GemvPlan([it[r] for r in group], 1))

    def run(st):
        for pl in plans:
            pl.prepare(st)
            pl.product(st)
    run(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(None)
    settle(torch, lambda i: g.replay())
    ms = time_events(torch, g.replay, steps, stream)
    del g
    return {"ms_per_step": round(ms, 4), "GB_s": round(weight_bytes / (ms * 1e-3) / 1e9, 1), "batches": len(plans),
            "note": "per layer: Q/K/V, O, up/gate, down as four prepared batches in order (graph replay)"}


def gemm_operands(L, synth, torch, dev, stream, N, K, M=512):
    """i2_s weights (seed 401) and bf16 activations N(0,1) (seed 402)
    quantized per token; output and a zero-filled split-K workspace."""
    w = synth.ternary(401, N, K)
    p = L.ll_pack_i2s(w, 0.05)
    W = L.upload_i2s(p, N, K, dev)
    xb = torch.from_numpy(synth.normal_bf16_bits(402, M, K).view(np.int16)).to(dev).view(torch.bfloat16)
    xq, xsc = L.quantize(xb, stream)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    gws = torch.zeros((max(L.ll_gemm_workspace_size(W, M), 16),), dtype=torch.uint8, device=dev)
    return W, xb, xq, xsc, y, gws


def gemm_roofline(L, synth, torch, dev, stream, steps, M=512):
    """The int8 GEMM kernel launched back to back `steps` times between two
    HIP events on its stream, per shape; TOPS = 2 M N K per launch / kernel
    time, against the dense int8 matrix-core peak."""
    lines = []
    for N, K in GEMM_SHAPES:
        W, _, xq, xsc, y, gws = gemm_operands(L, synth, torch, dev, stream, N, K, M)
        settle(torch, lambda i: L.ll_bitlinear_gemm(W, xq, xsc, M, None, y, None, gws, stream))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            L.ll_bitlinear_gemm(W, xq, xsc, M, None, y, None, gws, stream)
        e1.record(stream)
        e1.synchronize()
        ms = e0.elapsed_time(e1) / steps
        ops = 2 * M * N * K
        tops = ops / (ms * 1e-3) / 1e12
        lines.append({"workload": "i2_s int8 GEMM M=%d N=%d K=%d (bf16 x ~ N(0,1) quantized per token)" % (M, N, K),
                      "achieved": round(tops, 1), "frac": round(tops / INT8_PEAK_TOPS, 4),
                      "kernel_ms": round(ms, 5), "algorithmic_ops_per_launch": ops})
        del W, xq, xsc, y, gws
    kv = summary_values(GEMM_SUMMARY, GEMM_SOURCES)
    head = lines[0]
    res = {"bound": "mfma", "achieved": head["achieved"], "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
           "frac": head["frac"], "workload": head["workload"], "kernel": GEMM_KERNEL, "kernel_ms": head["kernel_ms"],
           "algorithmic_ops_per_launch": head["algorithmic_ops_per_launch"],
           "traffic": int(kv["hbm_bytes_per_launch"]) if "hbm_bytes_per_launch" in kv else None,
           "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
           "mfma_busy_frac": float(kv["mfma_busy_frac"]) if "mfma_busy_frac" in kv else None,
           "kernel_source_sha256_16": kernel_source_sha(GEMM_SOURCES),
           "other_shapes": lines[1:]}
    return res


def fused_decode_items(L, synth, torch, dev, items, eps=1e-5):
    """The decode step's products with the pages' fused kernels, as one
    BitNet layer runs them: Q, K, V from the RMS-normalised input; O and down
    from their sub-norms plus the residual stream (as the bias); gate and up
    as one gated pair (y = relu(gate)^2 * up) of the normalised FFN input.
    Returns (plan items, per-layer (norms, residuals)); the same weights."""
    fused, extra = [], []
    for layer in range(LAYERS):
        by = {name: items[len(ROLES) * layer + r] for r, (name, _, _, _) in enumerate(ROLES)}
        res_h = [torch.from_numpy(synth.normal_f32(5000 + 2 * layer + j, 1, HIDDEN)).to(dev).reshape(HIDDEN)
                 for j in range(2)]
        norms = [torch.from_numpy(synth.uniform_f32(6000 + 4 * layer + j, HIDDEN if j != 3 else FFN, 0.5, 1.5)).to(dev)
                 for j in range(4)]                       # attention input, attention sub, FFN input, FFN sub
        extra.append((norms, res_h))
        for name in ("q", "k", "v"):
            W, x, _, y = by[name]
            fused.append(L.Normed(W, x, norms[0], eps, None, y))
        W, x, _, y = by["o"]
        fused.append(L.Normed(W, x, norms[1], eps, res_h[0], y))
        (Wu, xu, _, yu), (Wg, _, _, _) = by["up"], by["gate"]
        fused.append(L.Relu2Mul(Wg, Wu, xu, yu, norm=(norms[2], eps)))
        W, x, _, y = by["down"]
        fused.append(L.Normed(W, x, norms[3], eps, res_h[1], y))
    return fused, extra


def fused_decode_step(L, synth, torch, dev, stream, items, weight_bytes, steps):
    """The same 30-layer decode step with the fused kernels (fused_decode_items);
    same weights and bytes as the headline step; prepare + product per step,
    timed with HIP events."""
    fused, extra = fused_decode_items(L, synth, torch, dev, items)
    plan = L.GemvPlan(fused, 1)
    settle(torch, lambda i: plan.run(stream))
    ms = time_events(torch, lambda: plan.run(stream), steps, stream)
    return {"ms_per_step": round(ms, 4), "GB_s": round(weight_bytes / (ms * 1e-3) / 1e9, 1),
            "products": len(fused), "tiles": int(plan.plan.tiles),
            "note": "RMSNorm prologues on Q/K/V, O, gate/up, down; gate+up as 30 gated pairs (relu^2 * up); "
                    "residual added to O and down"}


def w1_roofline(L, synth, torch, dev, stream, steps):
    """The W1A8 LM head (248320 x 5120, G = 128) at M = 1 and 8: whole calls
    (preparation + product) back to back between HIP events, rotating over 4
    device copies of the weights (past twice the Infinity Cache); effective
    weight bandwidth against the HBM peak."""
    N, K, G = W1_HEAD
    bits, sc = w1_weights(L, synth, 503, N, K, G)
    wbytes = bits.nbytes + sc.nbytes
    reps = max(1, int(np.ceil(2 ** 29 / wbytes)))
    Ws = [L.upload_w1(bits, sc, K, G, dev) for _ in range(reps)]
    lines = []
    for M in (1, 8):
        x = torch.from_numpy(synth.normal_f32(510 + M, M, K)).to(dev)
        xq, xsc = L.quantize(x, stream)
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        ws = torch.zeros((L.ll_gemv_workspace_size(Ws[0], L.LL_ACT_I8, M),), dtype=torch.uint8, device=dev)
        settle(torch, lambda i: L.ll_bitlinear_gemv(Ws[i % reps], L.LL_ACT_I8, xq, xsc, M, None, y, ws, stream))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = max(steps, 4 * reps)
        e0.record(stream)
        for i in range(n):
            L.ll_bitlinear_gemv(Ws[i % reps], L.LL_ACT_I8, xq, xsc, M, None, y, ws, stream)
        e1.record(stream)
        e1.synchronize()
        ms = e0.elapsed_time(e1) / n
        gbs = wbytes / (ms * 1e-3) / 1e9
        lines.append({"workload": "W1A8 LM head %d x %d, G = %d, M = %d (int8 x from N(0,1)), %d weight copies rotated"
                                  % (N, K, G, M, reps),
                      "achieved": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4), "call_ms": round(ms, 5),
                      "algorithmic_bytes_per_call": int(wbytes)})
    del Ws
    torch.cuda.empty_cache()
    kv = summary_values(W1_SUMMARY, W1_SOURCES)
    head = lines[0]
    return {"bound": "hbm", "achieved": head["achieved"], "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": head["frac"],
            "workload": head["workload"], "kernel": W1_KERNEL + " (the whole call is this one launch)",
            "call_ms": head["call_ms"], "algorithmic_bytes_per_call": head["algorithmic_bytes_per_call"],
            "traffic": int(kv["hbm_bytes_per_launch"]) if "hbm_bytes_per_launch" in kv else None,
            "traffic_unit": "HBM bytes per product launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "kernel_source_sha256_16": kernel_source_sha(W1_SOURCES), "other_shapes": lines[1:]}


def extras_single(L, synth, torch, dev, stream):
    out = {}
    # the 256 x 512 i2_s GEMV of the smallest configuration (scale 1/16, seed 101)
    w = synth.ternary(101, 256, 512)
    p = L.ll_pack_i2s(w, 0.0625)
    reps = max(1, int(np.ceil(2 ** 29 / p.size / 64)))
    Ws = [L.upload_i2s(p, 256, 512, dev) for _ in range(reps)]
    x = torch.from_numpy(synth.normal_f32(102, 1, 512)).to(dev)
    y = torch.empty((1, 256), dtype=torch.float32, device=dev)
    ms = time_graph(torch, lambda i, st: L.ll_bitlinear_gemv(Ws[i], L.LL_ACT_F32, x, None, 1, None, y, None, st),
                    reps, max(2 * reps, 64), stream)
    out["i2s_gemv_f32_single_call_256x512"] = {"us": round(ms * 1e3, 2), "GB_s": round(p.size / (ms * 1e-3) / 1e9, 1),
                                               "weight_bytes": int(p.size)}
    del Ws
    for name, N, K in [("2560x2560", 2560, 2560), ("6912x2560", 6912, 2560), ("2560x6912", 2560, 6912)]:
        w = synth.ternary(5, N, K)
        p = L.ll_pack_i2s(w, 0.05)
        # rotate over enough copies to exceed 2 x 256 MiB
        reps = max(1, int(np.ceil(2 ** 29 / p.size)))
        Ws = [L.upload_i2s(p, N, K, dev) for _ in range(reps)]
        x = torch.from_numpy(synth.normal_f32(6, 1, K)).to(dev)
        y = torch.empty((1, N), dtype=torch.float32, device=dev)
        ws = torch.zeros((L.ll_gemv_workspace_size(Ws[0], L.LL_ACT_F32, 1),), dtype=torch.uint8, device=dev)
        ms = time_graph(torch, lambda i, st: L.ll_bitlinear_gemv(Ws[i], L.LL_ACT_F32, x, None, 1, None, y, ws, st),
                        reps, 2 * reps, stream)
        out["i2s_gemv_f32_single_call_" + name] = {"us": round(ms * 1e3, 2),
                                                   "GB_s": round(p.size / (ms * 1e-3) / 1e9, 1)}
        # the same matrix with int8 activations (ll_bitlinear_gemv, act = LL_ACT_I8): one plane per
        # token, all tokens in one pass over the weights
        for M in (1, 8, 16):
            q = torch.from_numpy(np.clip(np.rint(synth.normal_f32(7 + M, M, K) * 40), -127, 127).astype(np.int8)).to(dev)
            xs8 = torch.full((M,), 0.025, dtype=torch.float32, device=dev)
            y8 = torch.empty((M, N), dtype=torch.float32, device=dev)
            ws8 = torch.zeros((max(L.ll_gemv_workspace_size(Ws[0], L.LL_ACT_I8, M), 16),), dtype=torch.uint8, device=dev)
            ms = time_graph(torch, lambda i, st: L.ll_bitlinear_gemv(Ws[i], L.LL_ACT_I8, q, xs8, M, None, y8, ws8, st),
                            reps, 2 * reps, stream)
            out["i2s_gemv_i8_single_call_%s_M%d" % (name, M)] = {"us": round(ms * 1e3, 2),
                                                                 "GB_s": round(p.size / (ms * 1e-3) / 1e9, 1)}
    # TQ2_0 small batch, N=6912, K=2560
    N, K = 6912, 2560
    w = synth.ternary(301, N, K)
    sc = synth.uniform_f16_bits(302, N * K // 256, 0.005, 0.05)
    blocks = L.ll_pack_tq2(w, sc)
    reps = max(1, int(np.ceil(2 ** 29 / blocks.size)))
    Ws = [L.upload_tq2(blocks, N, K, dev) for _ in range(reps)]
    for M in (1, 8, 16):
        x = torch.from_numpy(synth.normal_f32(303, M, K)).to(dev)
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        ws = torch.zeros((max(L.ll_gemv_workspace_size(Ws[0], L.LL_ACT_F32, M), 16),), dtype=torch.uint8, device=dev)
        ms = time_graph(torch, lambda i, st: L.ll_bitlinear_gemv(Ws[i], L.LL_ACT_F32, x, None, M, None, y, ws, st),
                        reps, 2 * reps, stream)
        out["tq2_gemv_f32_single_call_6912x2560_M%d" % M] = {
            "us": round(ms * 1e3, 2), "GB_s": round(blocks.size / (ms * 1e-3) / 1e9, 1),
            "GFLOP_s": round(2 * M * N * K / (ms * 1e-3) / 1e9, 1)}
    # TQ2_0 6912 x 2560 as a prepared batch of distinct copies past twice the
    # Infinity Cache (one launch each for preparation and product), M = 1, 8,
    # 16: the bandwidth view
    ncopy = max(1, int(np.ceil(2 ** 29 / blocks.size)))
    for M in (1, 8, 16):
        copies = [L.upload_tq2(blocks, N, K, dev) for _ in range(ncopy)]
        x = torch.from_numpy(synth.normal_f32(304 + M, M, K)).to(dev)
        ys = [torch.empty((M, N), dtype=torch.float32, device=dev) for _ in copies]
        plan = L.GemvPlan([(Wc, x, None, yc) for Wc, yc in zip(copies, ys)], M)
        settle(torch, lambda i: plan.run(stream))
        ms = time_events(torch, lambda: plan.run(stream), 20, stream)
        nbytes = ncopy * blocks.size
        out["tq2_plan_%dx6912x2560_M%d" % (ncopy, M)] = {"us": round(ms * 1e3, 2), "GB_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                                                 "frac_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del copies, plan
    # W1A8 decode, hidden 5120, G = 128: QKV, MLP gate, LM head at M = 1 and 8
    K, G = 5120, 128
    for name, N, seed in [("qkv", 7168, 501), ("qkv_card", 8192, 504), ("gate", 17408, 502), ("lm_head", 248320, 503)]:
        bits, sc = w1_weights(L, synth, seed, N, K, G)
        wbytes = bits.nbytes + sc.nbytes
        reps = max(1, int(np.ceil(2 ** 29 / wbytes)))
        Ws = [L.upload_w1(bits, sc, K, G, dev) for _ in range(reps)]
        for M in (1, 8):
            x = torch.from_numpy(synth.normal_f32(510 + M, M, K)).to(dev)
            xq, xsc = L.quantize(x, stream)
            y = torch.empty((M, N), dtype=torch.float32, device=dev)
            ws = torch.zeros((L.ll_gemv_workspace_size(Ws[0], L.LL_ACT_I8, M),), dtype=torch.uint8, device=dev)
            ms = time_graph(torch, lambda i, st: L.ll_bitlinear_gemv(Ws[i], L.LL_ACT_I8, xq, xsc, M, None, y, ws, st),
                            reps, max(2 * reps, 16), stream)
            out["w1a8_gemv_%s_%dx%d_M%d" % (name, N, K, M)] = {
                "us": round(ms * 1e3, 2), "GB_s": round(wbytes / (ms * 1e-3) / 1e9, 1),
                "frac_hbm_peak": round(wbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "weight_bytes": int(wbytes)}
        del Ws
        torch.cuda.empty_cache()
        # context only (the binary-gemm card compares its kernel with a dequantized bf16 matmul): the same
        # shape as a plain bf16 [M, K] x [K, N] product of random bf16 weights on this GPU, torch.mm on
        # contiguous operands, rotated over copies like the W1A8 line
        bbytes = N * K * 2
        breps = max(1, int(np.ceil(2 ** 29 / bbytes)))
        Wb = [torch.randn((K, N), dtype=torch.bfloat16, device=dev) for _ in range(breps)]
        for M in (1, 8):
            xb16 = torch.randn((M, K), dtype=torch.bfloat16, device=dev)
            settle(torch, lambda i: torch.mm(xb16, Wb[i % breps]))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n = max(20, 4 * breps)
            e0.record(stream)
            for i in range(n):
                torch.mm(xb16, Wb[i % breps])
            e1.record(stream)
            e1.synchronize()
            bms = e0.elapsed_time(e1) / n
            w1 = out["w1a8_gemv_%s_%dx%d_M%d" % (name, N, K, M)]["us"]
            out["bf16_mm_context_%s_%dx%d_M%d" % (name, N, K, M)] = {
                "us": round(bms * 1e3, 2), "GB_s": round(bbytes / (bms * 1e-3) / 1e9, 1),
                "w1a8_speedup": round(bms * 1e3 / w1, 2)}
        del Wb
        torch.cuda.empty_cache()
    # W1A8 prepared batches: 12 decoder layers of the same shapes (QKV 7168, O 5120, gate and up 17408 from one
    # activation, down 5120 x 17408; the down projection only where its operand fits, M <= 2), every matrix its
    # own device copy, two launches per step (ll_gemv_plan_init_i8)
    for M in (1, 8):
        shapes = [(7168, K, 0, 501), (K, K, 1, 505), (17408, K, 2, 502), (17408, K, 2, 506)]
        shapes += [(K, 17408, 3, 507)] if M <= 2 else []
        acts, items, wbytes = {}, [], 0
        for layer in range(12):
            for N, Kp, slot, seed in shapes:
                if slot not in acts:
                    acts[slot] = L.quantize(torch.from_numpy(synth.normal_f32(520 + slot, M, Kp)).to(dev), stream)
                bits, sc = w1_weights(L, synth, seed, N, Kp, G)
                items.append((L.upload_w1(bits, sc, Kp, G, dev), acts[slot][0], acts[slot][1], None,
                              torch.empty((M, N), dtype=torch.float32, device=dev)))
                wbytes += bits.nbytes + sc.nbytes
        plan = L.GemvPlanI8(items, M)
        settle(torch, lambda i: plan.run(stream))
        ms = time_events(torch, lambda: plan.run(stream), 20, stream)
        out["w1a8_plan_12_layers_M%d" % M] = {
            "us": round(ms * 1e3, 2), "GB_s": round(wbytes / (ms * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(wbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "weight_bytes": int(wbytes),
            "products": len(items)}
        del plan, items
        torch.cuda.empty_cache()
    # int8 prefill GEMM, M=512 (bf16 activations quantized per token), as graph replays
    for N, K in GEMM_SHAPES:
        W, xb, xq, xsc, y, gws = gemm_operands(L, synth, torch, dev, stream, N, K)
        ms = time_graph(torch, lambda i, st: L.ll_bitlinear_gemm(W, xq, xsc, 512, None, y, None, gws, st), 1, 20, stream)
        msq = time_graph(torch, lambda i, st: L.ll_quantize_act(xb, xq, xsc, st), 1, 20, stream)
        tops = 2 * 512 * N * K / (ms * 1e-3) / 1e12
        out["i2s_gemm_i8_M512_%dx%d" % (N, K)] = {"us": round(ms * 1e3, 2), "TOPS": round(tops, 1),
                                                   "frac_int8_peak": round(tops / INT8_PEAK_TOPS, 4),
                                                   "quantize_us": round(msq * 1e3, 2)}
    # the same product with TQ2_0 weights (fp16 scale per 256-k block, U(0.005, 0.05))
    for N, K in GEMM_SHAPES:
        _, xb, xq, xsc, y, _ = gemm_operands(L, synth, torch, dev, stream, N, K)
        sc = synth.uniform_f16_bits(424, N * K // 256, 0.005, 0.05)
        Wt = L.upload_tq2(L.ll_pack_tq2(synth.ternary(423, N, K), sc), N, K, dev)
        gws = torch.zeros((max(L.ll_gemm_workspace_size(Wt, 512), 16),), dtype=torch.uint8, device=dev)
        ms = time_graph(torch, lambda i, st: L.ll_bitlinear_gemm(Wt, xq, xsc, 512, None, y, None, gws, st), 1, 20, stream)
        tops = 2 * 512 * N * K / (ms * 1e-3) / 1e12
        out["tq2_gemm_i8_M512_%dx%d" % (N, K)] = {"us": round(ms * 1e3, 2), "TOPS": round(tops, 1),
                                                   "frac_int8_peak": round(tops / INT8_PEAK_TOPS, 4)}
    # W1A8 (G = 128) at M = 512 on the int8 matrix cores: the gate and the LM head
    for name, N, seed in [("gate", 17408, 502), ("lm_head", 248320, 503)]:
        K, G = 5120, 128
        bits, sc = w1_weights(L, synth, seed, N, K, G)
        Ww = L.upload_w1(bits, sc, K, G, dev)
        x = torch.from_numpy(synth.normal_f32(520, 512, K)).to(dev)
        xq, xsc = L.quantize(x, stream)
        y = torch.empty((512, N), dtype=torch.float32, device=dev)
        gws = torch.zeros((max(L.ll_gemm_workspace_size(Ww, 512), 16),), dtype=torch.uint8, device=dev)
        ms = time_graph(torch, lambda i, st: L.ll_bitlinear_gemm(Ww, xq, xsc, 512, None, y, None, gws, st), 1, 20, stream)
        tops = 2 * 512 * N * K / (ms * 1e-3) / 1e12
        out["w1a8_gemm_i8_M512_%s_%dx%d" % (name, N, K)] = {"us": round(ms * 1e3, 2), "TOPS": round(tops, 1),
                                                             "frac_int8_peak": round(tops / INT8_PEAK_TOPS, 4)}
        del Ww, y
        torch.cuda.empty_cache()
    # the one-shot bf16 layer (quantize + product + bf16 rounding, three launches)
    N, K = GEMM_SHAPES[0]
    W, xb, _, _, _, _ = gemm_operands(L, synth, torch, dev, stream, N, K)
    yb = torch.empty((512, N), dtype=torch.bfloat16, device=dev)
    lws = torch.zeros((L.ll_binary_linear_workspace_size(W, 512),), dtype=torch.uint8, device=dev)
    ms = time_graph(torch, lambda i, st: L.ll_binary_linear(W, xb, 512, None, yb, lws, st), 1, 20, stream)
    out["i2s_binary_linear_bf16_M512_%dx%d" % (N, K)] = {
        "us": round(ms * 1e3, 2), "TOPS": round(2 * 512 * N * K / (ms * 1e-3) / 1e12, 1)}
    N, K, G = W1_HEAD
    bits, sc = w1_weights(L, synth, 503, N, K, G)
    wbytes = bits.nbytes + sc.nbytes
    reps = max(1, int(np.ceil(2 ** 29 / wbytes)))
    Ws = [L.upload_w1(bits, sc, K, G, dev) for _ in range(reps)]
    xb1 = torch.from_numpy(synth.normal_bf16_bits(512, 1, K).view(np.int16)).to(dev).view(torch.bfloat16)
    yb1 = torch.empty((1, N), dtype=torch.bfloat16, device=dev)
    lws = torch.zeros((L.ll_binary_linear_workspace_size(Ws[0], 1),), dtype=torch.uint8, device=dev)
    ms = time_graph(torch, lambda i, st: L.ll_binary_linear(Ws[i], xb1, 1, None, yb1, lws, st), reps, 2 * reps, stream)
    out["w1a8_binary_linear_bf16_lm_head_%dx%d_M1" % (N, K)] = {
        "us": round(ms * 1e3, 2), "GB_s": round(wbytes / (ms * 1e-3) / 1e9, 1),
        "frac_hbm_peak": round(wbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del Ws
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--gemm-only", action="store_true")
    ap.add_argument("--w1-only", action="store_true")
    args = ap.parse_args()
    if args.copy_probe:
        copy_probe()
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the product shards by output "
              "rows; see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import oracle
    from binary_bit_weight_amd import lowbit as L
    from binary_bit_weight_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    if args.gemm_only:                                   # the GEMM roofline alone (for the profiler)
        print(json.dumps({"roofline_gemm": gemm_roofline(L, synth, torch, dev, stream, args.steps)}), flush=True)
        return
    if args.w1_only:                                     # the W1A8 LM-head line alone (for the profiler)
        print(json.dumps({"roofline_w1a8": w1_roofline(L, synth, torch, dev, stream, args.steps)}), flush=True)
        return
    log("building the decode step")
    packed, items, weight_bytes = build_decode_step(L, synth, torch, dev)
    plan = L.GemvPlan(items, 1)
    log("plan: %d products, %d tiles, %.1f MB of packed weights" % (plan.plan.count, plan.plan.tiles, weight_bytes / 1e6))

    def step():
        plan.prepare(stream)
        plan.product(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # whatever --warmup says, at least 80 ms of continuous steps before the
    # timing: after an idle period the clocks need about 20 ms to settle
    t_settle = time.perf_counter()
    settle(torch, lambda i: step(), 0.08)
    settle_ms = (time.perf_counter() - t_settle) * 1e3
    # the step's two launches captured once in a HIP graph and replayed
    # (reported beside the headline: same kernels, no host launch cost)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.prepare(None)
        plan.product(None)
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    # the headline: the same steps launched one by one on the stream
    t0 = time.perf_counter()
    for i in range(args.steps):
        plan.prepare(stream)
        plan.product(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step_stream = (t1 - t0) * 1e3 / args.steps
    # the product's duration inside steps: the same steps again with
    # per-launch events around the product (kept out of the headline loop:
    # two event records per step add about 5 us to it)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        plan.prepare(stream)
        ev[i][0].record(stream)
        plan.product(stream)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    launch_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    # the product kernel alone: the same number of launches back to back on
    # its stream (activations as last prepared), between two events -- the
    # per-launch events above also hold the wait for each launch to arrive
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record(stream)
    for i in range(args.steps):
        plan.product(stream)
    p1.record(stream)
    p1.synchronize()
    prod_ms = p0.elapsed_time(p1) / args.steps
    # the headline is the plain launch sequence; the graph replay is reported beside it
    ms_per_step_graph, ms_per_step = ms_per_step, ms_per_step_stream
    value = weight_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = weight_bytes / (prod_ms * 1e-3) / 1e9
    log("step %.3f ms (%.1f GB/s; %.3f ms as a graph replay); product kernel %.3f ms (%.1f GB/s); "
        "product launch inside the step %.3f ms" % (ms_per_step, value, ms_per_step_graph, prod_ms, achieved, launch_ms))

    res = {
        "metric": "M=1 effective weight GB/s (% HBM peak); M=512 int8 TOPS (% MFMA peak)",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "i2_s BitLinear decode step, M=1, fp32 x ~ N(0,1): 30 layers x (Q,K,V,O 2560x2560; "
                               "up,gate 6912x2560; down 2560x6912), ternary P(0)=0.4, per-tensor fp32 scale "
                               "~U(0.01,0.1); 210 products as one prepared batch (2 launches)",
                   "M": 1, "layers": LAYERS, "hidden": HIDDEN, "ffn": FFN,
                   "weight_bytes_per_step": int(weight_bytes),
                   "ms_per_step_graph_replay": round(ms_per_step_graph, 4),
                   "independent_products": "the 210 products run as one batch, each on its own activation: a "
                                           "throughput figure for the layer stack's weights; extras."
                                           "i2s_decode_step_dependent runs the layers in order",
                   "warmup_settle_ms": round(settle_ms, 1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": profiled_traffic(),
                     "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "algorithmic_bytes_per_launch": int(weight_bytes),
                     "kernel": KERNEL, "kernel_ms": round(prod_ms, 4), "kernel_ms_in_step": round(launch_ms, 4),
                     "kernel_source_sha256_16": kernel_source_sha()},
    }
    log("int8 GEMM roofline")
    res["roofline_gemm"] = gemm_roofline(L, synth, torch, dev, stream, args.steps)
    if not args.no_cpu:
        log("timing the CPU oracle")
        res["cpu_baseline"] = cpu_baseline(oracle, packed, items)
    log("stream probe")
    sp = stream_probe(L, torch, dev, stream)
    res["roofline"]["stream_probe_GB_s"] = sp["GB_s"]
    res["roofline"]["frac_of_stream_probe"] = round(achieved / sp["GB_s"], 4)
    if not args.no_extras:
        # the W1A8 LM head needs its 179 MB of weights built on the host: with the extras
        log("W1A8 LM head")
        res["roofline_w1a8"] = w1_roofline(L, synth, torch, dev, stream, args.steps)
        log("extras")
        res["extras"] = {"i2s_decode_step_fused_epilogues":
                         fused_decode_step(L, synth, torch, dev, stream, items, weight_bytes, args.steps),
                         "i2s_decode_step_dependent": dependent_decode_step(L, torch, items, weight_bytes, args.steps,
                                                                            stream)}
        res["extras"].update(extras_single(L, synth, torch, dev, stream))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
