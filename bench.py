"""Benchmark: one GPTQ layer (4096x4096, int4, group 128, blocksize 128,
percdamp 0.01) including H accumulation over 128 x 2048 calibration tokens,
on one MI355X.

A step is the whole path on inputs already resident in HBM:
    H = 0;  H += 2 X^T X  (262144 x 4096 fp16 tokens)
    Hinv = upper Cholesky factor of (H + lambda I)^-1
    codes, scales, zeros, losses = column sweep with lazy block updates
The printed JSON line reports ms per layer, the roofline of the dominant
kernel (the fp16 MFMA SYRK of the H accumulation) and the fp64 CPU oracle
timed on a bounded sample on this host.

Other workloads: --layer mlp_up | mlp_down | tiny (one layer each), and
--layer block, the seven layers of a Llama-7B-shaped block (four H's, four
Hinv preparations, seven quantizations in the order q, k, v, o, gate, up,
down); a block step is reported as ms per block.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--layer NAME]
                       [--no-cpu] [--copy-probe-mib M]
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import re
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published peaks (dense)
HBM_PEAK_GBS = 8000.0
FP16_MFMA_TFLOPS = 2500.0
FP32_MFMA_TFLOPS = 157.3
FP64_MFMA_TFLOPS = 78.6

SYRK_SOURCE = os.path.join(ROOT, "post_weight_quantization_02_amd", "csrc", "syrk_f16.hip")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "hessian_accumulate_attn_traffic.md")
LINEAR_SOURCE = os.path.join(ROOT, "post_weight_quantization_02_amd", "csrc", "linear_mfma.hip")
LINEAR_TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "mlp_pair_pipeline_kernels.md")
INFER_SOURCE = os.path.join(ROOT, "post_weight_quantization_02_amd", "csrc", "infer.hip")
# the same SYRK launch (262144 x 11008 fp16 inputs): the mlp_down layer and the pipeline's second H
TRAFFIC_SUMMARY_11008 = os.path.join(ROOT, "profiles", "hessian_accumulate_mlp_down_traffic.md")
DECODE_TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "decode_step_traffic.md")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_work(rows, d, n, B=128, three_step=False):
    """Flops of the method's own work: one triangle of H (with diagonal); for
    Hinv 2d^3/3 (one Cholesky factorization and one triangular inverse), or
    4d^3/3 on the three-step route (two factorizations, the triangular
    inverse and the product L^-T L^-1); the upper-triangular part of the lazy
    update and the in-block rank-1 updates."""
    syrk = float(d) * (d + 1) * n
    prep = (4.0 if three_step else 2.0) * d ** 3 / 3.0
    nb = (d + B - 1) // B
    lazy = 2.0 * rows * B * sum(d - min((b + 1) * B, d) for b in range(nb))
    sweep = 2.0 * rows * (B * (B + 1) / 2.0) * nb
    return dict(syrk=syrk, prep=prep, lazy=lazy, sweep=sweep)


def source_digest(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def recorded_traffic(summary=None, source=None, key="syrk_source_sha256_16"):
    """HBM bytes per call of a kernel from its committed counter summary, or
    None when there is none or the kernel's source has changed since the
    counters were taken (default: the accumulate call's SYRK)."""
    summary = summary or TRAFFIC_SUMMARY
    source = source or SYRK_SOURCE
    try:
        text = open(summary).read()
    except OSError:
        return None
    m_b = re.search(r"^traffic_bytes_per_call:\s*([0-9.eE+]+)\s*$", text, re.M)
    m_h = re.search(r"^" + key + r":\s*([0-9a-f]+)\s*$", text, re.M)
    if not (m_b and m_h) or m_h.group(1) != source_digest(source):
        return None
    return float(m_b.group(1))


def measured_peaks(torch, dev):
    """Attainable rates on this GPU from library kernels: hipBLASLt/rocBLAS
    GEMMs per dtype and a device-to-device copy.  Context for the roofline
    fractions, which use the published peaks."""
    out = {}

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    for name, dt, m in (("f16_gemm_tflops", torch.float16, 8192),
                        ("f32_gemm_tflops", torch.float32, 8192),
                        ("f64_gemm_tflops", torch.float64, 4096)):
        a = torch.randn(m, m, device=dev, dtype=dt)
        b = torch.randn(m, m, device=dev, dtype=dt)
        c = torch.empty(m, m, device=dev, dtype=dt)
        t = timed(lambda: torch.mm(a, b, out=c), 10)
        out[name] = round(2.0 * m ** 3 / t / 1e12, 1)
        del a, b, c
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    t = timed(lambda: dst.copy_(src), 10)
    out["copy_gbs"] = round(2.0 * src.numel() / t / 1e9, 1)
    del src, dst
    torch.cuda.empty_cache()
    return out


def cpu_baseline(layer, X, W, budget_s=8.0, act_order=False):
    """The fp64 oracle, as it is, on a bounded sample of the same layer,
    scaled to one full layer: H on as many 8192-token chunks as fit in about
    budget_s seconds, the full Hinv preparation (with act-order: the order and
    the permuted H first), and the sweep on a doubling number of rows until a
    call takes about budget_s seconds."""
    import numpy as np

    import oracle
    d, rows, n = layer.x.d, layer.w.rows, layer.x.n
    cores = len(os.sched_getaffinity(0))
    # H
    t0 = time.perf_counter()
    Hs = np.zeros((d, d))
    toks = 0
    while toks < n:
        t1 = min(toks + 8192, n)
        Hs += oracle.hessian([X[toks:t1]], d)
        toks = t1
        if time.perf_counter() - t0 >= budget_s:
            break
    t_h = time.perf_counter() - t0
    Hfull = Hs * (n / toks)  # an H of the full layer's scale for timing prep and sweep
    # prep
    t0 = time.perf_counter()
    if act_order:
        perm = oracle.act_order_perm(np.diag(Hfull))
        U, _ = oracle.hinv_upper(Hfull[np.ix_(perm, perm)], layer.percdamp)
        W = W[:, perm]
    else:
        U, _ = oracle.hinv_upper(Hfull, layer.percdamp)
    t_p = time.perf_counter() - t0
    # sweep
    r = min(16, rows)
    while True:
        t0 = time.perf_counter()
        oracle.gptq(W[:r], U, layer.bits, layer.groupsize, layer.blocksize, precision="f32")
        t_s = time.perf_counter() - t0
        if t_s >= budget_s or r >= rows:
            break
        r = min(rows, 2 * r)
    est = t_h * (n / toks) + t_p + t_s * (rows / r)
    return {
        "value": round(est * 1e3, 1), "unit": "ms", "cores": cores, "kind": "oracle",
        "sample": (f"H on {toks} of {n} tokens (x{n / toks:.1f}), full Hinv prep at d={d}, "
                   f"sweep on {r} of {rows} rows (x{rows / r:.1f}); measured s: H {t_h:.2f}, "
                   f"prep {t_p:.2f}, sweep {t_s:.2f}"),
    }


class Job:
    """Device buffers of one workload and its per-step call sequence
    (post_weight_quantization_02_amd.block: one H and one Hinv per
    activation stream, shared by that stream's layers). With several streams
    (the block) and `concurrent`, the streams run in `lanes` lanes of their
    own (quantize_streams_concurrent, a workspace per lane); otherwise in
    order with one workspace of the largest size for every call
    (quantize_streams)."""

    def __init__(self, torch, gq, synth, groups, dev, act_order=False, concurrent=False, lanes=2):
        from post_weight_quantization_02_amd import block
        self.torch, self.gq, self.block = torch, gq, block
        self.act_order = act_order
        self.concurrent = concurrent and len(groups) > 1
        self.groups = []
        self.streams = []
        threads = min(16, len(os.sched_getaffinity(0)))
        for xs, layers in groups:
            log(f"generating X {xs.n}x{xs.d} fp16")
            X = synth.activations(xs, threads=threads)
            Xd = torch.from_numpy(X).to(dev)
            H = torch.empty((xs.d, xs.d), dtype=torch.float32, device=dev)
            U = torch.empty((xs.d, xs.d), dtype=torch.float32, device=dev)
            perm = torch.empty((xs.d,), dtype=torch.int32, device=dev) if act_order else None
            ls = []
            for L in layers:
                W = synth.weights(L.w)
                Wd = torch.from_numpy(W).to(dev)
                outs = block.allocate_outputs(torch, Wd, L.groupsize, act_order)
                ls.append((L, W, Wd, outs))
            self.groups.append((xs, X, Xd, H, U, perm, ls))
            self.streams.append(block.BlockStream(
                X=Xd, H=H, U=U, perm=perm, percdamp=layers[0].percdamp,
                layers=[block.BlockLayer(W=Wd, bits=L.bits, groupsize=L.groupsize,
                                         blocksize=L.blocksize, out=outs)
                        for L, _, Wd, outs in ls]))
        def ws_of(nbytes):
            raw = torch.empty(nbytes + 256, dtype=torch.uint8, device=dev)
            off = (-raw.data_ptr()) % 256
            return raw[off:off + nbytes]

        if self.concurrent:
            # one workspace and one device stream per lane of calibration streams
            self.wss = [ws_of(b) for b in block.lane_workspace_bytes(self.streams, lanes, act_order)]
            self.dstreams = [torch.cuda.Stream(device=dev) for _ in self.wss]
        else:
            self.ws = ws_of(block.workspace_bytes(self.streams, act_order))
        self.ev = {k: [] for k in ("acc", "prep", "quant")}

    def step(self, record):
        torch = self.torch
        local = threading.local()

        def mark(phase, begin):
            # events on the calling thread's current stream (its calibration
            # stream's device stream in the concurrent block)
            e = torch.cuda.Event(enable_timing=True)
            e.record(torch.cuda.current_stream())
            if not hasattr(local, "open"):
                local.open = {}
            if begin:
                local.open[phase] = e
            else:
                self.ev[phase].append((local.open.pop(phase), e))

        if self.concurrent:
            self.block.quantize_streams_concurrent(self.streams, self.wss, self.act_order,
                                                   device_streams=self.dstreams,
                                                   mark=mark if record else None)
        else:
            self.block.quantize_streams(self.streams, self.ws, self.act_order,
                                        mark=mark if record else None)


DECODE_SHAPES = (("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
                 ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008))
# q|k|v and gate|up stored as one matrix each (the same bytes in 4 products)
DECODE_SHAPES_FUSED = (("qkv", 12288, 4096), ("o", 4096, 4096), ("gate_up", 22016, 4096),
                       ("down", 4096, 11008))
DECODE_BLOCKS = 32


def decode_cpu_baseline(m, bits, g, budget_s=10.0):
    """The oracle's dequantizing product (unpack, dequantize, multiply in
    fp64) on one matrix of each decode shape, scaled to the 224 calls of a
    step."""
    import numpy as np

    import oracle
    rng = np.random.default_rng(0)
    cores = len(os.sched_getaffinity(0))
    total, parts = 0.0, []
    for shape in ({s[1:] for s in DECODE_SHAPES}):
        rows, cols = shape
        count = sum(1 for s in DECODE_SHAPES if s[1:] == shape) * DECODE_BLOCKS
        codes = rng.integers(0, 1 << bits, size=(rows, cols))
        packed = oracle.pack_codes(codes, bits)
        ng = -(-cols // g)
        sc = rng.uniform(1e-3, 2e-3, (rows, ng))
        zr = rng.integers(0, 1 << bits, (rows, ng)).astype(np.float64)
        x = rng.standard_normal((m, cols)).astype(np.float16)
        t0 = time.perf_counter()
        oracle.dequant_matmul(x, packed, bits, cols, sc, zr, g)
        dt = time.perf_counter() - t0
        total += dt * count
        parts.append(f"{rows}x{cols}: {dt:.2f} s x {count}")
    return {"value": round(total * 1e3, 1), "unit": "ms", "cores": cores, "kind": "oracle",
            "sample": "one call per distinct shape (" + "; ".join(parts) + "), scaled by the "
                      "number of calls of that shape in a step"}


def decode_main(args):
    """One decode step of W4A16 products over 32 Llama-7B-shaped blocks."""
    import numpy as np
    import torch

    import post_weight_quantization_02_amd as gq

    dev = torch.device("cuda:0")
    copy_probe(torch, dev, args.copy_probe_mib)
    m, bits, g = args.tokens, 4, 128
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    log(f"generating {DECODE_BLOCKS} blocks of packed int{bits} g{g} weights on the device")
    shapes = DECODE_SHAPES_FUSED if args.fused else DECODE_SHAPES
    mats = []
    alg_bytes = 0
    for b in range(DECODE_BLOCKS):
        for name, rows, cols in shapes:
            nw = gq.packed_words(cols, bits)
            ng = -(-cols // g)
            packed = torch.randint(-2 ** 31, 2 ** 31 - 1, (rows, nw), dtype=torch.int32,
                                   device=dev, generator=gen)
            sc = torch.rand((rows, ng), device=dev, generator=gen) * 1e-3 + 1e-3
            zr = torch.randint(0, 1 << bits, (rows, ng), device=dev, generator=gen).float()
            mats.append((name, rows, cols, packed, sc, zr))
            alg_bytes += rows * nw * 4 + 2 * rows * ng * 4 + m * cols * 2 + m * rows * 4
    xs = {c: torch.randn((m, c), device=dev, generator=gen).half() for c in (4096, 11008)}
    ys = {r: torch.empty((m, r), dtype=torch.float32, device=dev)
          for r in {rows for _, rows, _ in shapes}}
    stream = torch.cuda.current_stream(dev)

    def step(events=None):
        for i, (name, rows, cols, packed, sc, zr) in enumerate(mats):
            if events is not None:
                events[i][0].record(stream)
            gq.dequant_gemm(xs[cols], packed, bits, cols, sc, zr, g, out=ys[rows])
            if events is not None:
                events[i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # The 224 launches of a step are replayed from a HIP graph: launched one by
    # one from Python, the host's per-call cost (about 9 us) exceeds a
    # launch's GPU time and the GPU would wait for the host.
    graph = None
    if not args.no_graph:
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()  # warm-up on the capture stream
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
    run = graph.replay if graph is not None else step
    for _ in range(2):
        run()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    ev_ms_step = e0.elapsed_time(e1) / args.steps
    # per-launch durations (a separate eager pass with events around every call)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in mats]
    step(ev)
    torch.cuda.synchronize()
    launch_ms = [a.elapsed_time(b) for a, b in ev]
    kernel_ms = float(np.sum(launch_ms))
    # roofline: the step's algorithmic bytes over its event-timed duration
    # (every launch of the step, gaps between launches included)
    achieved = alg_bytes / (ev_ms_step * 1e-3) / 1e9
    per_shape = {}
    for (name, rows, cols, *_), t in zip(mats, launch_ms):
        per_shape.setdefault(f"{rows}x{cols}", []).append(t)
    cpu = None if args.no_cpu else decode_cpu_baseline(m, bits, g)
    line = {
        "metric": f"ms per decode step ({DECODE_BLOCKS} Llama-7B-shaped blocks, int{bits} g{g} "
                  f"W{bits}A16 products{', fused qkv and gate_up' if args.fused else ''}, "
                  f"{m} token{'s' if m > 1 else ''})",
        "value": round(ms_step, 4),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 codes, f32 dequant and accumulate, f16 activations",
        "data": "synthetic (seeded random codes, scales and zeros generated on the device; "
                "random fp16 activations)",
        "config": {"workload": f"decode: {DECODE_BLOCKS} x (q,k,v,o 4096x4096; gate,up "
                               f"11008x4096; down 4096x11008)"
                               + (", q|k|v and gate|up stored fused" if args.fused else "")
                               + f", {len(mats)} products per step, {m} token(s)",
                   "algorithmic_bytes_per_step": alg_bytes,
                   "graph_replay": graph is not None,
                   "event_ms_per_step": round(ev_ms_step, 4),
                   "eager_launch_us_by_shape": {k: round(1e3 * float(np.mean(v)), 2)
                                                for k, v in per_shape.items()},
                   "eager_ms_per_step": round(kernel_ms, 4)},
        "roofline": {"bound": "hbm",
                     "kernel": "dequant_gemv_fast_kernel (the %d launches of a step, gaps "
                               "included)" % len(mats),
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": (recorded_traffic(DECODE_TRAFFIC_SUMMARY, INFER_SOURCE,
                                                  "infer_source_sha256_16")
                                 if m == 1 and not args.fused else None),
                     "bytes_per_step": alg_bytes},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def copy_probe(torch, dev, mib):
    """One plain device copy of known size: the reference the HBM counters
    (FETCH_SIZE, WRITE_SIZE) are scaled by."""
    if not mib:
        return
    nb = mib << 20
    src = torch.ones(nb // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy probe: {nb} bytes read, {nb} bytes written")
    del src, dst


def pipeline_cpu_baseline(x, W1, W2, bits=4, budget_s=4.0):
    """The fp64 oracle's layer-by-layer block on a bounded sample, each phase
    timed on a slice and scaled to the full block: H1 and H2 on 4096-token
    chunks until about budget_s, the two Hinv preparations at full size
    (d = 4096) and at half size scaled by 8 (d = 11008, cubic), the two sweeps
    on 512 rows, the forward product on 2048 tokens."""
    import numpy as np

    import oracle
    from oracle.pipeline64 import relu_to_f16
    n, d = x.shape
    m, dout = W1.shape[0], W2.shape[0]
    cores = len(os.sched_getaffinity(0))

    def hess(X, dd):
        t0, toks, H = time.perf_counter(), 0, np.zeros((dd, dd))
        while toks < X.shape[0] and time.perf_counter() - t0 < budget_s:
            H += oracle.hessian([X[toks:toks + 4096]], dd)
            toks = min(toks + 4096, X.shape[0])
        return (time.perf_counter() - t0) * X.shape[0] / toks, H * (X.shape[0] / toks), toks

    t_h1, H1, tok1 = hess(x, d)
    t0 = time.perf_counter()
    U1, _ = oracle.hinv_upper(H1, 0.01)
    t_p1 = time.perf_counter() - t0
    r1 = min(512, m)
    t0 = time.perf_counter()
    q1 = oracle.gptq(W1[:r1], U1, bits, 128, 128, precision="f32")
    t_s1 = (time.perf_counter() - t0) * m / r1
    nf = min(2048, n)
    t0 = time.perf_counter()
    y = relu_to_f16(oracle.quantized_layer_output(x[:nf], q1["codes"], q1["scales"], q1["zeros"],
                                                  128))
    t_f = (time.perf_counter() - t0) * (n / nf) * (m / r1)
    y1 = np.tile(y, (1, -(-m // r1)))[:, :m]  # inputs of the right shape for timing H2
    t0, toks, H2 = time.perf_counter(), 0, np.zeros((m, m))
    while toks < nf and time.perf_counter() - t0 < budget_s:
        H2 += oracle.hessian([y1[toks:toks + 1024]], m)
        toks += 1024
    t_h2 = (time.perf_counter() - t0) * n / toks
    h = m // 2
    Hh = H2[:h, :h] + np.eye(h) * np.mean(np.diag(H2))
    t0 = time.perf_counter()
    U2h, _ = oracle.hinv_upper(Hh, 0.01)
    t_p2 = (time.perf_counter() - t0) * (m / h) ** 3
    r2 = min(256, dout)
    U2 = np.kron(np.eye(2), U2h)  # a 2h x 2h factor: the sweep's cost does not depend on values
    t0 = time.perf_counter()
    oracle.gptq(W2[:r2, :U2.shape[0]], U2, bits, 128, 128, precision="f32")
    t_s2 = (time.perf_counter() - t0) * dout / r2
    est = t_h1 + t_p1 + t_s1 + t_f + t_h2 + t_p2 + t_s2
    return {
        "value": round(est * 1e3, 1), "unit": "ms", "cores": cores, "kind": "oracle",
        "sample": (f"H1 on {tok1} of {n} tokens, prep at d={d}, sweep 1 on {r1} of {m} rows, "
                   f"forward on {nf} tokens x {r1} outputs, H2 on {toks} tokens, prep at "
                   f"d={h} (x{(m / h) ** 3:.0f}), sweep 2 on {r2} of {dout} rows; each scaled "
                   f"to the full block; s: H1 {t_h1:.1f}, prep1 {t_p1:.1f}, sweep1 {t_s1:.1f}, "
                   f"forward {t_f:.1f}, H2 {t_h2:.1f}, prep2 {t_p2:.1f}, sweep2 {t_s2:.1f}"),
    }


def pipeline_main(args):
    """Layer-by-layer quantization of the Llama-7B-shaped MLP up -> ReLU ->
    down pair: the down projection's H is recorded from the quantized up
    projection's outputs."""
    import contextlib

    import numpy as np
    import torch

    import post_weight_quantization_02_amd as gq
    import synth

    dev = torch.device("cuda:0")
    copy_probe(torch, dev, args.copy_probe_mib)
    up = [L for L in synth.BLOCK if L.name == "up"][0]
    down = [L for L in synth.BLOCK if L.name == "down"][0]
    n, d, m, dout = up.x.n, up.x.d, up.w.rows, down.w.rows
    bits = 4 if args.bits is None else args.bits
    log(f"generating x {n}x{d} fp16, W_up {m}x{d}, W_down {dout}x{m}")
    x = synth.activations(up.x, threads=min(16, len(os.sched_getaffinity(0))))
    W1, W2 = synth.weights(up.w), synth.weights(down.w)
    xd, W1d, W2d = (torch.from_numpy(a).to(dev) for a in (x, W1, W2))
    stream = torch.cuda.current_stream(dev)
    ev = {}

    def timer(name):
        @contextlib.contextmanager
        def cm():
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            yield
            b.record(stream)
            ev.setdefault(name, []).append((a, b))
        return cm()

    for _ in range(args.warmup):
        out = gq.quantize_relu_block(xd, W1d, W2d, bits=bits)
        del out
    torch.cuda.synchronize()
    ev.clear()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        out = gq.quantize_relu_block(xd, W1d, W2d, bits=bits, timer=timer)
        del out
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    ph = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in ev.items()}
    log("phase ms:", {k: round(v, 3) for k, v in ph.items()})
    w1 = algorithmic_work(m, d, n)
    w2 = algorithmic_work(dout, m, n)
    fwd_flops = 2.0 * n * d * m
    work = w1["syrk"] + w1["prep"] + w1["lazy"] + w1["sweep"] + fwd_flops + \
        w2["syrk"] + w2["prep"] + w2["lazy"] + w2["sweep"]
    # roofline of the dominant single kernel: the larger of the forward product
    # (one launch) and the second H accumulation (one SYRK call)
    cand = {"forward1": ("linear_kernel<%d, true> (the up projection's forward product)" % bits,
                         fwd_flops),
            "acc2": ("hessian accumulate call at d=%d: syrk_fast_kernel + syrk_reduce_kernel" % m,
                     w2["syrk"])}
    dom = max(cand, key=lambda k: ph[k])
    rf = {}
    for k, (name, flops) in cand.items():
        ach = flops / (ph[k] * 1e-3) / 1e12
        if k == "forward1":
            tr = recorded_traffic(LINEAR_TRAFFIC_SUMMARY, LINEAR_SOURCE, "linear_source_sha256_16")
        else:
            tr = recorded_traffic(TRAFFIC_SUMMARY_11008) if m == 11008 else None
        rf[k] = {"bound": "mfma", "kernel": name, "achieved": round(ach, 2),
                 "peak": FP16_MFMA_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(ach / FP16_MFMA_TFLOPS, 4), "traffic": tr,
                 "per_launch_ms": round(ph[k], 4), "flops_per_launch": flops}
    cpu = None
    if not args.no_cpu:
        log("cpu baseline (oracle on a bounded sample)")
        cpu = pipeline_cpu_baseline(x, W1, W2, bits)
        log("  ", cpu)
    line = {
        "metric": "ms per layer-by-layer quantized MLP pair (up 11008x4096 -> ReLU -> down "
                  f"4096x11008, int{bits} g128; down's H from the quantized up's outputs)",
        "value": round(ms_step, 4),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16-in/f32-acc SYRK and forward product, f64 Hinv, f32 sweep",
        "data": "synthetic (seeded low-rank-plus-noise activations, Gaussian weights)",
        "config": {"workload": f"MLP pair: x {n}x{d} fp16 (128x2048 tokens), W_up {m}x{d} fp16, "
                               f"W_down {dout}x{m} fp16, int{bits} g128 B128 percdamp 0.01; "
                               "y1 = fp16(relu(x W_up_hat^T)) recorded for the down projection",
                   "phase_ms": {k: round(v, 4) for k, v in ph.items()},
                   "effective_tflops": round(work / (ms_step * 1e-3) / 1e12, 2),
                   "roofline_other": rf["acc2" if dom == "forward1" else "forward1"]},
        "roofline": rf[dom],
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layer", default="attn",
                    choices=["attn", "mlp_up", "mlp_down", "tiny", "block"])
    ap.add_argument("--act-order", action="store_true",
                    help="process columns in decreasing order of diag(H) (desc_act)")
    ap.add_argument("--groupsize", type=int, default=None,
                    help="override the layer's group size (0: one group per row, per-channel)")
    ap.add_argument("--bits", type=int, default=None, help="override the layer's bit width")
    ap.add_argument("--lanes", type=int, default=2,
                    help="block: calibration streams run in this many concurrent lanes")
    ap.add_argument("--serial", action="store_true",
                    help="block: quantize the calibration streams one after another on one "
                         "stream (default: each on a stream and host thread of its own)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--no-peaks", action="store_true", help="skip the library peak probes")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one device copy of this size first (counter calibration)")
    ap.add_argument("--decode", action="store_true",
                    help="time one decode step of packed int4 products instead of quantization")
    ap.add_argument("--tokens", type=int, default=1, help="tokens per decode step (--decode)")
    ap.add_argument("--fused", action="store_true",
                    help="--decode: q|k|v and gate|up stored as one matrix each")
    ap.add_argument("--pipeline", action="store_true",
                    help="layer-by-layer quantization of the MLP up -> ReLU -> down pair")
    ap.add_argument("--three-step", action="store_true",
                    help="form Hinv by the pages' three steps (Cholesky, inverse through the "
                         "factor, upper Cholesky of the inverse) instead of one factorization "
                         "of the reversed H_d")
    ap.add_argument("--no-other-route", action="store_true",
                    help="skip timing the other Hinv route after the timed steps (kernel traces)")
    ap.add_argument("--no-graph", action="store_true",
                    help="--decode: launch the step's products one by one instead of a graph")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); how this path "
              "shards over several GPUs is a design note, not a measured run.", file=sys.stderr)
        sys.exit(2)

    if args.decode:
        decode_main(args)
        return
    if args.pipeline:
        pipeline_main(args)
        return

    import numpy as np
    import torch

    import post_weight_quantization_02_amd as gq
    import synth

    dev = torch.device("cuda:0")
    copy_probe(torch, dev, args.copy_probe_mib)

    if args.layer == "block":
        groups = []
        for L in synth.BLOCK:
            if groups and groups[-1][0] == L.x:
                groups[-1][1].append(L)
            else:
                groups.append((L.x, [L]))
        layers = synth.BLOCK
        workload = ("Llama-7B-shaped block: q,k,v,o 4096x4096, gate,up 11008x4096, down "
                    "4096x11008 fp16; 4 H's (attn-in, o-in, mlp-in 262144x4096, down-in "
                    "262144x11008 fp16, 128x2048 tokens each); int4 g128 B128 percdamp 0.01; "
                    "layers in order q,k,v,o,gate,up,down")
        metric = "ms per Llama-7B-shaped block (7 layers, 4 H's incl. accumulate)"
    else:
        L = synth.LAYERS[args.layer]
        if args.groupsize is not None or args.bits is not None:
            g = L.groupsize if args.groupsize is None else args.groupsize
            L = dataclasses.replace(L, groupsize=(L.w.cols if g <= 0 else g),
                                    bits=L.bits if args.bits is None else args.bits)
        groups = [(L.x, [L])]
        layers = [L]
        rows, d, n = L.w.rows, L.x.d, L.x.n
        extra = ""
        if L.x.zero_frac:
            extra = f", {int(L.x.zero_frac * 100)}% zeros, {L.x.dead} dead channels"
        workload = (f"{L.name}: W {rows}x{d} {L.w.dtype}, X {n}x{d} fp16{extra}, "
                    f"int{L.bits} g{L.groupsize} B{L.blocksize} percdamp {L.percdamp}")
        metric = "ms per 4096x4096 int4 g128 GPTQ layer (incl. H accumulate); % MFMA roofline"
        if args.layer != "attn" or args.groupsize is not None or args.bits is not None:
            metric = f"ms per {rows}x{d} int{L.bits} g{L.groupsize} GPTQ layer (incl. H accumulate)"
    if args.three_step:
        if args.act_order:
            print("--three-step has no act-order variant", file=sys.stderr)
            sys.exit(2)
        workload += "; Hinv by the three-step route"
    if args.act_order:
        workload += "; act-order (columns in decreasing order of diag(H), groups in that order)"
        metric = metric.replace(" GPTQ layer", " GPTQ layer with act-order").replace(
            " GPTQ layers", " GPTQ layers with act-order")
        if args.layer == "block":
            metric = metric.replace("block (", "block with act-order (")

    job = Job(torch, gq, synth, groups, dev, act_order=args.act_order,
              concurrent=not args.serial, lanes=args.lanes)
    for st in job.streams:
        st.three_step = args.three_step
    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        job.step(False)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        job.step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    per = {k: [a.elapsed_time(b) for a, b in v] for k, v in job.ev.items()}
    ph = {k: float(np.sum(v)) / args.steps for k, v in per.items()}  # ms per step per phase
    log("phase ms per step:", {k: round(v, 3) for k, v in ph.items()})
    if len(job.groups) == 1:
        log("ms per timed step (phase sum):",
            [round(sum(per[k][i] for k in per), 3) for i in range(args.steps)])
    # The other Hinv route on the same H, after the timed steps: the three-step
    # preparation when the step used one factorization, and the other way
    # round (event-timed, median of 3; not part of the step).
    prep_other = None
    if not args.act_order and not args.no_other_route and len(job.groups) == 1:
        st = job.streams[0]
        fn = gq.prepare_hinv if args.three_step else gq.prepare_hinv_three_step
        ts = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn(st.H, st.percdamp, out=st.U, workspace=job.ws)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        prep_other = {"route": "one factorization of the reversed H_d" if args.three_step
                      else "three steps (Cholesky, inverse through the factor, re-factorization)",
                      "ms": round(sorted(ts)[1], 4)}
        log("other Hinv route:", prep_other)
    # library peaks after the timed steps, so their full-power GEMMs do not
    # precede the measurement
    peaks = None if args.no_peaks else measured_peaks(torch, dev)
    if peaks:
        log("measured peaks:", peaks)

    # algorithmic work per step
    work = dict(syrk=0.0, prep=0.0, lazy=0.0, sweep=0.0)
    for xs, X, Xd, H, U, _, ls in job.groups:
        w0 = algorithmic_work(0, xs.d, xs.n, three_step=args.three_step)
        work["syrk"] += w0["syrk"]
        work["prep"] += w0["prep"]
        for Lq, *_ in ls:
            w1 = algorithmic_work(Lq.w.rows, xs.d, 0, Lq.blocksize)
            work["lazy"] += w1["lazy"]
            work["sweep"] += w1["sweep"]
    floor = {"acc": work["syrk"] / FP16_MFMA_TFLOPS / 1e9,
             "prep": work["prep"] / FP64_MFMA_TFLOPS / 1e9,
             "quant": work["lazy"] / FP32_MFMA_TFLOPS / 1e9}
    floor_ms = sum(floor.values())
    eff_tflops = sum(work.values()) / (ms_step * 1e-3) / 1e12

    # dominant kernel: the SYRK of the H accumulation (one call per H)
    acc_calls = per["acc"]
    acc_ms = float(np.mean(acc_calls))
    syrk_flops_call = work["syrk"] / len(job.groups)
    syrk_tflops = syrk_flops_call / (acc_ms * 1e-3) / 1e12
    traffic = None
    if args.layer == "attn" and not args.act_order:
        traffic = recorded_traffic()
    elif args.layer == "mlp_down" and not args.act_order:
        traffic = recorded_traffic(TRAFFIC_SUMMARY_11008)

    cpu = None
    if not args.no_cpu and args.layer != "block":
        log("cpu baseline (oracle on a bounded sample)")
        xs, X, *_ = job.groups[0]
        cpu = cpu_baseline(layers[0], X, job.groups[0][6][0][1], act_order=args.act_order)
        log("  ", cpu)

    line = {
        "metric": metric,
        "value": round(ms_step, 4),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16-in/f32-acc SYRK, f64 Hinv, f32 sweep",
        "data": "synthetic (seeded low-rank-plus-noise activations, Gaussian weights)",
        "config": {"workload": workload,
                   "phase_ms": {k: round(v, 4) for k, v in ph.items()},
                   "prep_route": ("three steps (Cholesky, inverse through the factor, "
                                  "re-factorization; gptq_prepare_hinv_three_step)"
                                  if args.three_step else
                                  "one factorization of the reversed H_d and one triangular "
                                  "inverse (gptq_prepare_hinv)"),
                   "prep_other_route": prep_other,
                   "phase_floor_ms": {k: round(v, 4) for k, v in floor.items()},
                   "phase_frac_of_floor": {k: round(floor[k] / ph[k], 4) for k in floor},
                   "effective_tflops": round(eff_tflops, 2),
                   "roofline_floor_ms": round(floor_ms, 3),
                   "frac_of_floor": round(floor_ms / ms_step, 4),
                   "streams": (f"concurrent: calibration streams in {len(job.wss)} lanes, each "
                               "lane on a device stream and host thread of its own; the phases "
                               "of different lanes overlap, so phase_ms (summed over streams) "
                               "exceeds ms_per_step and the accumulate calls in the roofline "
                               "share the GPU" if job.concurrent else "serial"),
                   "peaks_measured": peaks},
        "roofline": {"bound": "mfma",
                     "kernel": "hessian accumulate call: syrk_fast_kernel + syrk_reduce_kernel",
                     "achieved": round(syrk_tflops, 2), "peak": FP16_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(syrk_tflops / FP16_MFMA_TFLOPS, 4),
                     "traffic": traffic,
                     "per_launch_ms": round(acc_ms, 4),
                     "flops_per_launch": syrk_flops_call},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
