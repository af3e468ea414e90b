"""Benchmark of the KDA chunked forward (one libkda kda_chunk_fwd call = one step of
the whole hot path: gate, WY stage, state passing, output) on one MI355X.

Default workload: B=4, H=32, T=16384, K=V=128, chunk 64, bf16 activations, fp32
state, synthetic seeded inputs resident in HBM before the timed region.
Prints one JSON line: head-tokens/s (B*H*T per second), the roofline of the fused
kernel (algorithmic HBM bytes per launch / measured launch time vs 8 TB/s) and the
f64 CPU oracle timed on a bounded sample of the same workload.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from concurrent.futures import ProcessPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
METRIC = "KDA chunked-forward tokens/s (B·H·T/s) + % of roofline, H=32,K=V=128,T=16k"
METRIC_SCALAR = "KDA chunked-forward tokens/s, scalar-decay gate (kda_chunk_fwd_scalar), H=32,K=V=128,T=16k"
METRIC_NORM = "KDA chunked-forward tokens/s with the output RMSNorm fused (kda_chunk_fwd_norm), H=32,K=V=128,T=16k"


def algorithmic_bytes(wl, scalar_gate=False) -> int:
    """HBM bytes one kda_chunk_fwd call must move at minimum: read q, k, z, v, beta
    and the initial state once, write o and the final state once (A_log, dt_bias
    are negligible but counted).  With the scalar-decay gate, z is one value per
    head-token and dt_bias one per head."""
    es = 2 if wl.dtype == "bf16" else 4
    ht = wl.B * wl.H * wl.T
    zc = 1 if scalar_gate else wl.K
    acts = ht * (2 * wl.K + zc + wl.V + 1) * es + ht * wl.V * es
    state = 2 * wl.B * wl.H * wl.K * wl.V * 4
    params = wl.H * 4 + wl.H * zc * 4
    return acts + state + params


KERNEL_SOURCES = ("kda_chunk_fwd_pc.h", "kda_common.h")
KERNEL_NAME = "kda::chunk_fwd_pc_kernel<128,64,32,false,false>"


def kernel_label(wl, scalar_gate=False, paired=False, norm=False) -> str:
    """The forward instance a kda_chunk_fwd call of this workload launches (the tiling rules
    of the library's forward plan)."""
    C = min(wl.chunk, 32)
    if norm:
        return "kda::chunk_fwd_pc_kernel<%d,64,32,false,true>" % max(32, wl.K)
    if paired:
        return "kda::chunk_fwd_px_kernel<%d,%s>" % (max(32, wl.K), str(scalar_gate).lower())
    if wl.dtype == "bf16":
        return "kda::chunk_fwd_pc_kernel<%d,%d,%d,%s,false>" % (max(32, wl.K), min(64, max(16, wl.V)), C,
                                                               str(scalar_gate).lower())
    KD = max(16, wl.K)
    VT = min(16 if KD >= 64 else 64, max(16, wl.V))
    return "kda::chunk_fwd_kernel<float,%d,%d,%d>" % (KD, VT, wl.chunk if KD < 128 else C)


def kernel_source_hash() -> str:
    """sha256 over the sources of the fused bf16 forward kernel: counter-measured traffic
    is only reported while the kernel it was measured on is unchanged."""
    import hashlib
    hs = hashlib.sha256()
    for name in KERNEL_SOURCES:
        hs.update(open(os.path.join(ROOT, "gated_delta_rule_47_amd", "csrc", name), "rb").read())
    return hs.hexdigest()


def _oracle_head(args):
    """CPU baseline worker: the f64 oracle's token recurrence on one head."""
    wl_name, b, h, scalar_gate = args
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    import kda_synth as ks
    from oracle import kda_ref as R
    wl = ks.WORKLOADS[wl_name]
    A_log, dt_bias = ks.head_params(wl)
    sl = ks.head_slice(wl, b, h)
    t0 = time.time()
    if scalar_gate:
        g, _ = R.gate_scalar(sl["z"][None, None, :, 0], A_log[h:h + 1], dt_bias[h:h + 1, 0])
        R.recurrent_scalar(sl["q"][None, None], sl["k"][None, None], sl["v"][None, None], g, sl["beta"][None, None],
                           sl["state_in"][None, None])
    else:
        g, _ = R.gate(sl["z"][None, None], A_log[h:h + 1], dt_bias[h:h + 1])
        R.recurrent(sl["q"][None, None], sl["k"][None, None], sl["v"][None, None], g, sl["beta"][None, None],
                    sl["state_in"][None, None])
    return t0, time.time()


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def block_tokens(wl) -> int:
    """Tokens per block the forward kernel runs for this workload: the library serves a
    chunk above 32 with 32-token blocks for bf16, and for fp32 at K = 128 (the same
    function; the block is an internal tiling)."""
    return min(wl.chunk, 32) if (wl.dtype == "bf16" or wl.K == 128) else wl.chunk


def copy_bandwidth_gbs(torch, mib: int = 1024, launches: int = 10) -> float:
    """Device-to-device copy bandwidth (read + write bytes per second), the practical
    ceiling an HBM-bound kernel is compared with besides the 8 TB/s peak."""
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(launches):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    secs = a.elapsed_time(b) * 1e-3 / launches
    del src, dst
    return 2 * n / secs / 1e9


def cpu_baseline(wl, n_heads: int, workers: int, scalar_gate: bool = False) -> dict:
    """The f64 oracle (gate + token recurrence) on n_heads whole heads, one per task of a pool
    of `workers` processes:
    head-tokens per second of wall time from the first head's start to the last head's
    end (input generation excluded)."""
    heads = [(i // wl.H % wl.B, i % wl.H) for i in range(n_heads)]
    with ProcessPoolExecutor(workers) as ex:
        spans = list(ex.map(_oracle_head, [(wl.name, b, h, scalar_gate) for b, h in heads]))
    wall = max(e for _, e in spans) - min(s for s, _ in spans)
    cpu = sum(e - s for s, e in spans)
    return {"value": n_heads * wl.T / wall, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cores": os.cpu_count(),
            "sample": "%d of %d heads at full T=%d (f64 numpy token recurrence, one head per task on %d worker "
                      "processes; %.1f s wall, %.1f s of CPU work)" % (n_heads, wl.B * wl.H, wl.T, workers, wall, cpu)}


def _pmc_per_dispatch(directory: str, counter: str, kernel_match: str) -> list:
    """Per-dispatch sums of one rocprofv3 --pmc counter (CSV output) for matching kernels."""
    import collections
    import csv
    rows = csv.DictReader(open(os.path.join(directory, "run_counter_collection.csv")))
    agg = collections.defaultdict(float)
    for r in rows:
        if r["Counter_Name"] == counter and kernel_match in r["Kernel_Name"]:
            agg[r["Dispatch_Id"]] += float(r["Counter_Value"])
    return list(agg.values())


def traffic_from_pmc(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_mib, workload, out_path):
    """HBM bytes per launch of the fused forward from two counter runs (FETCH_SIZE, then
    WRITE_SIZE, KiB per dispatch), each calibrated by the same counter on a plain device
    copy of known size: factor = counter KiB * 1024 / copied bytes."""
    f = _pmc_per_dispatch(fetch_dir, "FETCH_SIZE", "chunk_fwd_pc")
    w = _pmc_per_dispatch(write_dir, "WRITE_SIZE", "chunk_fwd_pc")
    cf = _pmc_per_dispatch(copy_fetch_dir, "FETCH_SIZE", "copyBuffer")
    cw = _pmc_per_dispatch(copy_write_dir, "WRITE_SIZE", "copyBuffer")
    if not (f and w and cf and cw):
        raise SystemExit("missing dispatches in the counter files")
    nbytes = copy_mib * (1 << 20)
    mean = lambda x: sum(x) / len(x)
    ff, wf = mean(cf) * 1024 / nbytes, mean(cw) * 1024 / nbytes
    fb, wb = mean(f) * 1024 / ff, mean(w) * 1024 / wf
    out = {"workload": workload, "kernel": KERNEL_NAME, "kernel_source_sha256": kernel_source_hash(),
           "fetch_size_kib_per_dispatch": mean(f), "write_size_kib_per_dispatch": mean(w),
           "copy_calibration": {"bytes": nbytes, "fetch_size_kib": mean(cf), "write_size_kib": mean(cw),
                                "fetch_factor": ff, "write_factor": wf},
           "fetch_bytes_per_launch": int(fb), "write_bytes_per_launch": int(wb), "bytes_per_launch": int(fb + wb)}
    json.dump(out, open(out_path, "w"), indent=1)
    print(json.dumps(out, indent=1))


def decode_bench(B, steps, warmup, H=32, K=128, V=128):
    """Decode step at one token per sequence: the state (B,H,K,V) fp32 is read and written
    once, so the bound is HBM at 2*K*V*4 bytes per head plus the token's activations.
    Prints one JSON line (not the headline metric)."""
    import torch
    import gated_delta_rule_47_amd as kda
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(7)
    act = lambda *s: (torch.randn(*s, device=dev, generator=g) * 0.1).to(torch.bfloat16)
    q, k, z, v = act(B, H, K), act(B, H, K), act(B, H, K), act(B, H, V)
    beta = torch.rand(B, H, device=dev, generator=g).to(torch.bfloat16)
    A_log = torch.zeros(H, device=dev)
    dt_bias = torch.zeros(H, K, device=dev)
    S = torch.randn(B, H, K, V, device=dev, generator=g) * 0.1
    o = torch.empty(B, H, V, dtype=torch.bfloat16, device=dev)
    for _ in range(warmup):
        kda.recurrent_step(q, k, v, z, A_log, dt_bias, beta, S, out=o)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        kda.recurrent_step(q, k, v, z, A_log, dt_bias, beta, S, out=o)
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / steps
    # The same steps replayed from a HIP graph of 50 consecutive steps (no host launch per
    # step): what a serving loop that captures its decode steps sees.
    ng = 50
    step = lambda: kda.recurrent_step(q, k, v, z, A_log, dt_bias, beta, S, out=o)
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(ng):
            step()
    graph.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // ng)
    a.record(stream)
    for _ in range(reps):
        graph.replay()
    b.record(stream)
    torch.cuda.synchronize()
    us_graph = a.elapsed_time(b) * 1e3 / (reps * ng)
    nbytes = B * H * (2 * K * V * 4 + (3 * K + 2 * V + 1) * 2)
    print(json.dumps({"metric": "decode step state bandwidth (kda_recurrent_step)", "value": round(nbytes / us / 1e3, 1),
                      "unit": "GB/s", "frac_of_8TBps": round(nbytes / us / 1e3 / 8000.0, 4), "us_per_step": round(us, 2),
                      "graph_us_per_step": round(us_graph, 2),
                      "graph_GBps": round(nbytes / us_graph / 1e3, 1),
                      "bytes_per_step": nbytes, "steps": steps,
                      "config": {"B": B, "H": H, "K": K, "V": V, "activations": "bf16", "state": "f32"},
                      "note": "HIP events around the launches (includes launch gaps when the host is slower); "
                              "graph_*: the same steps replayed from a captured graph of %d steps" % ng}))


def gate_bench(steps, warmup):
    """The standalone gate (kda_gate: g and alpha, fp32) over the long workload's gate
    input (4 x 32 heads x 16384 tokens x 128 channels, bf16): 10 bytes per element."""
    import torch
    import gated_delta_rule_47_amd as kda
    dev = torch.device("cuda:0")
    B, H, T, K = 4, 32, 16384, 128
    gen = torch.Generator(device=dev).manual_seed(11)
    z = torch.randn(B, H, T, K, device=dev, generator=gen).to(torch.bfloat16)
    A_log = torch.linspace(-2.0, 1.0, H, device=dev)
    dt_bias = 0.5 * torch.randn(H, K, device=dev, generator=gen)
    for _ in range(warmup):
        kda.gate(z, A_log, dt_bias)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        kda.gate(z, A_log, dt_bias)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / steps
    nbytes = B * H * T * K * (2 + 4 + 4)
    del z
    # Ceilings measured in the same run: a plain device copy (read + write) and a write-only
    # fill of the size of the gate's two outputs (four fifths of the gate's bytes are writes).
    copy_gbs = copy_bandwidth_gbs(torch)
    fill = torch.empty(2 * B * H * T * K, dtype=torch.float32, device=dev)
    for _ in range(3):
        fill.fill_(1.0)
    torch.cuda.synchronize()
    a.record()
    for _ in range(steps):
        fill.fill_(1.0)
    b.record()
    torch.cuda.synchronize()
    fill_gbs = fill.numel() * 4 / (a.elapsed_time(b) * 1e-3 / steps) / 1e9
    del fill
    gbs = nbytes / us / 1e3
    print(json.dumps({"metric": "gate bandwidth (kda_gate, g and alpha)", "value": round(gbs, 1),
                      "unit": "GB/s", "frac_of_8TBps": round(gbs / HBM_PEAK_GBS, 4),
                      "copy_GBps": round(copy_gbs, 1), "frac_of_copy": round(gbs / copy_gbs, 4),
                      "write_fill_GBps": round(fill_gbs, 1), "frac_of_write_fill": round(gbs / fill_gbs, 4),
                      "us_per_call": round(us, 2), "bytes_per_call": nbytes, "steps": steps,
                      "config": {"B": B, "H": H, "T": T, "K": K, "z": "bf16", "outputs": "f32 g, alpha"},
                      "note": "HIP events around the calls (each allocates its two outputs through torch's "
                              "caching allocator)"}))


def gate_bwd_bench(steps, warmup):
    """The gate adjoint (kda_gate_bwd: dz, dA_log, d dt_bias) on the long workload's gate
    shape (4 x 32 heads x 16384 tokens x 128 channels, bf16 z, fp32 dg and dz): 10 bytes
    per element (z 2, dg 4 read; dz 4 written), plus the small per-tile partial sums."""
    import torch
    import gated_delta_rule_47_amd as kda
    dev = torch.device("cuda:0")
    B, H, T, K = 4, 32, 16384, 128
    gen = torch.Generator(device=dev).manual_seed(12)
    z = torch.randn(B, H, T, K, device=dev, generator=gen).to(torch.bfloat16)
    dg = torch.randn(B, H, T, K, device=dev, generator=gen)
    A_log = torch.linspace(-2.0, 1.0, H, device=dev)
    dt_bias = 0.5 * torch.randn(H, K, device=dev, generator=gen)
    dz = torch.empty_like(dg)
    ws = torch.empty(max(kda.gate_bwd_workspace_bytes(B, H, T, K), 1), dtype=torch.uint8, device=dev)
    call = lambda: kda.gate_bwd(z, A_log, dt_bias, dg, workspace=ws, dz_out=dz)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        call()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / steps
    nbytes = B * H * T * K * (2 + 4 + 4)
    del z, dg, dz
    copy_gbs = copy_bandwidth_gbs(torch)
    gbs = nbytes / us / 1e3
    print(json.dumps({"metric": "gate adjoint bandwidth (kda_gate_bwd: dz, dA_log, d dt_bias)", "value": round(gbs, 1),
                      "unit": "GB/s", "frac_of_8TBps": round(gbs / HBM_PEAK_GBS, 4),
                      "copy_GBps": round(copy_gbs, 1), "frac_of_copy": round(gbs / copy_gbs, 4),
                      "us_per_call": round(us, 2), "bytes_per_call": nbytes, "steps": steps,
                      "config": {"B": B, "H": H, "T": T, "K": K, "z": "bf16", "dg": "f32", "outputs": "f32 dz"},
                      "note": "HIP events around the calls (caller workspace and dz; three fifths of the bytes "
                              "are reads)"}))


FP32_PEAK_TFLOPS = 157.3      # MI355X dense fp32 (matrix), published


def forward_flops_per_head_token(K: int, V: int, C: int) -> float:
    """Algorithmic flops of the chunked forward per head-token, counting triangular
    products by their nonzero half: 6KV for the state (the decayed read W~S, the output
    read Q~S and the update KR^T U), (C-1)K for the strictly-lower A, (C+1)(K+V) for the
    lower scores P and their product with U, (C-1)(K+V) for forming w and u, and C^2/3
    for the unit-triangular inverse."""
    return 6 * K * V + (C - 1) * K + (C + 1) * (K + V) + (C - 1) * (K + V) + C * C / 3


def adjoint_bench(steps, warmup):
    """kda_chunk_bwd on the adjoint workload (B=2, H=16, T=8192, K=V=128, fp32, chunk 64).
    One JSON line (not the headline metric): head-tokens/s and the fp32 matrix roofline,
    with algorithmic flops = the forward's recomputation plus two products per forward
    product (3x the forward's flops per head-token)."""
    import torch
    import gated_delta_rule_47_amd as kda
    import kda_synth as ks
    wl = ks.WORKLOADS["adjoint"]
    x = ks.generate(wl)
    dev = torch.device("cuda:0")
    d = {n: torch.from_numpy(x[n]).to(dev) for n in ("q", "k", "v", "z", "beta", "A_log", "dt_bias", "state_in",
                                                     "d_out")}
    del x
    ws = torch.empty(kda.chunk_bwd_workspace_bytes(wl.B, wl.H, wl.T, wl.K, wl.V, wl.chunk), dtype=torch.uint8,
                     device=dev)

    def step():
        return kda.chunk_bwd(d["q"], d["k"], d["v"], d["z"], d["A_log"], d["dt_bias"], d["beta"], d["state_in"],
                             d["d_out"], chunk=wl.chunk, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        out = step()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    if not all(torch.isfinite(t).all() for t in out.values()):
        raise SystemExit("non-finite gradient")
    ht = wl.B * wl.H * wl.T
    flops = 3 * forward_flops_per_head_token(wl.K, wl.V, wl.chunk) * ht
    nbytes = ht * ((3 * wl.K + 2 * wl.V + 1) + (3 * wl.K + wl.V + 1)) * 4 + 2 * wl.B * wl.H * wl.K * wl.V * 4
    achieved = flops / (ms * 1e-3) / 1e12
    print(json.dumps({"metric": "KDA chunked adjoint head-tokens/s (kda_chunk_bwd)", "value": round(ht / (ms * 1e-3), 1),
                      "unit": "tokens/s", "ms_per_step": round(ms, 3), "steps": steps, "warmup": warmup,
                      "dtype": "f32", "data": "synthetic",
                      "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "T": wl.T, "K": wl.K, "V": wl.V,
                                 "chunk": wl.chunk},
                      "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": FP32_PEAK_TFLOPS,
                                   "unit": "TFLOP/s", "frac": round(achieved / FP32_PEAK_TFLOPS, 5),
                                   "algorithmic_flops_per_call": flops, "algorithmic_bytes_per_call": nbytes,
                                   "note": "whole call (prep, forward and reverse passes over the chunks, gradient pass), "
                                           "HIP events on the launch stream"}}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed launches first: the GPU takes ~50 ms of load to reach its steady clock")
    ap.add_argument("--workload", default="long")
    ap.add_argument("--chunk", type=int, default=0,
                    help="override the workload's chunk (16, 32 or 64) to compare block sizes; the default "
                         "line uses the workload's own")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--paired", action="store_true",
                    help="pass kda_chunk_fwd a workspace: the two value-tile workgroups of a head share the gate "
                         "and WY stages (bf16, V = 128)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic_long.json"),
                    help="HBM traffic per launch measured by rocprofv3 counters (if present)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="instead of the benchmark, run a plain device-to-device copy of this many MiB "
                         "(--steps times), to calibrate the FETCH_SIZE/WRITE_SIZE counters")
    ap.add_argument("--traffic-from-pmc", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="write --traffic-json from rocprofv3 --pmc CSV directories of the kernel (FETCH_SIZE, "
                         "WRITE_SIZE) and of a --copy-calibration-mib run (same counters); no GPU work")
    ap.add_argument("--calibration-mib", type=int, default=1024, help="size of the calibration copy, MiB")
    ap.add_argument("--decode-batch", type=int, default=0,
                    help="instead of the benchmark, time the decode step (kda_recurrent_step) for this many "
                         "sequences of H=32 heads, K=V=128, bf16 activations (--steps launches)")
    ap.add_argument("--scalar-gate", action="store_true",
                    help="time kda_chunk_fwd_scalar instead (one gate input per head-token: channel 0 of the "
                         "workload's z, bias channel 0 of its dt_bias); a separate metric line")
    ap.add_argument("--norm", action="store_true",
                    help="time kda_chunk_fwd_norm instead (the forward with the output RMSNorm fused; weight "
                         "rows 1 + N(0, 0.1^2), eps 1e-6); a separate metric line")
    ap.add_argument("--gate", action="store_true",
                    help="instead of the benchmark, time the standalone gate (kda_gate) on the long workload's z")
    ap.add_argument("--gate-bwd", action="store_true",
                    help="instead of the benchmark, time the gate adjoint (kda_gate_bwd) on the long workload's z")
    ap.add_argument("--adjoint", action="store_true",
                    help="instead of the benchmark, time kda_chunk_bwd on the adjoint workload (fp32)")
    args = ap.parse_args()
    if args.traffic_from_pmc:
        traffic_from_pmc(*args.traffic_from_pmc, args.calibration_mib, args.workload, args.traffic_json)
        return
    if args.copy_calibration_mib:
        import torch
        n = args.copy_calibration_mib * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": args.steps}))
        return
    if args.gate:
        gate_bench(args.steps, min(args.warmup, 10))
        return
    if args.gate_bwd:
        gate_bwd_bench(args.steps, min(args.warmup, 10))
        return
    if args.adjoint:
        adjoint_bench(args.steps, min(args.warmup, 5))
        return
    if args.decode_batch:
        decode_bench(args.decode_batch, args.steps, args.warmup)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (heads shard across GPUs "
              "with no communication). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_47_amd as kda
    import kda_synth as ks

    wl = ks.WORKLOADS[args.workload]
    if args.chunk:
        wl = wl.with_(chunk=args.chunk)
    if wl.adjoint:
        raise SystemExit("the benchmark times the forward; pick a forward workload")
    print("bench: generating %s (%s)" % (wl.name, wl.desc), file=sys.stderr, flush=True)
    x = ks.generate(wl)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    d = {n: torch.from_numpy(x[n]).to(dev).to(dt) for n in ("q", "k", "v", "z", "beta")}
    A_log = torch.from_numpy(x["A_log"]).to(dev)
    dt_bias = torch.from_numpy(x["dt_bias"]).to(dev)
    state_in = torch.from_numpy(x["state_in"]).to(dev)
    del x
    if args.scalar_gate:
        d["z"] = d["z"][..., 0].contiguous()
        dt_bias = dt_bias[:, 0].contiguous()
    o = torch.empty((wl.B, wl.H, wl.T, wl.V), dtype=dt, device=dev)
    state_out = torch.empty_like(state_in)
    scale = kda.read_scale(wl.K)

    fwd = kda.chunk_fwd_scalar if args.scalar_gate else kda.chunk_fwd
    if args.norm:
        if args.scalar_gate or wl.dtype != "bf16" or args.paired:
            raise SystemExit("--norm times the bf16 per-channel-gate forward only")
        gen = torch.Generator(device=dev).manual_seed(13)
        norm_w = 1.0 + 0.1 * torch.randn((wl.H, wl.V), device=dev, generator=gen)
        nws = kda.chunk_fwd_norm_workspace_bytes(wl.B, wl.H, wl.T, wl.K, wl.V)
        norm_ws = torch.zeros(nws, dtype=torch.uint8, device=dev) if nws else None

        def fwd(q, k, v, z, A_log, dt_bias, beta, state_in, scale, chunk, out, state_out, workspace):
            return kda.chunk_fwd_norm(q, k, v, z, A_log, dt_bias, beta, state_in, norm_weight=norm_w, eps=1e-6,
                                      scale=scale, chunk=chunk, out=out, state_out=state_out, workspace=norm_ws)
    # the paired forward's ring (bf16, V = 128): allocated once, outside the timed region
    ws_bytes = 0 if not args.paired else kda.chunk_fwd_workspace_bytes(wl.B, wl.H, wl.T, wl.K, wl.V, wl.chunk, dt)
    workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None

    def step():
        fwd(d["q"], d["k"], d["v"], d["z"], A_log, dt_bias, d["beta"], state_in, scale=scale, chunk=wl.chunk, out=o,
            state_out=state_out, workspace=workspace)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [a.elapsed_time(b) for a, b in evs]
    if not (torch.isfinite(o[0, 0].float()).all() and torch.isfinite(state_out).all()):
        raise SystemExit("non-finite output")
    if workspace is not None and kda.chunk_fwd_status(workspace) != 0:
        raise SystemExit("the paired forward reported a failed exchange")
    if args.norm and norm_ws is not None and kda.chunk_fwd_status(norm_ws) != 0:
        raise SystemExit("the fused-norm forward reported a failed exchange")

    # the copy ceiling, measured after the timed region on the same (warm) GPU
    copy_gbs = copy_bandwidth_gbs(torch)

    ms_per_step = wall * 1e3 / args.steps
    avg_kernel_ms = float(np.mean(kern_ms))
    tokens = wl.B * wl.H * wl.T
    nbytes = algorithmic_bytes(wl, args.scalar_gate) + (wl.H * wl.V * 4 if args.norm else 0)
    achieved = nbytes / (avg_kernel_ms * 1e-3) / 1e9
    traffic = None
    if os.path.exists(args.traffic_json):
        try:
            tj = json.load(open(args.traffic_json))
            if (tj.get("workload") == wl.name and tj.get("kernel_source_sha256") == kernel_source_hash()
                    and not args.chunk and not args.scalar_gate and not args.norm and not args.paired):
                traffic = tj.get("bytes_per_launch")
        except Exception:
            traffic = None
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "copy_GBps": round(copy_gbs, 1), "frac_of_copy": round(achieved / copy_gbs, 4),
            "kernel": kernel_label(wl, args.scalar_gate, paired=workspace is not None, norm=args.norm),
            "algorithmic_bytes_per_launch": nbytes,
            "avg_kernel_ms": round(avg_kernel_ms, 4), "min_kernel_ms": round(float(np.min(kern_ms)), 4)}
    cpu = None
    if not args.no_cpu_baseline:
        workers = min(16, len(os.sched_getaffinity(0)))
        # two whole heads per worker: about 20 s of CPU work at the long workload
        print("bench: CPU oracle baseline on %d heads" % (2 * workers), file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, n_heads=2 * workers, workers=workers, scalar_gate=args.scalar_gate)
    out = {
        "metric": ((METRIC_NORM if args.norm else METRIC_SCALAR if args.scalar_gate else METRIC) if wl.name == "long"
                   else "KDA chunked-forward tokens/s (B·H·T/s), %s workload%s"
                   % (wl.name, ", scalar-decay gate" if args.scalar_gate else "")), "value": round(tokens / (ms_per_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "T": wl.T, "K": wl.K, "V": wl.V, "chunk": wl.chunk,
                   "block": block_tokens(wl), "activations": wl.dtype, "state": "f32", "global_batch": wl.B, "seq_len": wl.T,
                   "parallelism": "single-gpu"},
        "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
