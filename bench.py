#!/usr/bin/env python3
"""Benchmark of the MXFP8 m<=8 GEMM + Lamport publish + collect on one MI355X.

One step is one pass of the whole hot path over one call's inputs: the GEMM
with its BF16 publish into the mailbox (mxgemm_publish) and the collect that
empties the mailbox (mailbox_collect). The workload is N=7168, K=8192, m=8,
split-K 4, one rank slot, W ~ N(0, 0.02) and x ~ N(0, 1) with 1 % of channels
x50, MXFP8-quantized per 32 (seeded). Inputs are resident in HBM before the
timed region; every step reads one of ceil(cold MiB / |W|) copies of W and its
scales in turn, so W comes from HBM and not from the 256 MiB Infinity Cache.

The timed region is one replay of a HIP graph holding the K steps back to
back (the decode loop as it is served); `value` is algorithmic bytes per step
over the replay's time per step. The GEMM kernel's own duration comes from
HIP events recorded around each launch on its stream (hipExtLaunchKernel) in
a separate eager pass of K steps; the roofline compares algorithmic bytes per
launch over that mean duration with the 8 TB/s HBM peak. Also printed: the
eager time per step, the parity of the final output against the CPU oracle,
and the oracle's own time on the host (cpu_baseline).

    python bench.py [--gpus 1] [--steps 100] [--warmup 10] [--dist outliers]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("µs/call and achieved HBM GB/s (fraction of peak), MXFP8 m≤8 "
          "GEMM+publish")
HBM_PEAK_GBS = 8000.0


def parse() -> argparse.Namespace:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--dist", default="outliers", choices=["outliers", "normal"])
    ap.add_argument("--warm", action="store_true", help="one W copy (Infinity-Cache resident)")
    ap.add_argument("--cold-mib", type=int, default=2048,
                    help="total size of the rotating W copies")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-calls", type=int, default=40)
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="before the timed steps, one plain device copy of this many MiB "
                         "(the known-size reference for HBM byte counters)")
    return ap.parse_args()


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gemm_publish_n7168_k8192_m8_s4_hbm_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "mxfp8_decode_gemm_amd", "csrc", f)
                  for f in ("gemm_publish.hip", "mxgemm_internal.h")]


def kernel_source_hash() -> str:
    """SHA-256 over the GEMM kernel's source files, in order."""
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_from_profile():
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by its reading for a plain copy of
    known size), or None when the kernel sources changed since it was taken."""
    try:
        with open(TRAFFIC_PROFILE) as f:
            fields = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith("#"))
    except OSError:
        return None
    fields = {k.strip().strip("`- "): v.strip().strip("`") for k, v in fields.items()}
    if fields.get("source_sha256") != kernel_source_hash():
        return None
    try:
        return int(float(fields["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_baseline(problem, calls: int) -> tuple[dict, object]:
    """Time the CPU oracle on the same workload (test infrastructure, timed
    here only as a reported baseline)."""
    import numpy as np

    from oracle import gemm, mailbox

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    times = []
    result = None
    for _ in range(calls):
        t0 = time.perf_counter()
        bits, exact, abs_sum = gemm.gemm_publish_bits(problem.w, problem.ws, problem.x,
                                                      problem.xs)
        mb = mailbox.MailboxModel(1, 114688)
        mb.publish(0, bits)
        out = mb.collect(problem.out_bytes)
        times.append(time.perf_counter() - t0)
        result = (bits, exact, abs_sum, out)
    sec = float(np.median(times))
    cpu = {
        "value": round(problem.algorithmic_bytes() / sec / 1e9, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{calls} full calls of the same N=7168 K=8192 m=8 workload (dequantize, "
                   f"float64 GEMM, BF16 RNE, -0 clear, mailbox publish+collect model); "
                   f"median {sec:.3f} s per call"),
    }
    return cpu, result


def main() -> int:
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the exchange "
              "across GPUs is a design only, and the workload is one GPU's share",
              file=sys.stderr)
        return 2
    import numpy as np
    import torch

    from mxfp8_decode_gemm_amd import binding as mx
    from mxfp8_decode_gemm_amd import device as dv
    from workloads import generate

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    p = generate.config_problem(2, dist=args.dist)
    split_k = p.split_k
    wbytes = p.w.nbytes + p.ws.nbytes  # packed sizes are equal when N % 16 == 0
    copies = 1 if args.warm else max(1, -(-(args.cold_mib * 2**20) // wbytes))
    # W and its scales are packed once into the GEMM's tile layout (a load-time
    # re-layout), then copied so consecutive steps read different HBM.
    w0, ws0 = dv.pack_weight(dv.upload(p.w, dev), dv.upload(p.ws, dev), p.n, p.k)
    torch.cuda.synchronize()
    ws_copies = [(w0, ws0)] + [(w0.clone(), ws0.clone()) for _ in range(copies - 1)]
    x = dv.upload(p.x, dev)
    xs = dv.upload(p.xs, dev)
    mbx = dv.Mailbox(1, 114688, device=dev)
    wsp = dv.Workspace(p.n, split_k, device=dev)
    out = torch.empty(p.m * p.n, dtype=torch.int16, device=dev)
    stream = torch.cuda.Stream(device=dev)
    nbytes = p.out_bytes

    def step(i, ev=None):
        w, ws = ws_copies[i % copies]
        if ev is None:
            mx.mxgemm_publish(mbx.mb, w, ws, x, xs, p.m, p.n, p.k, split_k, wsp.buf,
                              wsp.nbytes, None, stream)
        else:
            mx.mxgemm_publish_timed(mbx.mb, w, ws, x, xs, p.m, p.n, p.k, split_k, wsp.buf,
                                    wsp.nbytes, None, stream, ev[0], ev[1])
        mx.mailbox_collect(mbx.mb, out, nbytes, stream)

    if args.copy_mib > 0:
        src = torch.empty(args.copy_mib * 2**20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    def gemm(i):
        w, ws = ws_copies[i % copies]
        mx.mxgemm_publish(mbx.mb, w, ws, x, xs, p.m, p.n, p.k, split_k, wsp.buf, wsp.nbytes,
                          None, stream)

    def replay(body):
        """Capture body() once as a HIP graph; replay it once warm, then once
        between two events on `stream`; returns the timed replay in ms."""
        mx.mxg_graph_begin(stream)
        body()
        graph = mx.mxg_graph_end(stream)
        mx.mxg_graph_launch(graph, stream)
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        mx.mxg_graph_launch(graph, stream)
        g1.record(stream)
        torch.cuda.synchronize()
        mx.mxg_graph_destroy(graph)
        return g0.elapsed_time(g1)

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
        stream.synchronize()
        # Eager pass: HIP events recorded around each GEMM launch itself
        # (hipExtLaunchKernel), and the eager time per step.
        kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for a, b in kev:  # materialize the event handles
            a.record(stream)
            b.record(stream)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            step(i, kev[i])
        e1.record(stream)
        torch.cuda.synchronize()
        eager_ms_step = e0.elapsed_time(e1) / args.steps
        ext_ms = [a.elapsed_time(b) for a, b in kev]

        # The GEMM kernel's duration: K launches back to back (no collect in
        # between; each republishes into the same generation), one graph,
        # events around the replay on the launch stream. A collect drains
        # the mailbox after each replay.
        def gemms():
            for i in range(args.steps):
                gemm(i)

        def drain():
            mx.mailbox_collect(mbx.mb, out, nbytes, stream)

        mx.mxg_graph_begin(stream)
        gemms()
        graph = mx.mxg_graph_end(stream)
        mx.mxg_graph_launch(graph, stream)
        drain()
        torch.cuda.synchronize()
        k0 = torch.cuda.Event(enable_timing=True)
        k1 = torch.cuda.Event(enable_timing=True)
        k0.record(stream)
        mx.mxg_graph_launch(graph, stream)
        k1.record(stream)
        drain()
        torch.cuda.synchronize()
        mx.mxg_graph_destroy(graph)
        kern_ms = k0.elapsed_time(k1) / args.steps

        # Timed region: the K whole steps captured once as a HIP graph.
        ms_step = replay(lambda: [step(i) for i in range(args.steps)]) / args.steps
        gemm_calls = args.warmup + 5 * args.steps
        collects = args.warmup + 3 * args.steps + 2
        st = mbx.state_words()
        hdr = wsp.header()
    got = dv.as_u16(out).reshape(p.m, p.n)

    algo = p.algorithmic_bytes()
    achieved = algo / (kern_ms * 1e-3) / 1e9
    traffic = traffic_from_profile()
    line = {
        "metric": METRIC,
        "value": round(algo / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "N=7168 K=8192 m=8 split-K 4 MXFP8 (e4m3 + E8M0/32) GEMM, BF16 "
                        "publish into a 1-slot 3-generation Lamport mailbox, then collect",
            "n": p.n, "k": p.k, "m": p.m, "split_k": split_k, "ranks": 1,
            "dist": args.dist, "seed": p.seed, "w_copies": copies,
            "algorithmic_bytes_per_call": algo,
        },
        "us_per_call": round(ms_step * 1e3, 3),
        "eager_us_per_call": round(eager_ms_step * 1e3, 3),
        "gemm_kernel_us": round(kern_ms * 1e3, 3),
        "gemm_launch_event_us": {"mean": round(float(np.mean(ext_ms)) * 1e3, 3),
                                 "min": round(min(ext_ms) * 1e3, 3),
                                 "max": round(max(ext_ms) * 1e3, 3)},
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
        },
        "state_ok": bool(st[mx.STATE_NEXT] == collects % 3 and st[mx.STATE_ERROR] == 0
                         and hdr[mx.WS_EPOCH] == 1 + gemm_calls and hdr[mx.WS_ERROR] == 0),
    }
    if not args.no_cpu_baseline:
        from oracle import codecs, tolerance

        cpu, (bits, exact, abs_sum, _) = cpu_baseline(p, args.cpu_calls)
        line["cpu_baseline"] = cpu
        ex = tolerance.excess(got, exact, abs_sum)
        same = codecs.bf16_to_f64(got) == codecs.bf16_to_f64(bits)
        line["parity"] = {"within_tolerance": bool(np.all(ex <= 1.0)),
                          "max_excess": round(float(ex.max()), 4),
                          "bits_equal_oracle_frac": round(float(same.mean()), 5),
                          "no_negative_zero": bool(not np.any(got == 0x8000))}
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
