"""Benchmark: effective INT8 TOPS of the ConvRot int8_linear (+ fused SwiGLU)
hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input, by
default the SwiGLU MLP block (workload c5: M=4096 tokens, hidden 3072,
intermediate 12288, group 128): activation quant -> packed [gate | up] INT8
GEMM -> fused SwiGLU + rotation + quant -> down INT8 GEMM, with INT8 operands
in the blocked layout.  The step calls the four stage entry points of the C ABI
in the order ck_swiglu_mlp uses (a test checks the two agree bit for bit) so
that each kernel can be bracketed by HIP events on the stream it runs on.
Weight preparation and the one-time weight relayout happen before timing, as at
model load.  Inputs are resident in HBM before the timed region.

Settling: before the W warm-up steps the step runs untimed for --settle-ms of
wall time (default 60 ms).  A GPU coming out of idle runs the first steps near
its boost clock, then its power manager pulls the clock well below the level it
sustains before settling there: c5's per-step time from a cold start was ~455 us,
570-586 us at 3-6 ms and 453 us from ~40 ms on, so a 20-step timed region right
after 5 warm-up steps fell into the dip (0.506 against 0.459 ms per step on the
same box).  The JSON line reports settle_ms and the steps it took.

Timing: after the warm-up, a short probe pass (HIP events between every stage)
picks the kernel with the largest share of the step.  In the K timed steps only
that kernel is bracketed by HIP events on its launch stream (events between
every stage stall the queue); its mean bracket is the roofline's duration.  The
per-stage breakdown ("stages") comes from a separate pass after the timed
region with events around every stage; the HBM-bound stages (the quantizers)
are then timed once more, each call alone after a 512 MB read pass that evicts
the 256 MB MALL, and that flushed median is their headline figure.  The CPU
baseline times the oracle stage by stage on the host cores.

Prints one JSON line.  Usage: python bench.py [--steps K] [--warmup W] [--settle-ms T]
[--workload c1..c5] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective INT8 TOPS of ConvRot int8_linear(+SwiGLU), % of MI355X INT8 peak"
PEAK_INT8_TOPS = 5000.0        # MI355X dense INT8 MFMA, 5.0 POP/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense BF16 MFMA, 2.5 PFLOP/s (the W8A16 GEMM)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
PROFILE_DIR = os.path.join(ROOT, "profiles")


class Event:
    """A HIP timing event on the runtime torch has loaded, created with
    hipEventDisableSystemFence: recording it writes a timestamp without the
    system-scope cache write-back and invalidation a default event performs
    (measured here: a default event record costs ~6 us of idle GPU between the
    kernels around it).  Same interface as torch.cuda.Event's timing use."""
    _hip = None

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            import ctypes
            h = ctypes.CDLL("libamdhip64.so.7")        # the copy torch loaded (same soname)
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            for f in (h.hipEventCreateWithFlags, h.hipEventRecord, h.hipEventElapsedTime, h.hipEventDestroy):
                f.restype = ctypes.c_int
            cls._hip = h
        return cls._hip

    def __init__(self):
        import ctypes
        self._h = ctypes.c_void_p()
        rc = self._lib().hipEventCreateWithFlags(ctypes.byref(self._h), 0x20000000)  # DisableSystemFence
        if rc:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")

    def record(self, stream=None):
        import torch
        st = stream if stream is not None else torch.cuda.current_stream()
        rc = self._lib().hipEventRecord(self._h, st.cuda_stream)
        if rc:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def elapsed_time(self, end) -> float:
        import ctypes
        ms = ctypes.c_float()
        rc = self._lib().hipEventElapsedTime(ctypes.byref(ms), self._h, end._h)
        if rc:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return ms.value

    def __del__(self):
        if self._hip is not None and self._h:
            self._hip.hipEventDestroy(self._h)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=60.0,
                    help="untimed steps for this long before the warm-up (0: none)")
    ap.add_argument("--workload", default="c5")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--bias-residual", action="store_true",
                    help="GEMM epilogues add an F32 bias and (down / single GEMM) a BF16 residual")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="rows of the workload the CPU oracle runs (0: automatic)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (for scaling HBM counters)")
    ap.add_argument("--small-m-sweep", action="store_true",
                    help="time the few-row GEMM at M = 1..64 instead of the step (one line per case)")
    ap.add_argument("--decode-mlp", action="store_true",
                    help="time the c5 MLP block at M = 1..64 tokens with weights in the decode layout "
                         "(one line per M)")
    ap.add_argument("--ceilings", action="store_true",
                    help="measure what the chip delivers for this path's kernels: the INT8 MFMA loop on the "
                         "workload's codes (with and without the GEMM's LDS reads) and row streams with the "
                         "quantizers' HBM traffic, beside the quantizers themselves (one line per case)")
    ap.add_argument("--w8a16", action="store_true",
                    help="the W8A16 variant: BF16 rotated activations (no activation quantization) "
                         "times the INT8 weights on BF16 MFMA")
    return ap.parse_args()


def small_m_sweep(steps: int, warmup: int):
    """The few-row path: ck_int8_gemm_bf16 at M in {1, 8, 16, 32, 64} for (N, K) =
    (4096, 4096) and (4096, 12288), with the weight in the blocked layout (scales
    apart) and in the decode layout (scales inside each 16-row group).  Bound by
    HBM: the algorithmic bytes are the weight N*K, the codes M*K, both scale
    vectors and the BF16 output 2*M*N."""
    import torch
    import swiglu_mlp_amd as ck
    dev = torch.device("cuda:0")
    L = ck.lib()
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    stream = torch.cuda.current_stream(dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    for n, k in ((4096, 4096), (4096, 12288)):
        w = torch.randint(-127, 128, (n, k), dtype=torch.int8, device=dev, generator=gen)
        sw = torch.rand(n, device=dev, generator=gen) * 1e-3
        weights = {"blocked": (ck.ck_weight_pack(w), sw, ck.CK_LAYOUT_BLOCKED),
                   "decode": (ck.ck_weight_pack_decode(w, sw), None, ck.CK_LAYOUT_DECODE)}
        for m in (1, 8, 16, 32, 64):
            xq = torch.randint(-127, 128, (ck.blocked_rows(m), k), dtype=torch.int8, device=dev,
                               generator=gen)
            sx = torch.rand(m, device=dev, generator=gen) * 1e-3
            y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            for lay_name, (wt, swt, lay) in weights.items():
                def call():
                    rc = L.ck_int8_gemm_bf16(xq.data_ptr(), sx.data_ptr(), wt.data_ptr(),
                                             None if swt is None else swt.data_ptr(), None, None,
                                             lay, m, n, k, y.data_ptr(), stream.cuda_stream)
                    if rc:
                        raise RuntimeError(L.ck_status_str(rc).decode())
                for _ in range(warmup):
                    call()
                torch.cuda.synchronize()
                # back to back: the weights may stay in the 256 MB MALL between calls
                e0, e1 = Event(), Event()
                e0.record(stream)
                for _ in range(steps):
                    call()
                e1.record(stream)
                torch.cuda.synchronize()
                us_warm = e0.elapsed_time(e1) * 1000.0 / steps
                # flushed: a 512 MB pass between calls evicts the 256 MB MALL and the
                # L2s, each call timed alone (the headline: weights come from HBM).
                # The pass reads (a reduction), so the evicted lines are clean; a
                # writing pass (zero fill) leaves dirty lines whose write-back then
                # competes with the call's reads, reported as the second figure.
                reps = max(5, steps // 5)

                def flushed(flush_op):
                    evs = [(Event(), Event())
                           for _ in range(reps)]
                    for a, b in evs:
                        flush_op()
                        a.record(stream)
                        call()
                        b.record(stream)
                    torch.cuda.synchronize()
                    return sorted(a.elapsed_time(b) for a, b in evs)[reps // 2] * 1000.0
                us = flushed(lambda: flush.view(torch.int32).sum())
                us_wflush = flushed(lambda: flush.zero_())
                nbytes = n * k + m * k + 4 * (m + n) + 2 * m * n
                print(json.dumps({"small_m": {"layout": lay_name, "m": m, "n": n, "k": k,
                                              "us": round(us, 2),
                                              "GBs": round(nbytes / us / 1e3, 1),
                                              "frac_hbm_peak": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 4),
                                              "TOPS": round(2 * m * n * k / us / 1e6, 2),
                                              "us_back_to_back": round(us_warm, 2),
                                              "us_after_write_flush": round(us_wflush, 2),
                                              "timing": "median of single calls after a 512 MB read"}}),
                      flush=True)


def decode_mlp(steps: int, warmup: int, w8a16: bool = False):
    """The c5 SwiGLU MLP block (hidden 3072, intermediate 12288, group 128) at
    decode sizes, M in {1, 2, 8, 16, 64}, through ck_swiglu_mlp with both weights
    in the decode layout, or (w8a16) through ck_swiglu_mlp_w8a16 with both in
    the blocked layout.  Bound by HBM: the weights (2 I H + H I bytes of codes
    plus their scales) are read once per call."""
    import torch
    import swiglu_mlp_amd as ck
    dev = torch.device("cuda:0")
    L = ck.lib()
    h, inter, g = 3072, 12288, 128
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    stream = torch.cuda.current_stream(dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    wgu = torch.randint(-127, 128, (2 * inter, h), dtype=torch.int8, device=dev, generator=gen)
    wd = torch.randint(-127, 128, (h, inter), dtype=torch.int8, device=dev, generator=gen)
    sgu = torch.rand(2 * inter, device=dev, generator=gen) * 1e-3
    sd = torch.rand(h, device=dev, generator=gen) * 1e-3
    if w8a16:
        dgu, dd = ck.ck_weight_pack(wgu), ck.ck_weight_pack(wd)
        wbytes = wgu.numel() + wd.numel() + 4 * (2 * inter + h)
    else:
        dgu, dd = ck.ck_weight_pack_decode(wgu, sgu), ck.ck_weight_pack_decode(wd, sd)
        wbytes = dgu.numel() + dd.numel()
    for m in (1, 2, 8, 16, 64):
        x = (torch.randn((m, h), device=dev, generator=gen)).to(torch.bfloat16)
        y = torch.empty((m, h), dtype=torch.bfloat16, device=dev)
        wsz = L.ck_swiglu_mlp_w8a16_workspace_size(m, h, inter) if w8a16 else \
            L.ck_swiglu_mlp_workspace_size(m, h, inter)
        ws = torch.empty(max(wsz, 1), dtype=torch.uint8, device=dev)

        def call(st=stream):
            if w8a16:
                rc = L.ck_swiglu_mlp_w8a16(x.data_ptr(), dgu.data_ptr(), sgu.data_ptr(), dd.data_ptr(),
                                           sd.data_ptr(), m, h, inter, g, y.data_ptr(), ws.data_ptr(),
                                           ws.numel(), st.cuda_stream)
            else:
                rc = L.ck_swiglu_mlp(x.data_ptr(), dgu.data_ptr(), None, dd.data_ptr(), None,
                                     ck.CK_LAYOUT_DECODE, m, h, inter, g, y.data_ptr(), ws.data_ptr(),
                                     ws.numel(), st.cuda_stream)
            if rc:
                raise RuntimeError(L.ck_status_str(rc).decode())
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        e0, e1 = Event(), Event()
        e0.record(stream)
        for _ in range(steps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        us_b2b = e0.elapsed_time(e1) * 1000.0 / steps
        reps = max(5, steps // 5)
        evs = [(Event(), Event()) for _ in range(reps)]
        for a, b in evs:
            flush.view(torch.int32).sum()
            a.record(stream)
            call()
            b.record(stream)
        torch.cuda.synchronize()
        us = sorted(a.elapsed_time(b) for a, b in evs)[reps // 2] * 1000.0
        # the same call captured in a HIP graph and replayed back to back
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                call(side)
        torch.cuda.synchronize()
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()
        cur = torch.cuda.current_stream(dev)
        e0.record(cur)
        for _ in range(steps):
            graph.replay()
        e1.record(cur)
        torch.cuda.synchronize()
        us_graph = e0.elapsed_time(e1) * 1000.0 / steps
        step = "rotation" if w8a16 else "quantizer"
        kernels = [f"gate_up with the x {step} inside"] if m <= 2 else [f"x {'rotate' if w8a16 else 'quant'}",
                                                                        "gate_up"]
        kernels += [f"down with the SwiGLU {step} inside"] if m <= 2 else \
            [f"SwiGLU {'rotate' if w8a16 else 'quant'}", "down"]
        print(json.dumps({"decode_mlp": {"m": m, "hidden": h, "intermediate": inter,
                                         "variant": "W8A16, blocked weights" if w8a16 else "INT8, decode weights",
                                         "us": round(us, 2),
                                         "weight_MB": round(wbytes / 1e6, 1),
                                         "GBs_weights": round(wbytes / us / 1e3, 1),
                                         "frac_hbm_peak": round(wbytes / us / 1e3 / PEAK_HBM_GBS, 4),
                                         "us_back_to_back": round(us_b2b, 2),
                                         "us_graph_back_to_back": round(us_graph, 2),
                                         "timing": "median of single calls after a 512 MB read",
                                         "kernels": kernels}}), flush=True)


def ceilings():
    """What MI355X delivers for the path's kernels, measured on the c5 shapes.

    The chip is power-limited: its INT8 MFMA rate depends on the operand bits,
    so the MFMA loop (ck_probe_mfma_i8: one workgroup per CU, 16 independent
    accumulators per wave) runs on 16 KB of the workload's own codes (weight
    and activation, blocked), on uniform codes and on zeros, alone and with the
    0.5 KB of LDS reads per MFMA that the 256 x 256 GEMM tile needs.  The HBM
    side: ck_probe_stream_rows moves each quantizer's exact bytes (rows of BF16
    in, one byte per element out) with trivial compute; it and the quantizer
    itself are timed as single calls after a 512 MB read pass (median of 11)."""
    import numpy as np
    import torch
    import swiglu_mlp_amd as ck
    from swiglu_mlp_amd import workloads as W
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = ck.lib()
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    wl = W.WORKLOADS["c5"]
    d = W.mlp_inputs(wl)
    g, m, h, inter = wl.group, wl.m, wl.k, wl.n

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    x = to_dev(d["x"].view(np.int16)).view(torch.bfloat16)
    wgu, sgu = ck.ck_weight_prep(to_dev(d["w_gu"]), g)
    xq, sx = ck.ck_act_quant(x, None, g)
    t1 = ck.ck_int8_gemm_bf16(xq, sx, wgu, sgu)
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    codes = {"workload codes (W_gu and x, blocked)": torch.cat([wgu.reshape(-1)[:8192], xq.reshape(-1)[:8192]]),
             "uniform codes in [-127, 127]": torch.randint(-127, 128, (16384,), dtype=torch.int8, device=dev,
                                                           generator=gen),
             "zero codes": torch.zeros(16384, dtype=torch.int8, device=dev)}
    nwg = L.ck_probe_mfma_workgroups()
    sink = torch.empty(nwg * 256, dtype=torch.int32, device=dev)
    iters = 20000
    ops = nwg * 4 * iters * 16 * 65536
    for name, buf in codes.items():
        buf = buf.contiguous()
        for lds in (0, 1):
            times = []
            for rep in range(4):
                e0, e1 = Event(), Event()
                e0.record(stream)
                rc = L.ck_probe_mfma_i8(buf.data_ptr(), iters, lds, sink.data_ptr(), sptr)
                e1.record(stream)
                if rc:
                    raise RuntimeError(L.ck_status_str(rc).decode())
                torch.cuda.synchronize()
                if rep:
                    times.append(e0.elapsed_time(e1) * 1000.0)
            us = sorted(times)[len(times) // 2]
            print(json.dumps({"ceiling": {"kind": "int8 MFMA loop", "operands": name,
                                          "lds_reads": "0.5 KB per MFMA" if lds else "none",
                                          "us": round(us, 1), "TOPS": round(ops / us / 1e6, 1),
                                          "frac_int8_peak": round(ops / us / 1e6 / PEAK_INT8_TOPS, 4)}}),
                  flush=True)

    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def flushed(call, reps=11):
        evs = [(Event(), Event()) for _ in range(reps)]
        for a, b in evs:
            flush.view(torch.int32).sum()
            a.record(stream)
            rc = call()
            b.record(stream)
            if rc:
                raise RuntimeError(L.ck_status_str(rc).decode())
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in evs)[reps // 2] * 1000.0

    hq = torch.empty((ck.blocked_rows(m), inter), dtype=torch.int8, device=dev)
    sh = torch.empty((m,), dtype=torch.float32, device=dev)
    cases = [
        ("swiglu_quant", t1, 2 * inter * 2, inter,
         lambda: L.ck_act_quant(t1.data_ptr(), 2 * inter, m, inter, 1, g, ck.CK_LAYOUT_BLOCKED, hq.data_ptr(),
                                sh.data_ptr(), sptr)),
        ("x_quant", x, h * 2, h,
         lambda: L.ck_act_quant(x.data_ptr(), h, m, h, 0, g, ck.CK_LAYOUT_BLOCKED, xq.data_ptr(), sx.data_ptr(),
                                sptr)),
    ]
    for name, src, rb, wb, quant in cases:
        dst = torch.empty(m * wb, dtype=torch.uint8, device=dev)
        stream_us = flushed(lambda: L.ck_probe_stream_rows(src.data_ptr(), rb, m, rb, wb, dst.data_ptr(), sptr))
        quant_us = flushed(quant)
        nbytes = m * rb + m * wb + 4 * m
        print(json.dumps({"ceiling": {"kind": "HBM row stream", "traffic_of": f"c5 {name}",
                                      "bytes": nbytes, "stream_us": round(stream_us, 2),
                                      "stream_GBs": round(nbytes / stream_us / 1e3, 1),
                                      "stream_frac_hbm_peak": round(nbytes / stream_us / 1e3 / PEAK_HBM_GBS, 4),
                                      "quantizer_us": round(quant_us, 2),
                                      "quantizer_GBs": round(nbytes / quant_us / 1e3, 1),
                                      "quantizer_frac_of_stream": round(stream_us / quant_us, 4),
                                      "timing": "median of single calls after a 512 MB read pass"}}), flush=True)


def copy_calibration():
    """A plain elementwise copy of a known size: the reference that scales the
    FETCH_SIZE / WRITE_SIZE counters of the path's kernels to bytes."""
    import torch
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.int32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"kernel": "torch.neg int32", "bytes_read": n,
                                           "bytes_written": n, "launches": 5}}), flush=True)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for f in ("gemm_blk.hip", "quant.hip", "ck_device.hpp"):
        with open(os.path.join(ROOT, "swiglu_mlp_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, per_launch_units: float):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE runs,
    only if they were taken on the current kernel sources."""
    path = os.path.join(PROFILE_DIR, f"traffic_{kernel}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha") != kernel_source_sha():
        return None
    return t.get("bytes_per_launch")


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.ceilings:
        ceilings()
        return
    if args.small_m_sweep:
        small_m_sweep(args.steps, args.warmup)
        return
    if args.decode_mlp:
        decode_mlp(args.steps, args.warmup, args.w8a16)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}).  Every step of the path is per token, so splitting "
              f"the tokens over N GPUs needs no exchange; that is not run here.",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import swiglu_mlp_amd as ck
    from swiglu_mlp_amd import workloads as W

    wl = W.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = ck.lib()
    print(f"[bench] workload {wl.name}: {wl.desc}", file=sys.stderr, flush=True)

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    g = wl.group
    BLK = ck.CK_LAYOUT_BLOCKED
    if wl.kind == "mlp":
        d = W.mlp_inputs(wl)
        m, h, inter = wl.m, wl.k, wl.n
        mp = ck.blocked_rows(m)
        x = to_dev(d["x"].view(np.int16)).view(torch.bfloat16)
        # load-time prep: rotated INT8 codes in the blocked layout, row scales
        wgu, sgu = ck.ck_weight_prep(to_dev(d["w_gu"]), g)
        wd, sd = ck.ck_weight_prep(to_dev(d["w_down"]), g)
        xq = torch.empty((mp, h), dtype=torch.int8, device=dev)
        sx = torch.empty((m,), dtype=torch.float32, device=dev)
        t1 = torch.empty((m, 2 * inter), dtype=torch.bfloat16, device=dev)
        hq = torch.empty((mp, inter), dtype=torch.int8, device=dev)
        sh = torch.empty((m,), dtype=torch.float32, device=dev)
        y = torch.empty((m, h), dtype=torch.bfloat16, device=dev)
        # optional epilogue terms: biases on both GEMMs, the block input as the
        # down projection's residual (a transformer block's skip connection)
        ex = args.bias_residual
        b_gu = torch.randn(2 * inter, device=dev) * 0.1 if ex else None
        b_d = torch.randn(h, device=dev) * 0.1 if ex else None
        gu_extra = (b_gu.data_ptr() if ex else None, None)
        d_extra = (b_d.data_ptr() if ex else None, x.data_ptr() if ex else None)
        xb = (2 * inter * 4) if ex else 0
        db = (h * 4 + m * h * 2) if ex else 0
        # (name, callable, algorithmic ops, algorithmic HBM bytes, bound)
        if args.w8a16:
            xr = torch.empty((mp, h), dtype=torch.bfloat16, device=dev)
            hr = torch.empty((mp, inter), dtype=torch.bfloat16, device=dev)
        stages = [
            ("x_rotate_bf16", lambda s: L.ck_act_rotate_bf16(x.data_ptr(), h, m, h, 0, g, BLK, xr.data_ptr(), s),
             0, m * h * 4, "hbm"),
            ("gate_up_w8a16", lambda s: L.ck_w8a16_gemm_bf16(xr.data_ptr(), wgu.data_ptr(), sgu.data_ptr(),
                                                             *gu_extra, m, 2 * inter, h, t1.data_ptr(), s),
             2 * m * 2 * inter * h, m * h * 2 + 2 * inter * h + m * 2 * inter * 2 + xb, "mfma_bf16"),
            ("swiglu_rotate_bf16", lambda s: L.ck_act_rotate_bf16(t1.data_ptr(), 2 * inter, m, inter, 1, g,
                                                                  BLK, hr.data_ptr(), s),
             0, m * inter * 6, "hbm"),
            ("down_w8a16", lambda s: L.ck_w8a16_gemm_bf16(hr.data_ptr(), wd.data_ptr(), sd.data_ptr(),
                                                          *d_extra, m, h, inter, y.data_ptr(), s),
             2 * m * h * inter, m * inter * 2 + h * inter + m * h * 2 + db, "mfma_bf16"),
        ] if args.w8a16 else [
            ("x_quant", lambda s: L.ck_act_quant(x.data_ptr(), h, m, h, 0, g, BLK, xq.data_ptr(),
                                                 sx.data_ptr(), s),
             0, m * h * 2 + m * h + m * 4, "hbm"),
            ("gate_up_gemm", lambda s: L.ck_int8_gemm_bf16(xq.data_ptr(), sx.data_ptr(),
                                                           wgu.data_ptr(), sgu.data_ptr(), *gu_extra, BLK,
                                                           m, 2 * inter, h, t1.data_ptr(), s),
             2 * m * 2 * inter * h, m * h + 2 * inter * h + m * 2 * inter * 2 + xb, "mfma"),
            ("swiglu_quant", lambda s: L.ck_act_quant(t1.data_ptr(), 2 * inter, m, inter, 1, g,
                                                      BLK, hq.data_ptr(), sh.data_ptr(), s),
             0, m * inter * 4 + m * inter + m * 4, "hbm"),
            ("down_gemm", lambda s: L.ck_int8_gemm_bf16(hq.data_ptr(), sh.data_ptr(),
                                                        wd.data_ptr(), sd.data_ptr(), *d_extra, BLK,
                                                        m, h, inter, y.data_ptr(), s),
             2 * m * h * inter, m * inter + h * inter + m * h * 2 + db, "mfma"),
        ]
    else:
        d = W.linear_inputs(wl)
        m, k, n = wl.m, wl.k, wl.n
        ldx = 2 * k if wl.act == 1 else k
        x = to_dev(d["x"].view(np.int16)).view(torch.bfloat16)
        wq, sw = ck.ck_weight_prep(to_dev(d["w"]), g)           # blocked layout
        xq = torch.empty((ck.blocked_rows(m), k), dtype=torch.int8, device=dev)
        sx = torch.empty((m,), dtype=torch.float32, device=dev)
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        ex = args.bias_residual
        bias = torch.randn(n, device=dev) * 0.1 if ex else None
        res = (torch.randn((m, n), device=dev) * 0.5).to(torch.bfloat16) if ex else None
        extra = (bias.data_ptr() if ex else None, res.data_ptr() if ex else None)
        eb = (n * 4 + m * n * 2) if ex else 0
        if args.w8a16:
            xr = torch.empty((ck.blocked_rows(m), k), dtype=torch.bfloat16, device=dev)
        stages = [
            ("act_rotate_bf16", lambda s: L.ck_act_rotate_bf16(x.data_ptr(), ldx, m, k, wl.act, g, BLK,
                                                               xr.data_ptr(), s),
             0, m * ldx * 2 + m * k * 2, "hbm"),
            ("w8a16_gemm", lambda s: L.ck_w8a16_gemm_bf16(xr.data_ptr(), wq.data_ptr(), sw.data_ptr(), *extra,
                                                          m, n, k, y.data_ptr(), s),
             2 * m * n * k, m * k * 2 + n * k + m * n * 2 + eb, "mfma_bf16"),
        ] if args.w8a16 else [
            ("act_quant", lambda s: L.ck_act_quant(x.data_ptr(), ldx, m, k, wl.act, g, BLK,
                                                   xq.data_ptr(), sx.data_ptr(), s),
             0, m * ldx * 2 + m * k + m * 4, "hbm"),
            ("gemm", lambda s: L.ck_int8_gemm_bf16(xq.data_ptr(), sx.data_ptr(), wq.data_ptr(),
                                                   sw.data_ptr(), *extra, BLK, m, n, k, y.data_ptr(), s),
             2 * m * n * k, m * k + n * k + m * n * 2 + eb, "mfma"),
        ]
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream

    def run_step(events=None, only=None):
        """One step; `events[j]` brackets stage j (all stages, or only stage `only`)."""
        for j, st in enumerate(stages):
            timed = events is not None and (only is None or j == only)
            if timed:
                events[j][0].record(stream)
            rc = st[1](sptr)
            if rc != 0:
                raise RuntimeError(f"{st[0]} returned {rc}: {L.ck_status_str(rc).decode()}")
            if timed:
                events[j][1].record(stream)

    def new_events():
        return [[Event(), Event()]
                for _ in stages]

    def stage_means(ev, steps, which):
        return {stages[j][0]: 1000.0 * sum(ev[i][j][0].elapsed_time(ev[i][j][1])
                                           for i in range(steps)) / steps for j in which}

    # settle (see the module docstring), then the warm-up, then a short pass
    # with every stage bracketed to find the kernel with the largest share of
    # the step
    settle_steps = 0
    if args.settle_ms > 0:
        t_end = time.perf_counter() + args.settle_ms / 1000.0
        while time.perf_counter() < t_end or settle_steps < 8:
            for _ in range(4):
                run_step()
            settle_steps += 4
            torch.cuda.synchronize()
    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()
    probe_steps = 3
    pev = [new_events() for _ in range(probe_steps)]
    for i in range(probe_steps):
        run_step(pev[i])
    torch.cuda.synchronize()
    probe = stage_means(pev, probe_steps, range(len(stages)))
    dom = max(range(len(stages)), key=lambda j: probe[stages[j][0]])

    # timed region: K steps; HIP events on the launch stream bracket only the
    # dominant kernel (events between every stage would stall the queue)
    K = args.steps
    ev = [new_events() for _ in range(K)]
    start, end = Event(), Event()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(K):
        run_step(ev[i], only=dom)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / K
    value = wl.int8_ops / (ms_per_step * 1e-3) / 1e12

    name, _, ops, nbytes, bound = stages[dom]
    dom_us = stage_means(ev, K, [dom])[name]
    t_s = dom_us * 1e-6
    if bound == "mfma_bf16":
        bound = "mfma"
        achieved, peak, unit = ops / t_s / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    elif bound == "mfma":
        achieved, peak, unit = ops / t_s / 1e12, PEAK_INT8_TOPS, "TOPS"
    else:
        achieved, peak, unit = nbytes / t_s / 1e9, PEAK_HBM_GBS, "GB/s"
    roofline = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": load_traffic(name, 1.0),
                "kernel": name, "avg_us": round(dom_us, 2)}

    # per-stage breakdown: a separate pass after the timed region, every stage
    # bracketed
    bk = min(K, 10)
    bev = [new_events() for _ in range(bk)]
    for i in range(bk):
        run_step(bev[i])
    torch.cuda.synchronize()
    kern_us = stage_means(bev, bk, range(len(stages)))
    # HBM-bound stages again, each call alone after a 512 MB read pass that
    # evicts the 256 MB MALL and the L2s (its inputs then come from HBM): the
    # headline figure for those stages; the back-to-back one is kept beside it
    flushed_us = {}
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    for j, st in enumerate(stages):
        if st[4] != "hbm":
            continue
        reps = 11
        fev = [(Event(), Event()) for _ in range(reps)]
        for a, b in fev:
            flush.view(torch.int32).sum()
            a.record(stream)
            rc = st[1](sptr)
            if rc != 0:
                raise RuntimeError(f"{st[0]} returned {rc}")
            b.record(stream)
        torch.cuda.synchronize()
        flushed_us[st[0]] = sorted(a.elapsed_time(b) for a, b in fev)[reps // 2] * 1000.0
    del flush
    stage_roofline = {}
    for st in stages:
        ts = kern_us[st[0]] * 1e-6
        if st[4] == "mfma":
            stage_roofline[st[0]] = {"us": round(kern_us[st[0]], 2),
                                     "TOPS": round(st[2] / ts / 1e12, 1),
                                     "frac_int8_peak": round(st[2] / ts / 1e12 / PEAK_INT8_TOPS, 4)}
        elif st[4] == "mfma_bf16":
            stage_roofline[st[0]] = {"us": round(kern_us[st[0]], 2),
                                     "TFLOPS": round(st[2] / ts / 1e12, 1),
                                     "frac_bf16_peak": round(st[2] / ts / 1e12 / PEAK_BF16_TFLOPS, 4)}
        else:
            tf = flushed_us[st[0]] * 1e-6
            stage_roofline[st[0]] = {"us": round(flushed_us[st[0]], 2),
                                     "GBs": round(st[3] / tf / 1e9, 1),
                                     "frac_hbm_peak": round(st[3] / tf / 1e9 / PEAK_HBM_GBS, 4),
                                     "timing": "median of single calls after a 512 MB read pass",
                                     "us_back_to_back": round(kern_us[st[0]], 2),
                                     "GBs_back_to_back": round(st[3] / ts / 1e9, 1)}

    cpu = None
    if not args.no_cpu_baseline and not args.w8a16:
        cpu = cpu_baseline(wl, d, args.cpu_rows)

    metric, unit, dtype = METRIC, "TOPS", "int8"
    if args.w8a16:
        metric = "effective TFLOP/s of the W8A16 ConvRot linear (BF16 activations, INT8 weights)"
        unit, dtype = "TFLOP/s", "bf16xint8"
    line = {
        "metric": metric, "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "settle_ms": args.settle_ms, "settle_steps": settle_steps,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.desc}", "m": wl.m, "k": wl.k, "n": wl.n,
                   "group": g, "int8_ops_per_step": wl.int8_ops, "parallelism": "single-gpu",
                   "epilogue": "bias+residual" if args.bias_residual else "dequant",
                   "activations": "bf16 (W8A16)" if args.w8a16 else "int8"},
        ("frac_of_bf16_peak" if args.w8a16 else "frac_of_int8_peak"):
            round(value / (PEAK_BF16_TFLOPS if args.w8a16 else PEAK_INT8_TOPS), 4),
        "roofline": roofline, "stages": stage_roofline, "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(line), flush=True)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, d, rows):
    """The CPU oracle, as it stands, on a bounded row sample of the same step,
    each stage timed on its own: weight prep (load time, once per weight),
    activation quant (with SwiGLU for the down projection), the int32 GEMM
    and the dequant epilogue.  Rates use the GPU lines' formulas: quantizers
    and epilogue in GB/s of algorithmic bytes, the GEMM in TOPS."""
    import numpy as np
    import oracle
    g = wl.group
    threads = int(os.environ.get("OMP_NUM_THREADS") or len(os.sched_getaffinity(0)))
    t0 = time.perf_counter()
    if wl.kind == "mlp":
        gq, gs = oracle.weight_prep(d["w_gu"], g)
        dq, ds = oracle.weight_prep(d["w_down"], g)
        wbytes = d["w_gu"].size * 5 + d["w_down"].size * 5
        linears = [(0, gq, gs), (1, dq, ds)]
    else:
        wq, sw = oracle.weight_prep(d["w"], g)
        wbytes = d["w"].size * 5
        linears = [(wl.act, wq, sw)]
    t_prep = time.perf_counter() - t0

    def run(r):
        """One pass over the first r rows; per-stage seconds and bytes/ops."""
        st = {"act_quant": [0.0, 0], "int_gemm": [0.0, 0], "epilogue": [0.0, 0]}
        a = np.ascontiguousarray(d["x"][:r])
        for act, q, s in linears:
            n, k = q.shape
            t = time.perf_counter()
            xq, sx = oracle.act_quant(a, act, g, k=k)
            t1 = time.perf_counter()
            acc = oracle.gemm_i32(xq, q)
            t2 = time.perf_counter()
            a = oracle.dequant(acc, sx, s)
            t3 = time.perf_counter()
            st["act_quant"][0] += t1 - t
            st["act_quant"][1] += r * k * (4 if act == 1 else 2) + r * k + 4 * r
            st["int_gemm"][0] += t2 - t1
            st["int_gemm"][1] += 2 * r * n * k
            st["epilogue"][0] += t3 - t2
            st["epilogue"][1] += r * n * 4 + r * n * 2 + 4 * (r + n)
        return st

    ops_per_row = (6 if wl.kind == "mlp" else 2) * wl.k * wl.n
    if not rows:
        # size the sample to ~12 s of CPU work: a prefix of the rows, or the
        # whole batch repeated when that is cheaper
        probe = min(wl.m, 32)
        st = run(probe)
        per_row = sum(v[0] for v in st.values()) / probe
        rows = int(min(wl.m, max(probe, 12.0 / max(per_row, 1e-9))))
    reps, tot = 0, None
    t0 = time.perf_counter()
    while True:
        st = run(rows)
        reps += 1
        tot = st if tot is None else {k: [tot[k][0] + v[0], tot[k][1] + v[1]] for k, v in st.items()}
        if rows < wl.m or time.perf_counter() - t0 > 8.0 or reps >= 16:
            break
    dt = sum(v[0] for v in tot.values())
    what = f"first {rows} of {wl.m} rows" if rows < wl.m else f"all {rows} rows, {reps} time(s)"
    stages = {
        "weight_prep": {"s": round(t_prep, 3), "GBs": round(wbytes / t_prep / 1e9, 3),
                        "what": "rotate + quantize every weight once (load time, not in value)"},
        "act_quant": {"s": round(tot["act_quant"][0], 3),
                      "GBs": round(tot["act_quant"][1] / tot["act_quant"][0] / 1e9, 3)},
        "int_gemm": {"s": round(tot["int_gemm"][0], 3),
                     "TOPS": round(tot["int_gemm"][1] / tot["int_gemm"][0] / 1e12, 5)},
        "epilogue": {"s": round(tot["epilogue"][0], 3),
                     "GBs": round(tot["epilogue"][1] / tot["epilogue"][0] / 1e9, 3)},
    }
    return {"value": round(ops_per_row * rows * reps / dt / 1e12, 5), "unit": "TOPS", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{what} of {wl.name}: the whole step (activation quant, int GEMM, "
                      f"epilogue; both stages for the MLP), {dt:.1f} s",
            "stages": stages}


if __name__ == "__main__":
    main()
