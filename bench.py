#!/usr/bin/env python3
"""Benchmark of the Leech-lattice dequantize-plus-matvec hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one batch-1 Leech GEMV y = W x at 4096 x 12288 (down_proj-shaped,
shells 2..6 with P(m) ~ 2^-m, the workload the metric is quoted on), on seeded
synthetic inputs already resident in HBM.  Parity of every kernel at exactly
these shapes and seeds is the GPU test suite's job; here the cpu_baseline leg,
which runs the f64 oracle on the same workload to time it, also reports the
largest error ratio of the timed Leech output.  To keep the 256 MB Infinity
Cache from serving the weights,
the timed launches rotate over enough copies of the blob to touch more than
512 MB.  Per-launch HIP events on the launch stream give the kernel's average
duration (roofline.achieved); the region's events give whole-job throughput
(value).  The comparison arms (fp16 control, BPDQ, bitshift trellis) are timed
the same way and reported under "arms".  The oracle is timed on the host cores
as cpu_baseline.  Prints one JSON line.

--profile KERNEL runs only that kernel's launch loop (for rocprofv3 counters);
--profile copy runs a plain fp32->fp16 conversion of known size, the
reference that scales the FETCH_SIZE / WRITE_SIZE counters to bytes.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E datasheet peak
MALL_BYTES = 256 << 20          # Infinity Cache
ROTATE_BYTES = 512 << 20        # bytes touched per rotation of copies
METRIC = "µs/GEMV and weight-stream GB/s as % of HBM peak, batch 1, 4096×12288"
ROWS, COLS = 4096, 12288


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=400)
    p.add_argument("--warmup", type=int, default=40)
    p.add_argument("--copies", type=int, default=0, help="blob copies (0: enough for 512 MB)")
    p.add_argument("--no-arms", action="store_true")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--profile", choices=["leech", "fp16", "bpdq", "trellis", "copy"], default=None)
    return p.parse_args()


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def copies_for(nbytes, requested):
    if requested:
        return requested
    return max(2, -(-ROTATE_BYTES // max(nbytes, 1)))


class Timed:
    """K launches of fn(i) on the current stream, enqueued while the GPU is
    held busy by a bounded spin kernel (torch.cuda._sleep), so the host's
    submission time never shows up on the GPU timeline.
      region_ms:  events around K back-to-back launches (whole-job time)
      per-launch: a second pass with an event pair around every launch."""

    cycles_per_ms = None

    def __init__(self, torch, fn, steps, warmup):
        self.torch = torch
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        st = torch.cuda.current_stream()
        hold = self._hold_cycles(torch, 3.0 + steps * 0.06)
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(hold)
        r0.record(st)
        for i in range(steps):
            fn(i)
        r1.record(st)
        torch.cuda.synchronize()
        self.region_ms = r0.elapsed_time(r1)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        torch.cuda._sleep(hold)
        for i in range(steps):
            ev[i][0].record(st)
            fn(i)
            ev[i][1].record(st)
        torch.cuda.synchronize()
        per = sorted(a.elapsed_time(b) for a, b in ev)
        self.kernel_ms_mean = sum(per) / len(per)
        self.kernel_ms_median = per[len(per) // 2]
        self.kernel_ms_min = per[0]
        self.kernel_ms_max = per[-1]
        self.steps = steps

    @classmethod
    def _hold_cycles(cls, torch, ms):
        if cls.cycles_per_ms is None:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n = 1 << 22
            torch.cuda._sleep(n)  # warm
            torch.cuda.synchronize()
            a.record()
            torch.cuda._sleep(n)
            b.record()
            torch.cuda.synchronize()
            cls.cycles_per_ms = n / max(a.elapsed_time(b), 1e-3)
        return int(cls.cycles_per_ms * ms)


def dev_copies(torch, blob_np, n):
    """n device copies of a byte blob, each starting on a 256-byte boundary."""
    nb = blob_np.size
    stride = (nb + 255) // 256 * 256
    buf = torch.empty((n, stride), dtype=torch.uint8, device="cuda")
    src = torch.from_numpy(blob_np).to("cuda")
    for i in range(n):
        buf[i, :nb].copy_(src)
    return buf


def to_dev(torch, a):
    import numpy as np
    view = {np.dtype(np.uint16): np.int16, np.dtype(np.uint32): np.int32,
            np.dtype(np.uint8): np.uint8, np.dtype(np.int8): np.int8}[a.dtype]
    return torch.from_numpy(np.ascontiguousarray(a).view(view)).to("cuda")


def kernel_sha():
    h = hashlib.sha256()
    for f in ("lvq_gemv.hip", "common.h", "layout.h"):
        h.update(open(os.path.join(ROOT, "dequant_gemv_lvq_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profile():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "leech_gemv_4096x12288_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_sha:\s*([0-9a-f]+)", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != kernel_sha():
        return None
    return float(t.group(1))


# ---------------------------------------------------------------------- arms

def leech_logical_bytes(rows, cols):
    """Algorithmic weight bytes of the Leech layout: 14 per 24-weight block
    (16-bit class, 24-bit sign plane, three 24-bit rank planes), 2 per row for
    the scale and 2 per unquantized tail column."""
    nb, tau = cols // 24, cols % 24
    return rows * (14 * nb + 2 + 2 * tau)


def leech_setup(lvq, synth):
    t0 = time.perf_counter()
    d = synth.leech_matrix(ROWS, COLS, 4)
    x = synth.activations(COLS, 1, 4, rows=ROWS)
    blob = lvq.expand(d["coords"], d["scale"], d["tail"], ROWS, COLS)
    log("leech workload drawn and expanded in %.1fs" % (time.perf_counter() - t0))
    return d, x, blob, leech_logical_bytes(ROWS, COLS)


def arm_record(tm, nbytes_alg, copies):
    us = tm.kernel_ms_mean * 1e3
    gbps = nbytes_alg / (us * 1e-6) / 1e9
    return {
        "us_per_gemv": round(us, 3),
        "us_median": round(tm.kernel_ms_median * 1e3, 3),
        "us_min": round(tm.kernel_ms_min * 1e3, 3),
        "us_max": round(tm.kernel_ms_max * 1e3, 3),
        "gbps": round(gbps, 1),
        "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBS, 2),
        "region_us_per_launch": round(tm.region_ms * 1e3 / tm.steps, 3),
        "weight_bytes": int(nbytes_alg),
        "copies": copies,
    }


def run_arm(torch, launch, nbytes_alg, copies, steps, warmup):
    return arm_record(Timed(torch, launch, steps, warmup), nbytes_alg, copies)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(rows would shard with one all-gather of y); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import dequant_gemv_lvq_amd as lvq
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    props = torch.cuda.get_device_properties(0)
    log("device %s (%s), %d CUs" % (props.name, getattr(props, "gcnArchName", "?"),
                                    props.multi_processor_count))

    # ------------------------------------------------ plain copy (counter scale)
    if args.profile == "copy":
        n = 64 << 20
        a = torch.randn(n, device="cuda", dtype=torch.float32)
        b = torch.empty(n, device="cuda", dtype=torch.float16)
        for _ in range(max(args.steps, 1)):
            b.copy_(a)
        torch.cuda.synchronize()
        log("copy: %d fp32 -> fp16 elements per launch (reads %d B, writes %d B)"
            % (n, 4 * n, 2 * n))
        return

    steps, warmup = args.steps, args.warmup
    arms = {}

    # ------------------------------------------------ Leech (the step)
    if args.profile in (None, "leech"):
        d, x, blob, alg = leech_setup(lvq, synth)
        n = copies_for(blob.size, args.copies)
        bufs = dev_copies(torch, blob, n)
        xd = to_dev(torch, x)
        yd = torch.empty((1, ROWS), dtype=torch.float32, device="cuda")

        def leech_launch(i):
            lvq.gemv(bufs[i % n], ROWS, COLS, xd, yd, 1)

        if args.profile == "leech":
            for i in range(steps):
                leech_launch(i)
            torch.cuda.synchronize()
            log("profile leech: %d launches" % steps)
            return
        leech = run_arm(torch, leech_launch, alg, n, steps, warmup)
        torch.cuda.synchronize()
        y_timed = yd.cpu().numpy()  # output of the last timed launch
        leech.update({
            "bits_per_weight": round(8 * alg / (ROWS * COLS), 4),
            "blob_bytes": int(blob.size),
        })
        arms["leech"] = leech
        del bufs
        torch.cuda.empty_cache()

    # ------------------------------------------------ comparison arms
    if not args.no_arms or args.profile in ("fp16", "bpdq", "trellis"):
        if args.profile in (None, "fp16"):
            wb = synth.dense_matrix(ROWS, COLS, cfg=2)
            xf = synth.activations(COLS, 1, 2, rows=ROWS)
            nbytes = wb.size * 2
            n = copies_for(nbytes, 0)
            buf = torch.empty((n, ROWS * COLS), dtype=torch.int16, device="cuda")
            src = to_dev(torch, wb.reshape(-1))
            for i in range(n):
                buf[i].copy_(src)
            xd = to_dev(torch, xf)
            yd = torch.empty((1, ROWS), dtype=torch.float32, device="cuda")
            fn = lambda i: lvq.fp16_gemv(buf[i % n], ROWS, COLS, xd, yd, 1)  # noqa: E731
            if args.profile == "fp16":
                for i in range(steps):
                    fn(i)
                torch.cuda.synchronize()
                return
            arms["fp16"] = run_arm(torch, fn, nbytes, n, steps, warmup)
            arms["fp16"]["bits_per_weight"] = 16.0
            arms["fp16"]["shape"] = [ROWS, COLS]
            del buf
            torch.cuda.empty_cache()

        if args.profile in (None, "bpdq"):
            R2 = K2 = 4096
            db = synth.bpdq_matrix(R2, K2)
            xb = synth.activations(K2, 1, 2, rows=R2)
            nbytes = db["codes"].size * 4 + db["coeffs"].size * 2
            n = copies_for(nbytes, 0)
            codes = [to_dev(torch, db["codes"]) for _ in range(n)]
            coeffs = [to_dev(torch, db["coeffs"]) for _ in range(n)]
            xd = to_dev(torch, xb)
            yd = torch.empty((1, R2), dtype=torch.float32, device="cuda")
            fn = lambda i: lvq.bpdq_gemv(codes[i % n], coeffs[i % n], R2, K2, xd, yd, 1)  # noqa
            if args.profile == "bpdq":
                for i in range(steps):
                    fn(i)
                torch.cuda.synchronize()
                return
            arms["bpdq"] = run_arm(torch, fn, nbytes, n, steps, warmup)
            arms["bpdq"]["bits_per_weight"] = round(8 * nbytes / (R2 * K2), 4)
            arms["bpdq"]["shape"] = [R2, K2]
            del codes, coeffs
            torch.cuda.empty_cache()

        if args.profile in (None, "trellis"):
            dt = synth.trellis_matrix(ROWS, COLS)
            xt = synth.activations(COLS, 1, 4, rows=ROWS)
            nbytes = dt["bits"].size * 4 + dt["scale"].size * 2 + dt["table"].size * 2
            n = copies_for(nbytes, 0)
            bits = [to_dev(torch, dt["bits"]) for _ in range(n)]
            table = to_dev(torch, dt["table"])
            scale = to_dev(torch, dt["scale"])
            xd = to_dev(torch, xt)
            yd = torch.empty((1, ROWS), dtype=torch.float32, device="cuda")
            fn = lambda i: lvq.trellis_gemv(bits[i % n], table, scale, ROWS, COLS, xd, yd, 1)  # noqa
            if args.profile == "trellis":
                for i in range(steps):
                    fn(i)
                torch.cuda.synchronize()
                return
            arms["trellis"] = run_arm(torch, fn, nbytes, n, steps, warmup)
            arms["trellis"]["bits_per_weight"] = round(8 * nbytes / (ROWS * COLS), 4)
            arms["trellis"]["shape"] = [ROWS, COLS]
            del bits
            torch.cuda.empty_cache()

    leech = arms["leech"]
    if "fp16" in arms:
        leech["pct_fp16_control"] = round(100 * leech["gbps"] / arms["fp16"]["gbps"], 1)

    # ------------------------------------------------ CPU baseline: the oracle
    cpu = None
    if not args.no_cpu:
        from oracle import gemv as og
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        except Exception:
            threads = 1
        passes, t_cpu = 0, 0.0
        while t_cpu < 10.0 and passes < 200:
            t0 = time.perf_counter()
            w = og.leech_weights(d["coords"], d["scale"], d["tail"], COLS)
            y64, bound = og.gemv(w, x)
            t_cpu += time.perf_counter() - t0
            passes += 1
            del w
        leech["parity_max_ratio"] = round(og.check(y_timed, y64, bound), 5)
        cpu = {"value": round(alg * passes / t_cpu / 1e9, 3), "unit": "GB/s",
               "cores": int(threads), "kind": "oracle",
               "sample": "the full 4096x12288 Leech matrix, f64 reconstruction + matvec + "
                         "per-row bound, %d passes in %.1fs (%.1f ms per GEMV)"
                         % (passes, t_cpu, 1e3 * t_cpu / passes)}

    value = leech["weight_bytes"] / (leech["region_us_per_launch"] * 1e-6) / 1e9
    region_gbps = round(value, 1)
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(leech["region_us_per_launch"] / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "Leech GEMV 4096x12288 (down_proj-shaped), batch 1, "
                               "shells 2..6 with P(m)~2^-m, LP3 layout 4.668 b/w",
                   "rows": ROWS, "cols": COLS, "batch": 1, "copies": leech["copies"],
                   "device": props.name, "torch": torch.__version__},
        "roofline": {"bound": "hbm", "achieved": region_gbps, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(region_gbps / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profile()},
        "cpu_baseline": cpu,
        "us_per_gemv": leech["us_per_gemv"],
        "arms": arms,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
