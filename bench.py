#!/usr/bin/env python3
"""Benchmark of the Leech-lattice dequantize-plus-matvec hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--trials T]
                    [--no-arms] [--no-stack] [--no-cpu] [--profile KERNEL [--profile-batch B]]

A step is one batch-1 Leech GEMV y = W x at 4096 x 12288 (down_proj-shaped,
shells 2..6 with P(m) ~ 2^-m), the workload the metric is quoted on, on
seeded synthetic inputs already resident in HBM.  W warm-up launches, then T
trials of K back-to-back launches on one stream, each trial bracketed by HIP
events on that stream; the median trial gives `value` (weight-stream GB/s on
the layout's algorithmic bytes) and `roofline.achieved`.  Every timed
workload rotates over enough copies of its weights to touch more than 512 MB,
so the 256 MB Infinity Cache never serves them.

Beside the headline the JSON line carries one record per arm x config x
batch (Leech at every config shape and batch 1 and 4, the BPDQ and bitshift-
trellis arms, the fp16 dense control at the same shapes, the rotation and
the rotated GEMV, the shape-gain GEMV, the LP2, LP2X, direct and one-hot
layouts, load-time unfolding of 48-bit words), each with its
fraction of a read-only streaming kernel over the same bytes and rotation
(lvq_stream_read), the metric shape captured in a HIP graph, the Qwen3-8B
Leech stack of 252 GEMVs (GEMV-only time on precomputed inputs, and the
dependent chain with its renormalisations), and the f64 oracle timed on the
host cores (cpu_baseline: all cores; the per-record oracle times: one core
and all cores, reconstruction and matvec separately).  Parity of every
kernel at these shapes is the GPU test suite's job; the cpu_baseline leg,
which runs the oracle on the timed workload anyway, also reports the largest
error ratio of the timed Leech output.

--profile KERNEL runs only that kernel's timed launches (for rocprofv3: the
same warm-up and trials of back-to-back launches; the Leech kinds at
4096 x 12288, batch --profile-batch);
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

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E datasheet peak
ROTATE_BYTES = 512 << 20        # bytes touched per rotation of copies (> 256 MB MALL)
METRIC = "µs/GEMV and weight-stream GB/s as % of HBM peak, batch 1, 4096×12288"
ROWS, COLS = 4096, 12288
QWEN_LAYERS = 36


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=400)
    p.add_argument("--warmup", type=int, default=40)
    p.add_argument("--trials", type=int, default=7)
    p.add_argument("--no-arms", action="store_true")
    p.add_argument("--no-stack", action="store_true")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--stack-layers", type=int, default=QWEN_LAYERS)
    p.add_argument("--profile", choices=["leech", "noweights", "direct", "fp16", "bpdq", "trellis", "copy"], default=None)
    p.add_argument("--profile-batch", type=int, default=1, choices=[1, 2, 3, 4])
    p.add_argument("--ceiling", action="store_true",
                   help="sweep the launch shape of a plain read of the headline's bytes "
                        "(the streaming ceiling) and time a device-to-device copy of them")
    p.add_argument("--ceiling-bytes", type=int, default=None)
    return p.parse_args()


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def cpu_share():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ---------------------------------------------------------------- stack workers

def _stack_worker(job):
    """(layer, matrix) -> the expanded Leech blob of that Qwen3-8B matrix."""
    import dequant_gemv_lvq_amd as lvq
    import synth
    layer, matrix = job
    d = synth.qwen3_8b_matrix(layer, matrix)
    blob = lvq.expand(d["coords"], d["scale"], d["tail"], d["rows"], d["cols"])
    return layer, matrix, d["rows"], d["cols"], blob


def _stack_check(job):
    """The oracle leg's check of one stack GEMV, run in a worker process:
    (layer, matrix, x fp16 bits, y) -> (layer, matrix, parity ratio)."""
    import synth
    from oracle import gemv as og
    layer, matrix, x_bits, y = job
    d = synth.qwen3_8b_matrix(layer, matrix)
    y64, bound = og.gemv(og.leech_weights(d["coords"], d["scale"], d["tail"], d["cols"]), x_bits)
    return layer, matrix, og.check(y, y64, bound)


def start_stack_pool(layers):
    """Draw and expand the stack in worker processes, forked before the GPU is
    touched; results stream back while the single-matrix records run."""
    import multiprocessing as mp
    import synth
    jobs = [(li, mi) for li in range(layers) for mi in range(len(synth.QWEN3_8B_MATRICES))]
    pool = mp.get_context("fork").Pool(cpu_share())
    return pool, pool.imap_unordered(_stack_worker, jobs, chunksize=1), len(jobs)


# ---------------------------------------------------------------- timing

class Timed:
    """`trials` runs of `steps` back-to-back launches fn(i) on the current
    stream, each bracketed by events on that stream.  A bounded spin kernel
    (torch.cuda._sleep) holds the GPU while a trial is enqueued, so host
    submission never shows on the GPU timeline.  That is checked: if the GPU
    has already passed the trial's start event when the last launch has been
    enqueued, the spin ended first and the GPU may have waited for the host,
    so the trial is run again with twice the hold (at most `retries` times,
    the hold at most 2^retries times the first; `redone` counts these over
    the process).  Trials of more than about a thousand launches (the stack
    records) cannot pass the check: the host's enqueue then blocks until the
    GPU has completed earlier launches, so they run with retries=0."""

    cycles_per_ms = None
    redone = 0

    def __init__(self, torch, fn, steps, warmup, trials, enqueue_ms=0.04, retries=3):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        st = torch.cuda.current_stream()
        hold_ms = 2.0 + steps * enqueue_ms
        max_hold_ms = hold_ms * (1 << retries)
        per = []
        for t in range(trials):
            for attempt in range(retries + 1):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda._sleep(self._hold_cycles(torch, hold_ms))
                a.record(st)
                for i in range(steps):
                    fn(t * steps + i)
                b.record(st)
                drained = a.query()  # the spin ended before the enqueue did
                torch.cuda.synchronize()
                if not drained or attempt == retries:
                    break
                Timed.redone += 1
                hold_ms = min(2 * hold_ms, max_hold_ms)
            per.append(a.elapsed_time(b) * 1e3 / steps)
        per.sort()
        self.us = per
        self.median = per[len(per) // 2]

    @classmethod
    def _hold_cycles(cls, torch, ms):
        if cls.cycles_per_ms is None:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n = 1 << 22
            torch.cuda._sleep(n)
            torch.cuda.synchronize()
            a.record()
            torch.cuda._sleep(n)
            b.record()
            torch.cuda.synchronize()
            cls.cycles_per_ms = n / max(a.elapsed_time(b), 1e-3)
        return int(cls.cycles_per_ms * ms)


def copies_for(nbytes):
    return max(2, -(-ROTATE_BYTES // max(nbytes, 1)))


def dev_copies(torch, arr, n):
    """n device copies of a numpy array's bytes, each on a 256-byte boundary."""
    import numpy as np
    raw = np.ascontiguousarray(arr).view(np.uint8).reshape(-1)
    stride = (raw.size + 255) // 256 * 256
    buf = torch.empty((n, stride), dtype=torch.uint8, device="cuda")
    src = torch.from_numpy(raw).to("cuda")
    for i in range(n):
        buf[i, :raw.size].copy_(src)
    return buf


def to_dev(torch, a):
    import numpy as np
    view = {np.dtype(np.uint16): np.int16, np.dtype(np.uint32): np.int32,
            np.dtype(np.uint8): np.uint8, np.dtype(np.int8): np.int8}[a.dtype]
    return torch.from_numpy(np.ascontiguousarray(a).view(view)).to("cuda")


def code_text(src):
    """Source text without comments and with whitespace collapsed: what the
    compiler sees, so that a comment edit does not stale a profile."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return re.sub(r"\s+", " ", src).strip()


def kernel_sha():
    h = hashlib.sha256()
    for f in ("lvq_gemv.hip", "common.h", "layout.h", "rotate_dev.h"):
        src = open(os.path.join(ROOT, "dequant_gemv_lvq_amd", "csrc", f)).read()
        h.update(code_text(src).encode())
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


# ---------------------------------------------------------------- algorithmic bytes

def leech_bytes(rows, cols):
    """14 B per 24-weight block (16-bit class, sign plane, three rank planes),
    2 B per row for the scale, 2 B per unquantized tail column."""
    nb, tau = cols // 24, cols % 24
    return rows * (14 * nb + 2 + 2 * tau)


def lp2_bytes(rows, cols):
    """LP2: 12 B per 24-weight block (ranks, signs and class), 2 B per row
    for the scale, 2 B per unquantized tail column."""
    nb, tau = cols // 24, cols % 24
    return rows * (12 * nb + 2 + 2 * tau)


def direct_bytes(rows, cols):
    """Direct layout: 16 B per 24-weight block (parity, three magnitude bits
    and a sign per coordinate, no class), 2 B per row for the scale, 2 B per
    unquantized tail column."""
    nb, tau = cols // 24, cols % 24
    return rows * (16 * nb + 2 + 2 * tau)


def onehot_bytes(rows, cols):
    """One-hot layout: 16 B of rank-indicator masks and signs plus a 2 B class
    id per 24-weight block, 2 B per row for the scale, 2 B per tail column."""
    nb, tau = cols // 24, cols % 24
    return rows * (18 * nb + 2 + 2 * tau)


def bpdq_bytes(rows, cols):
    return (cols // 16) * rows * 4 + (cols // 256) * 3 * rows * 2


def trellis_bytes(rows, cols):
    return rows * cols // 4 + 2 * rows + 2 * 65536


def fp16_bytes(rows, cols):
    return 2 * rows * cols


# ---------------------------------------------------------------- oracle leg

class ParityGateError(RuntimeError):
    pass


class OracleLeg:
    """The cpu_baseline leg: the f64 oracle (test infrastructure) on the host
    cores.  Every arm's GPU output at the shape and launch it is timed in is
    checked here before that arm is timed: |y - y_f64| <= 1e-4 * sum_c |w x|
    per output (activation rotations: one fp16 ulp plus 1e-5 of the term
    magnitudes), decoded lattice points and unfolded words bit-exact.  The
    first failure stops the run (non-zero exit, no result line).  The same leg
    times the oracle on the headline workload (cpu_baseline)."""

    def __init__(self, enabled):
        self.enabled = enabled
        self.ratios = {}

    def _done(self, name, r, bar=1.0):
        self.ratios[name] = round(float(r), 5)
        if not r <= bar:
            raise ParityGateError("%s: parity ratio %.4g exceeds %.3g" % (name, r, bar))
        return r

    def weights(self, name, w_fn, x, y):
        """w_fn() -> f64 W [rows][cols]; x fp16 bits [batch][cols]; y GPU fp32."""
        if not self.enabled:
            return None
        from oracle import gemv as og
        y64, bound = og.gemv(w_fn(), x)
        return self._done(name, og.check(y, y64, bound))

    def leech(self, name, d, x, y):
        if not self.enabled:
            return None
        from oracle import gemv as og
        return self.weights(name, lambda: og.leech_weights(d["coords"], d["scale"], d["tail"],
                                                          d["cols"]), x, y)

    def fp16(self, name, wb, rows, cols, x, y):
        if not self.enabled:
            return None
        from oracle import gemv as og
        return self.weights(name, lambda: og.fp16_weights(wb, rows, cols), x, y)

    def bpdq(self, name, d, x, y):
        if not self.enabled:
            return None
        from oracle import gemv as og
        return self.weights(name, lambda: og.bpdq_weights(d["codes"], d["coeffs"], d["rows"],
                                                          d["cols"]), x, y)

    def trellis(self, name, d, x, y):
        if not self.enabled:
            return None
        from oracle import gemv as og
        return self.weights(name, lambda: og.trellis_weights(d["bits"], d["table"], d["scale"],
                                                             d["rows"], d["cols"]), x, y)

    def bitexact(self, name, ok):
        self.ratios[name] = bool(ok)
        if not ok:
            raise ParityGateError("%s: not bit-exact" % name)
        return ok

    def rotation(self, name, x, n, m, words, q, y_bits):
        if not self.enabled:
            return None
        from oracle import rotate as orot
        y64, bound = orot.rotate(x, n, m, words, q)
        return self._done(name, orot.rotate_check(y_bits, y64, bound))

    def unfold(self, name, words, coords, gains):
        if not self.enabled:
            return None
        from oracle import index as oi
        ok = True
        for i, w in enumerate(words):
            idx, g = oi.split_word(int(w))
            ok &= bool(np.array_equal(coords[i], oi.unrank(idx))) and int(gains[i]) == g
        return self.bitexact(name, ok)

    def gain(self, name, d, gbits, gains, x, y):
        if not self.enabled:
            return None
        from oracle import index as oi
        return self.weights(name, lambda: oi.shape_gain_weights(
            d["coords"], gbits, d["scale"], gains, d["tail"], d["cols"]), x, y)

    def worst(self):
        r = [v for v in self.ratios.values() if not isinstance(v, bool)]
        return max(r) if r else None


# ---------------------------------------------------------------- records

class Bench:
    def __init__(self, torch, lvq, args, props, leg):
        self.torch, self.lvq, self.args, self.props = torch, lvq, args, props
        self.leg = leg
        self.sink = torch.zeros(lvq.STREAM_SINK_WORDS, dtype=torch.int32, device="cuda")
        self.ceiling = {}

    def first(self, fn, yd):
        """One launch of the timed call (copy 0), its output on the host: what
        the oracle leg checks before the call is timed."""
        fn(0)
        self.torch.cuda.synchronize()
        return yd.cpu().numpy()

    def time(self, fn, steps=None):
        a = self.args
        return Timed(self.torch, fn, steps or a.steps, a.warmup, a.trials)

    def stream_ceiling(self, nbytes):
        """Median µs of lvq_stream_read over nbytes with the same rotation."""
        if nbytes in self.ceiling:
            return self.ceiling[nbytes]
        torch, lvq = self.torch, self.lvq
        n = copies_for(nbytes)
        stride = (nbytes + 255) // 256 * 256
        buf = torch.empty((n, stride), dtype=torch.uint8, device="cuda")
        buf.fill_(0x5A)
        nb4 = nbytes // 4 * 4
        tm = self.time(lambda i: lvq.stream_read(buf[i % n], nb4, self.sink))
        del buf
        self.ceiling[nbytes] = tm.median
        return tm.median

    def record(self, arm, cfg, rows, cols, batch, nbytes, copies, tm, **extra):
        us = tm.median
        gbps = nbytes / (us * 1e-6) / 1e9
        ceil = self.stream_ceiling(nbytes)
        r = {
            "arm": arm, "cfg": cfg, "R": rows, "K": cols, "batch": batch,
            "bytes_weights": int(nbytes), "bytes_x": 2 * cols * batch, "bytes_y": 4 * rows * batch,
            "bits_per_weight": round(8.0 * nbytes / (rows * cols), 4),
            "us_median": round(us, 3), "us_min": round(tm.us[0], 3), "us_max": round(tm.us[-1], 3),
            "gbps": round(gbps, 1), "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBS, 2),
            "stream_ceiling_us": round(ceil, 3), "pct_stream_ceiling": round(100 * ceil / us, 1),
            "copies": copies, "reps": self.args.steps, "trials": self.args.trials, "graph": False,
        }
        r.update(extra)
        note = ""
        if "us_noweights" in extra:
            note = "  (no weights %.3f us)" % extra["us_noweights"]
        if "us_rotate_then_gemv" in extra:
            note = "  (rotate + gemv: %.3f us)" % extra["us_rotate_then_gemv"]
        log("%-8s cfg%s %5dx%-5d b%d: %7.3f us  %7.1f GB/s  %5.1f%% peak  %5.1f%% of stream%s"
            % (arm, cfg, rows, cols, batch, us, gbps, r["pct_hbm_peak"], r["pct_stream_ceiling"],
               note))
        return r

    # one Leech matrix at one shape and batch
    def leech(self, cfg, rows, cols, batch, d=None, keep=False):
        import synth
        torch, lvq = self.torch, self.lvq
        if d is None:
            d = synth.leech_matrix(rows, cols, cfg)
        x = synth.activations(cols, batch, cfg, rows=rows)
        blob = lvq.expand(d["coords"], d["scale"], d["tail"], rows, cols)
        nbytes = leech_bytes(rows, cols)
        n = copies_for(blob.size)
        bufs = dev_copies(torch, blob, n)
        xd = to_dev(torch, x)
        yd = torch.empty((batch, rows), dtype=torch.float32, device="cuda")
        shape = "%dx%d b%d" % (rows, cols, batch)
        gate = {}
        if keep:
            # the bit-exact gate: the timed blob decodes to the input points on
            # the GPU, and they re-expand to the same blob
            dec = torch.empty((rows, cols // 24, 24), dtype=torch.int8, device="cuda")
            lvq.decode(bufs[0], rows, cols, dec)
            got = dec.cpu().numpy()
            gate["bitexact"] = self.leg.bitexact("lvq_decode " + shape, np.array_equal(
                got, d["coords"]) and np.array_equal(
                lvq.expand(got, d["scale"], d["tail"], rows, cols), blob))
            del dec
        fn = lambda i: lvq.gemv(bufs[i % n], rows, cols, xd, yd, batch)  # noqa: E731
        gate["parity_max_ratio"] = self.leg.leech("lvq_gemv cfg%d %s" % (cfg, shape), d, x,
                                                  self.first(fn, yd))
        tm = self.time(fn)
        # the no-weights control: the same launch reading no weight bytes
        y0 = torch.empty_like(yd)
        t0 = self.time(lambda i: lvq.gemv_noweights(bufs[i % n], rows, cols, xd, y0, batch))
        rec = self.record("leech", cfg, rows, cols, batch, nbytes, n, tm,
                          blob_bytes=int(blob.size), us_noweights=round(t0.median, 3),
                          pct_time_noweights=round(100 * t0.median / tm.median, 1), **gate)
        out = (rec, d, x) if keep else rec
        if keep:
            self.graph_us = self.graph(fn)
        del bufs
        torch.cuda.empty_cache()
        return out

    def graph(self, fn):
        """Median µs per launch of `steps` launches captured in one HIP graph
        and replayed (the same rotation); None if capture is unavailable."""
        torch = self.torch
        steps = self.args.steps
        try:
            g = torch.cuda.CUDAGraph()
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                fn(0)
                torch.cuda.synchronize()
                with torch.cuda.graph(g, stream=s):
                    for i in range(steps):
                        fn(i)
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            per = []
            for _ in range(self.args.trials):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                g.replay()
                b.record()
                torch.cuda.synchronize()
                per.append(a.elapsed_time(b) * 1e3 / steps)
            per.sort()
            return round(per[len(per) // 2], 3)
        except Exception as e:  # graph capture is optional context
            log("graph capture unavailable: %s" % e)
            return None

    def fp16(self, cfg, rows, cols, batch):
        import synth
        torch, lvq = self.torch, self.lvq
        wb = synth.dense_matrix(rows, cols, cfg=2)
        x = synth.activations(cols, batch, 2, rows=rows)
        nbytes = fp16_bytes(rows, cols)
        n = copies_for(nbytes)
        bufs = dev_copies(torch, wb, n)
        xd = to_dev(torch, x)
        yd = torch.empty((batch, rows), dtype=torch.float32, device="cuda")
        fn = lambda i: lvq.fp16_gemv(bufs[i % n], rows, cols, xd, yd, batch)  # noqa: E731
        r = self.leg.fp16("fp16_gemv %dx%d b%d" % (rows, cols, batch), wb, rows, cols, x,
                          self.first(fn, yd))
        tm = self.time(fn)
        del bufs
        torch.cuda.empty_cache()
        return self.record("fp16", cfg, rows, cols, batch, nbytes, n, tm, parity_max_ratio=r)

    def bpdq(self, rows, cols, batch):
        import synth
        torch, lvq = self.torch, self.lvq
        d = synth.bpdq_matrix(rows, cols)
        x = synth.activations(cols, batch, 2, rows=rows)
        nbytes = bpdq_bytes(rows, cols)
        n = copies_for(nbytes)
        codes = dev_copies(torch, d["codes"], n)
        coeffs = dev_copies(torch, d["coeffs"], n)
        xd = to_dev(torch, x)
        yd = torch.empty((batch, rows), dtype=torch.float32, device="cuda")
        fn = lambda i: lvq.bpdq_gemv(codes[i % n], coeffs[i % n], rows, cols, xd, yd,  # noqa
                                     batch)
        r = self.leg.bpdq("bpdq_gemv %dx%d b%d" % (rows, cols, batch), d, x, self.first(fn, yd))
        tm = self.time(fn)
        del codes, coeffs
        torch.cuda.empty_cache()
        return self.record("bpdq", 2, rows, cols, batch, nbytes, n, tm, parity_max_ratio=r)

    def trellis(self, rows, cols, batch):
        import synth
        torch, lvq = self.torch, self.lvq
        d = synth.trellis_matrix(rows, cols)
        x = synth.activations(cols, batch, 4, rows=rows)
        nbytes = trellis_bytes(rows, cols)
        n = copies_for(nbytes)
        bits = dev_copies(torch, d["bits"], n)
        table = to_dev(torch, d["table"])
        scale = to_dev(torch, d["scale"])
        xd = to_dev(torch, x)
        yd = torch.empty((batch, rows), dtype=torch.float32, device="cuda")
        fn = lambda i: lvq.trellis_gemv(bits[i % n], table, scale, rows, cols, xd, yd,  # noqa
                                        batch)
        r = self.leg.trellis("trellis_gemv %dx%d b%d" % (rows, cols, batch), d, x,
                             self.first(fn, yd))
        tm = self.time(fn)
        del bits
        torch.cuda.empty_cache()
        return self.record("trellis", 4, rows, cols, batch, nbytes, n, tm, parity_max_ratio=r)

    def unfold(self, nblocks):
        """Load-time unfolding of random 48-bit words (one per 24-weight block)."""
        import numpy as np
        torch, lvq = self.torch, self.lvq
        rng = np.random.default_rng(nblocks)
        ball = 111_043_117_458_001
        words = (rng.integers(0, ball, nblocks, dtype=np.int64).astype(np.uint64) |
                 (rng.integers(0, 2, nblocks).astype(np.uint64) << np.uint64(47)))
        wd = torch.from_numpy(words.view(np.int64)).cuda()
        cd = torch.empty((nblocks, 24), dtype=torch.int8, device="cuda")
        gd = torch.empty(nblocks, dtype=torch.uint8, device="cuda")
        lvq.unfold(wd, nblocks, cd, gd)  # uploads the tables once
        torch.cuda.synchronize()
        pick = np.random.default_rng(1).choice(nblocks, 256, replace=False)
        ok = self.leg.unfold("lvq_unfold %d words (256 sampled)" % nblocks, words[pick],
                             cd.cpu().numpy()[pick], gd.cpu().numpy()[pick])
        tm = Timed(torch, lambda i: lvq.unfold(wd, nblocks, cd, gd), 20, 3, self.args.trials)
        us = tm.median
        rec = {"arm": "unfold", "blocks": nblocks, "weights": 24 * nblocks,
               "us_median": round(us, 1), "us_min": round(tm.us[0], 1),
               "gblocks_per_s": round(nblocks / (us * 1e-6) / 1e9, 3),
               "bytes_in": 8 * nblocks, "bytes_out": 25 * nblocks, "trials": self.args.trials,
               "bitexact_sample": ok}
        log("unfold   %d blocks: %.1f us (%.3f G blocks/s)" % (nblocks, us, rec["gblocks_per_s"]))
        return rec

    def leech_lp2(self, cfg, rows, cols, batch, d=None):
        """The LP2 layout (two rank planes, class in the record) at one shape."""
        import synth
        torch, lvq = self.torch, self.lvq
        if d is None:
            d = synth.leech_matrix(rows, cols, cfg)
        blob = lvq.expand_lp2(d["coords"], d["scale"], d["tail"], rows, cols)
        x = synth.activations(cols, batch, cfg, rows=rows)
        n = copies_for(blob.size)
        bufs = dev_copies(torch, blob, n)
        xd = to_dev(torch, x)
        yd = torch.empty((batch, rows), dtype=torch.float32, device="cuda")
        fn = lambda i: lvq.gemv_lp2(bufs[i % n], rows, cols, xd, yd, batch)  # noqa: E731
        r = self.leg.leech("lvq_gemv_lp2 cfg%d %dx%d b%d" % (cfg, rows, cols, batch), d, x,
                           self.first(fn, yd))
        tm = self.time(fn)
        del bufs
        torch.cuda.empty_cache()
        return self.record("leech_lp2", cfg, rows, cols, batch, lp2_bytes(rows, cols), n, tm,
                           blob_bytes=int(blob.size), parity_max_ratio=r)

    def leech_direct(self, cfg, rows, cols, batch, d=None):
        """The table-free direct layout (|x| = 2e + parity) at one shape."""
        return self._layout("leech_direct", self.lvq.expand_direct, self.lvq.gemv_direct,
                            direct_bytes, cfg, rows, cols, batch, d)

    def leech_onehot(self, cfg, rows, cols, batch, d=None):
        """The one-hot layout (rank-indicator masks) at one shape."""
        return self._layout("leech_onehot", self.lvq.expand_onehot, self.lvq.gemv_onehot,
                            onehot_bytes, cfg, rows, cols, batch, d)

    def _layout(self, arm, expand, gemv, nbytes, cfg, rows, cols, batch, d):
        import synth
        torch = self.torch
        if d is None:
            d = synth.leech_matrix(rows, cols, cfg)
        blob = expand(d["coords"], d["scale"], d["tail"], rows, cols)
        x = synth.activations(cols, batch, cfg, rows=rows)
        n = copies_for(blob.size)
        bufs = dev_copies(torch, blob, n)
        xd = to_dev(torch, x)
        yd = torch.empty((batch, rows), dtype=torch.float32, device="cuda")
        fn = lambda i: gemv(bufs[i % n], rows, cols, xd, yd, batch)  # noqa: E731
        r = self.leg.leech("%s cfg%d %dx%d b%d" % (arm, cfg, rows, cols, batch), d, x,
                           self.first(fn, yd))
        tm = self.time(fn)
        del bufs
        torch.cuda.empty_cache()
        return self.record(arm, cfg, rows, cols, batch, nbytes(rows, cols), n, tm,
                           blob_bytes=int(blob.size), parity_max_ratio=r)

    def leech_lp2x(self, cfg, rows, cols, batch, d=None):
        """LP2 with the exception side channel, decoded in each row's epilogue of
        the same launch, at one shape."""
        import synth
        torch, lvq = self.torch, self.lvq
        if d is None:
            d = synth.leech_matrix(rows, cols, cfg)
        blob, n_exc = lvq.expand_lp2x(d["coords"], d["scale"], d["tail"], rows, cols)
        x = synth.activations(cols, batch, cfg, rows=rows)
        n = copies_for(blob.size)
        bufs = dev_copies(torch, blob, n)
        xd = to_dev(torch, x)
        yd = torch.empty((batch, rows), dtype=torch.float32, device="cuda")
        fn = lambda i: lvq.gemv_lp2x(bufs[i % n], rows, cols, n_exc, xd, yd, batch)  # noqa
        r = self.leg.leech("lvq_gemv_lp2x cfg%d %dx%d b%d" % (cfg, rows, cols, batch), d, x,
                           self.first(fn, yd))
        tm = self.time(fn)
        del bufs
        torch.cuda.empty_cache()
        nbytes = lp2_bytes(rows, cols) + 16 * n_exc + 4 * (rows + 1)
        return self.record("leech_lp2x", cfg, rows, cols, batch, nbytes, n, tm,
                           side_channel_blocks=int(n_exc), blob_bytes=int(blob.size),
                           parity_max_ratio=r)

    def leech_gain(self, rows, cols, batch):
        """The shape-gain GEMV at one shape (random gain bits, two gain levels)."""
        import numpy as np
        import synth
        torch, lvq = self.torch, self.lvq
        d = synth.leech_matrix(rows, cols, 4)
        g = np.random.default_rng(rows).integers(0, 2, (rows, cols // 24)).astype(np.uint8)
        blob = lvq.expand_gain(d["coords"], g, d["scale"], d["tail"], rows, cols)
        x = synth.activations(cols, batch, 4, rows=rows)
        n = copies_for(blob.size)
        bufs = dev_copies(torch, blob, n)
        xd = to_dev(torch, x)
        yd = torch.empty((batch, rows), dtype=torch.float32, device="cuda")
        gains = (0.8125, 1.1875)
        fn = lambda i: lvq.gemv_gain(bufs[i % n], rows, cols, gains[0], gains[1], xd, yd,  # noqa
                                     batch)
        r = self.leg.gain("lvq_gemv_gain %dx%d b%d" % (rows, cols, batch), d, g, gains, x,
                          self.first(fn, yd))
        tm = self.time(fn)
        del bufs
        torch.cuda.empty_cache()
        return self.record("leech_gain", 4, rows, cols, batch, leech_bytes(rows, cols), n, tm,
                           parity_max_ratio=r)

    def rotated_gemv(self, rows, cols, m, batch):
        """Rotation fused into the GEMV against the two launches it replaces."""
        import numpy as np
        import synth
        torch, lvq = self.torch, self.lvq
        d = synth.leech_matrix(rows, cols, 3)
        blob = lvq.expand(d["coords"], d["scale"], d["tail"], rows, cols)
        rng = np.random.default_rng(cols + m)
        x = synth.activations(cols, batch, 3, rows=rows)
        words = rng.integers(0, 1 << 32, (cols + 31) // 32, dtype=np.uint64).astype(np.uint32)
        q = np.linalg.qr(rng.standard_normal((m, m)))[0].astype(np.float32) if m > 1 else None
        n = copies_for(blob.size)
        bufs = dev_copies(torch, blob, n)
        xd, wd = to_dev(torch, x), to_dev(torch, words)
        qd = None if q is None else torch.from_numpy(q).cuda()
        xr = torch.empty((batch, cols), dtype=torch.int16, device="cuda")
        yd = torch.empty((batch, rows), dtype=torch.float32, device="cuda")
        fn = lambda i: lvq.gemv_rotated(bufs[i % n], rows, cols, wd, qd, m, xd, yd,  # noqa
                                        batch)
        # the gate: the rotated input against the f64 rotation, and the fused
        # output against the f64 GEMV on that input
        lvq.rotate(xd, cols, m, wd, qd, xr, batch)
        xr_bits = xr.cpu().numpy().view(np.uint16)
        shape = "%dx%d m%d b%d" % (rows, cols, m, batch)
        r_rot = self.leg.rotation("lvq_rotate (for lvq_gemv_rotated) " + shape, x, cols, m,
                                  words, q, xr_bits)
        r = self.leg.leech("lvq_gemv_rotated " + shape, d, xr_bits, self.first(fn, yd))
        tf = self.time(fn)

        def two(i):
            lvq.rotate(xd, cols, m, wd, qd, xr, batch)
            lvq.gemv(bufs[i % n], rows, cols, xr, yd, batch)
        t2 = Timed(torch, two, self.args.steps, self.args.warmup, self.args.trials, enqueue_ms=0.08)
        del bufs
        torch.cuda.empty_cache()
        return self.record("leech_rot", 3, rows, cols, batch, leech_bytes(rows, cols), n, tf,
                           rot_m=m, us_rotate_then_gemv=round(t2.median, 3),
                           parity_max_ratio=r, rotate_parity_ratio=r_rot)

    def rotate(self, n, m, batch):
        """The activation rotation (H kron Q)(S x) at width n = K m."""
        import numpy as np
        torch, lvq = self.torch, self.lvq
        rng = np.random.default_rng(n + m)
        x = (rng.standard_normal((batch, n)) * 0.5).astype(np.float16).view(np.uint16)
        words = rng.integers(0, 1 << 32, (n + 31) // 32, dtype=np.uint64).astype(np.uint32)
        q = np.linalg.qr(rng.standard_normal((m, m)))[0].astype(np.float32) if m > 1 else None
        xd, wd = to_dev(torch, x), to_dev(torch, words)
        qd = None if q is None else torch.from_numpy(q).cuda()
        yd = torch.empty((batch, n), dtype=torch.int16, device="cuda")
        fn = lambda i: lvq.rotate(xd, n, m, wd, qd, yd, batch)  # noqa: E731
        r = self.leg.rotation("lvq_rotate n%d m%d b%d" % (n, m, batch), x, n, m, words, q,
                              self.first(fn, yd).view(np.uint16))
        tm = self.time(fn)
        us = tm.median
        rec = {"arm": "rotate", "N": n, "m": m, "batch": batch,
               "bytes": 4 * n * batch, "us_median": round(us, 3),
               "us_min": round(tm.us[0], 3), "us_max": round(tm.us[-1], 3),
               "reps": self.args.steps, "trials": self.args.trials, "parity_max_ratio": r}
        log("rotate   n=%5d m=%2d b%d: %7.3f us" % (n, m, batch, us))
        return rec

    # the Qwen3-8B stack: 36 layers x 7 Leech GEMVs
    def load_stack(self, results, njobs):
        torch = self.torch
        t0 = time.perf_counter()
        blobs = {}
        for li, mi, rows, cols, blob in results:
            blobs[(li, mi)] = (rows, cols, to_dev(torch, blob))
        torch.cuda.synchronize()
        log("stack: %d matrices drawn, expanded and uploaded in %.1fs"
            % (njobs, time.perf_counter() - t0))
        return blobs

    def stack(self, blobs, layers, pool):
        import synth
        torch, lvq = self.torch, self.lvq
        total = sum(leech_bytes(r, c) for (r, c, _) in blobs.values())
        ys = {}
        for (li, mi), (rows, cols, _) in blobs.items():
            ys[(li, mi)] = torch.empty((1, rows), dtype=torch.float32, device="cuda")

        def renorm(y):
            v = y.double()
            return ((v - v.mean()) / v.std(unbiased=False)).half().view(torch.int16).contiguous()

        def gemv(li, mi, xin):
            rows, cols, b = blobs[(li, mi)]
            lvq.gemv(b, rows, cols, xin, ys[(li, mi)], 1)
            return ys[(li, mi)]

        h0 = to_dev(torch, synth.activations(4096, 1, 5, key=(0,)))
        inputs = {}

        def chain(record):
            h = h0
            for li in range(layers):
                for mi in (0, 1, 2):
                    if record:
                        inputs[(li, mi)] = h
                    gemv(li, mi, h)
                xo = renorm(ys[(li, 0)])
                if record:
                    inputs[(li, 3)] = xo
                gemv(li, 3, xo)
                xg = renorm(ys[(li, 3)])
                for mi in (4, 5):
                    if record:
                        inputs[(li, mi)] = xg
                    gemv(li, mi, xg)
                xd = renorm(ys[(li, 5)])
                if record:
                    inputs[(li, 6)] = xd
                gemv(li, 6, xd)
                h = renorm(ys[(li, 6)])
            return h

        chain(True)
        torch.cuda.synchronize()
        order = [(li, mi) for li in range(layers) for mi in range(7)]
        # the gate: every GEMV of the chain against the f64 oracle on its own
        # fp16 input, in the worker pool (the oracle leg), before any timing
        worst = None
        if self.leg.enabled and pool is not None:
            t0 = time.perf_counter()
            jobs = [(li, mi, inputs[k].cpu().numpy().view(np.uint16), ys[k].cpu().numpy())
                    for k in order for (li, mi) in [k]]
            ratios = {(li, mi): r for li, mi, r in pool.imap_unordered(_stack_check, jobs)}
            top = max(ratios, key=ratios.get)
            worst = self.leg._done("lvq_gemv stack, worst of %d (layer %d, matrix %d)"
                                   % (len(ratios), top[0], top[1]), ratios[top])
            log("stack: all %d GEMVs within the oracle bound (worst %.3g) in %.1fs"
                % (len(ratios), worst, time.perf_counter() - t0))

        def gemv_only(_):
            for li, mi in order:
                gemv(li, mi, inputs[(li, mi)])

        # q/k/v share their input, and so do gate/up: one launch each
        groups = []
        for li in range(layers):
            groups += [(li, (0, 1, 2)), (li, (3,)), (li, (4, 5)), (li, (6,))]
        fused_args = []
        for li, mis in groups:
            cols = blobs[(li, mis[0])][1]
            fused_args.append(([blobs[(li, mi)][2] for mi in mis],
                               [blobs[(li, mi)][0] for mi in mis], cols, inputs[(li, mis[0])],
                               [ys[(li, mi)] for mi in mis]))

        def fused_only(_):
            for a in fused_args:
                lvq.gemv_fused(*a, 1)

        def noweights_only(_):
            for li, mi in order:
                rows, cols, b = blobs[(li, mi)]
                lvq.gemv_noweights(b, rows, cols, inputs[(li, mi)], ys[(li, mi)], 1)

        gemv_only(0)
        torch.cuda.synchronize()
        y_sep = {k: v.clone() for k, v in ys.items()}
        fused_only(0)
        torch.cuda.synchronize()
        fused_same = all(torch.equal(ys[k].view(torch.int32), y_sep[k].view(torch.int32))
                         for k in ys)
        del y_sep

        # host enqueue time per pass: ~252 launches (GEMV only), ~1000 with the
        # renormalisation ops; the hold covers it
        tm = Timed(torch, gemv_only, 5, 2, self.args.trials, enqueue_ms=len(order) * 0.02,
                   retries=0)
        tf = Timed(torch, fused_only, 5, 2, self.args.trials, enqueue_ms=len(groups) * 0.08,
                   retries=0)
        t0 = Timed(torch, noweights_only, 5, 2, self.args.trials, enqueue_ms=len(order) * 0.02,
                   retries=0)
        tc = Timed(torch, lambda _: chain(False), 3, 1, self.args.trials,
                   enqueue_ms=len(order) * 0.08, retries=0)
        us = tm.median  # µs per pass over all GEMVs
        rec = {
            "arm": "leech", "cfg": 5, "model": "Qwen3-8B-shaped Leech stack, random init",
            "layers": layers, "gemvs": len(order),
            "bytes_weights": int(total), "bits_per_weight": round(
                8.0 * total / sum(r * c for (r, c, _) in blobs.values()), 4),
            "us_gemv_only": round(us, 1), "us_min": round(tm.us[0], 1), "us_max": round(tm.us[-1], 1),
            "gbps": round(total / (us * 1e-6) / 1e9, 1),
            "pct_hbm_peak": round(100 * total / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
            "us_chain_with_renorm": round(tc.median, 1),
            "launches": len(order), "trials": self.args.trials, "graph": False,
            "us_fused": round(tf.median, 1), "launches_fused": len(groups),
            "fused_speedup": round(us / tf.median, 4), "fused_bit_equal": bool(fused_same),
            "gbps_fused": round(total / (tf.median * 1e-6) / 1e9, 1),
            "us_noweights": round(t0.median, 1),
            "pct_time_noweights": round(100 * t0.median / us, 1),
            "parity_max_ratio": worst, "parity_checked_gemvs": len(order) if worst is not None else 0,
        }
        log("stack: %d GEMVs %.1f us (%.1f GB/s, %.1f%% peak); chain with renorm %.1f us"
            % (len(order), us, rec["gbps"], rec["pct_hbm_peak"], tc.median))
        log("stack: fused %d launches %.1f us (x%.3f, bit-equal %s); no-weights %.1f us"
            % (len(groups), tf.median, rec["fused_speedup"], fused_same, t0.median))
        del blobs, inputs, ys
        torch.cuda.empty_cache()
        return rec


# ---------------------------------------------------------------- CPU baseline

def cpu_baseline(d, x, per_shape):
    """The oracle as it stands on the host cores: the metric workload for at
    least 10 s with every core (the reported value), one core and all cores
    with the reconstruction and the matvec timed apart, and the other config
    shapes (median of 3 with all cores).  `cores` is the thread count numpy's
    BLAS runs the matvec with (the reconstruction is single-threaded numpy),
    `cores_available` the cores this process may run on."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import gemv as og
    import synth
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    alg = leech_bytes(ROWS, COLS)

    def phases(dd, xx, cols):
        t0 = time.perf_counter()
        w = og.leech_weights(dd["coords"], dd["scale"], dd["tail"], cols)
        t1 = time.perf_counter()
        y64, bound = og.gemv(w, xx)
        t2 = time.perf_counter()
        return t1 - t0, t2 - t1, y64, bound

    passes, t_cpu = 0, 0.0
    while t_cpu < 10.0 and passes < 200:
        a, b, _, _ = phases(d, x, COLS)
        t_cpu += a + b
        passes += 1
    one = []
    with threadpool_limits(limits=1):
        for _ in range(3):
            one.append(phases(d, x, COLS)[:2])
    one.sort(key=lambda p: p[0] + p[1])
    a1, b1 = one[1]
    many = sorted((phases(d, x, COLS)[:2] for _ in range(3)), key=lambda p: p[0] + p[1])[1]
    shapes = {}
    for (cfg, rows, cols) in per_shape:
        dd = synth.leech_matrix(rows, cols, cfg)
        xx = synth.activations(cols, 1, cfg, rows=rows)
        ts = sorted(sum(phases(dd, xx, cols)[:2]) for _ in range(3))
        shapes["cfg%d_%dx%d" % (cfg, rows, cols)] = round(ts[1] * 1e6, 1)
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    cpu = {"value": round(alg * passes / t_cpu / 1e9, 3), "unit": "GB/s",
           "cores": int(threads), "cores_available": int(avail), "kind": "oracle",
           "value_1core": round(alg / (a1 + b1) / 1e9, 4),
           "sample": "the full 4096x12288 Leech matrix, f64 reconstruction + matvec + per-row "
                     "bound, %d passes in %.1fs (%.1f ms per GEMV)"
                     % (passes, t_cpu, 1e3 * t_cpu / passes),
           "oracle_us_1core": {"reconstruct": round(a1 * 1e6, 1), "matvec": round(b1 * 1e6, 1)},
           "oracle_us_ncores": {"reconstruct": round(many[0] * 1e6, 1),
                                "matvec": round(many[1] * 1e6, 1)},
           "oracle_us_per_shape_ncores": shapes}
    return cpu


# ---------------------------------------------------------------- streaming ceiling

def ceiling_sweep(torch, lvq, args, nbytes):
    """The fastest plain read of nbytes: every launch shape of
    lvq_stream_read_geom (workgroup size, workgroups per CU or one trip per
    thread, 16-byte loads in flight, non-temporal or ordinary loads) over the
    same rotation of copies the GEMV records use, beside a device-to-device
    copy of the same bytes (which also writes them) and the launch floor (a
    read of nothing)."""
    n = copies_for(nbytes)
    stride = (nbytes + 255) // 256 * 256
    buf = torch.empty((n, stride), dtype=torch.uint8, device="cuda")
    buf.fill_(0x5A)
    sink = torch.zeros(lvq.STREAM_GEOM_SINK_WORDS, dtype=torch.int32, device="cuda")
    nb4 = nbytes // 4 * 4
    rows = []

    def timed(fn):
        return Timed(torch, fn, args.steps, args.warmup, args.trials)

    for threads in (256, 512, 1024):
        for wpc in (0, 1, 2, 4, 8):
            for unroll in (1, 2, 4, 8):
                for nt in (1, 0):
                    try:
                        lvq.stream_read_geom(buf[0], nb4, sink, threads, wpc, unroll, nt)
                    except lvq.LvqError:
                        continue
                    tm = timed(lambda i: lvq.stream_read_geom(buf[i % n], nb4, sink, threads,
                                                              wpc, unroll, nt))
                    rows.append({"threads": threads, "wgs_per_cu": wpc, "unroll": unroll,
                                 "nontemporal": nt, "us": round(tm.median, 3),
                                 "us_min": round(tm.us[0], 3)})
                    log("read %4d thr %d/CU u%d nt%d: %.3f us" % (threads, wpc, unroll, nt,
                                                                 tm.median))
    tfl = timed(lambda i: lvq.stream_read_geom(buf[0], 0, sink, 256, 1, 1, 1))
    floor = tfl.median
    base = timed(lambda i: lvq.stream_read(buf[i % n], nb4, sink[:lvq.STREAM_SINK_WORDS])).median
    dst = torch.empty((2, stride), dtype=torch.uint8, device="cuda")
    cp = timed(lambda i: dst[i % 2].copy_(buf[i % n])).median
    best = min(rows, key=lambda r: r["us"])
    rec = {"arm": "stream_ceiling", "bytes": nbytes, "copies": n, "reps": args.steps,
           "trials": args.trials, "sweep": rows, "best": best,
           "best_gbps": round(nbytes / (best["us"] * 1e-6) / 1e9, 1),
           "lvq_stream_read_us": round(base, 3), "launch_floor_us": round(floor, 3),
           "launch_floor_us_min": round(tfl.us[0], 3), "timing_trials_redone": Timed.redone,
           "d2d_copy_us": round(cp, 3),
           "d2d_copy_gbps_read_plus_write": round(2 * nbytes / (cp * 1e-6) / 1e9, 1)}
    log("ceiling over %d B: best %.3f us (%s), lvq_stream_read %.3f us, d2d copy %.3f us, "
        "empty launch %.3f us" % (nbytes, best["us"], best, base, cp, floor))
    del buf, dst
    torch.cuda.empty_cache()
    return rec


# ---------------------------------------------------------------- main

def profile_only(torch, lvq, args):
    import synth
    steps = max(args.steps, 1)
    if args.profile == "copy":
        n = 64 << 20
        a = torch.randn(n, device="cuda", dtype=torch.float32)
        b = torch.empty(n, device="cuda", dtype=torch.float16)
        for _ in range(steps):
            b.copy_(a)
        torch.cuda.synchronize()
        log("copy: %d fp32 -> fp16 elements per launch (reads %d B, writes %d B)"
            % (n, 4 * n, 2 * n))
        return
    if args.profile in ("leech", "noweights", "direct"):
        bt = args.profile_batch
        d = synth.leech_matrix(ROWS, COLS, 4)
        ex = lvq.expand_direct if args.profile == "direct" else lvq.expand
        blob = ex(d["coords"], d["scale"], d["tail"], ROWS, COLS)
        n = copies_for(blob.size)
        bufs = dev_copies(torch, blob, n)
        xd = to_dev(torch, synth.activations(COLS, bt, 4, rows=ROWS))
        yd = torch.empty((bt, ROWS), dtype=torch.float32, device="cuda")
        call = {"leech": lvq.gemv, "noweights": lvq.gemv_noweights, "direct": lvq.gemv_direct}[args.profile]
        fn = lambda i: call(bufs[i % n], ROWS, COLS, xd, yd, bt)  # noqa: E731
    elif args.profile == "fp16":
        wb = synth.dense_matrix(ROWS, COLS, cfg=2)
        n = copies_for(wb.size * 2)
        bufs = dev_copies(torch, wb, n)
        xd = to_dev(torch, synth.activations(COLS, 1, 2, rows=ROWS))
        yd = torch.empty((1, ROWS), dtype=torch.float32, device="cuda")
        fn = lambda i: lvq.fp16_gemv(bufs[i % n], ROWS, COLS, xd, yd, 1)  # noqa: E731
    elif args.profile == "bpdq":
        bt = args.profile_batch
        d = synth.bpdq_matrix(4096, 4096)
        n = copies_for(bpdq_bytes(4096, 4096))
        codes = dev_copies(torch, d["codes"], n)
        coeffs = dev_copies(torch, d["coeffs"], n)
        xd = to_dev(torch, synth.activations(4096, bt, 2, rows=4096))
        yd = torch.empty((bt, 4096), dtype=torch.float32, device="cuda")
        fn = lambda i: lvq.bpdq_gemv(codes[i % n], coeffs[i % n], 4096, 4096, xd, yd, bt)  # noqa
    else:
        d = synth.trellis_matrix(ROWS, COLS)
        n = copies_for(trellis_bytes(ROWS, COLS))
        bits = dev_copies(torch, d["bits"], n)
        table, scale = to_dev(torch, d["table"]), to_dev(torch, d["scale"])
        xd = to_dev(torch, synth.activations(COLS, 1, 4, rows=ROWS))
        yd = torch.empty((1, ROWS), dtype=torch.float32, device="cuda")
        fn = lambda i: lvq.trellis_gemv(bits[i % n], table, scale, ROWS, COLS, xd, yd, 1)  # noqa
    # the bench's protocol: warm-up, then trials of back-to-back launches
    # enqueued behind a spin kernel, so the GPU runs them without gaps (a
    # profiler's per-dispatch times then match the bench's events)
    tm = Timed(torch, fn, steps, args.warmup, args.trials)
    log("profile %s: %d warm-up + %d x %d launches, median %.3f us per launch"
        % (args.profile, args.warmup, args.trials, steps, tm.median))


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(rows would shard with one all-gather of y); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import dequant_gemv_lvq_amd as lvq

    pool = None
    if args.profile is None and not args.no_stack and not args.no_arms:
        pool, stack_results, stack_jobs = start_stack_pool(args.stack_layers)
        log("stack: drawing %d matrices in %d worker processes" % (stack_jobs, cpu_share()))

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    props = torch.cuda.get_device_properties(0)
    arch = getattr(props, "gcnArchName", "?")
    log("device %s (%s), %d CUs" % (props.name, arch, props.multi_processor_count))
    if args.profile:
        profile_only(torch, lvq, args)
        return
    if args.ceiling:
        rec = ceiling_sweep(torch, lvq, args, args.ceiling_bytes or leech_bytes(ROWS, COLS))
        rec.update({"device": props.name, "arch": arch, "torch": torch.__version__,
                    "hip": getattr(torch.version, "hip", None)})
        print(json.dumps(rec))
        return

    leg = OracleLeg(enabled=not args.no_cpu)
    if not leg.enabled:
        log("--no-cpu: the oracle leg is off, so no output is checked before it is timed")
    B = Bench(torch, lvq, args, props, leg)
    try:
        out = run(torch, lvq, args, props, arch, B, leg, pool,
                  stack_results if pool is not None else None,
                  stack_jobs if pool is not None else 0)
    except ParityGateError as e:
        log("PARITY GATE FAILED, nothing is reported: %s" % e)
        sys.exit(1)
    finally:
        if pool is not None:
            pool.terminate()
            pool.join()
    print(json.dumps(out))


def run(torch, lvq, args, props, arch, B, leg, pool, stack_results, stack_jobs):
    stack_blobs = None
    if pool is not None:
        # the whole stack is drawn and on the device before anything is
        # timed (busy host cores would slow the enqueueing); the workers stay,
        # idle, for the oracle leg's check of the stack
        stack_blobs = B.load_stack(stack_results, stack_jobs)
    t0 = time.perf_counter()
    head, d, x = B.leech(4, ROWS, COLS, 1, keep=True)
    log("headline done in %.1fs (bit-exact decode %s, parity ratio %s)"
        % (time.perf_counter() - t0, head.get("bitexact"), head.get("parity_max_ratio")))

    records = [head]
    stack = None
    if not args.no_arms:
        records.append(B.fp16(4, ROWS, COLS, 1))
        records.append(B.leech(4, ROWS, COLS, 4, d=d))
        records.append(B.leech(1, 1536, 1536, 1))
        records.append(B.bpdq(4096, 4096, 1))
        records.append(B.bpdq(4096, 4096, 4))
        records.append(B.fp16(2, 4096, 4096, 1))
        for rows in (4096, 12288):
            d3 = __import__("synth").leech_matrix(rows, 4096, 3)
            records.append(B.leech(3, rows, 4096, 1, d=d3))
            records.append(B.leech(3, rows, 4096, 4, d=d3))
        records.append(B.trellis(ROWS, COLS, 1))
        for n, m in ((4096, 1), (12288, 3), (25600, 25)):
            records.append(B.rotate(n, m, 1))
        records.append(B.rotate(12288, 3, 4))
        records.append(B.rotated_gemv(4096, 12288, 3, 1))
        records.append(B.rotated_gemv(4096, 4096, 1, 1))
        records.append(B.rotated_gemv(12288, 4096, 1, 1))
        records.append(B.leech_gain(ROWS, COLS, 1))
        records.append(B.leech_lp2(4, ROWS, COLS, 1, d=d))
        records.append(B.leech_lp2(4, ROWS, COLS, 4, d=d))
        for rows in (4096, 12288):
            records.append(B.leech_lp2(3, rows, 4096, 1))
        d6 = __import__("synth").leech_matrix(ROWS, COLS, 6)
        records.append(B.leech(6, ROWS, COLS, 1, d=d6))
        records.append(B.leech_lp2x(6, ROWS, COLS, 1, d=d6))
        records.append(B.leech_direct(6, ROWS, COLS, 1, d=d6))
        records.append(B.leech_direct(4, ROWS, COLS, 1, d=d))
        records.append(B.leech_direct(4, ROWS, COLS, 4, d=d))
        records.append(B.leech_direct(3, 12288, 4096, 1))
        records.append(B.leech_onehot(4, ROWS, COLS, 1, d=d))
        records.append(B.leech_onehot(3, 12288, 4096, 1))
        records.append(B.unfold(ROWS * (COLS // 24)))
        fp16_by_shape = {(r["R"], r["K"]): r["gbps"] for r in records if r["arm"] == "fp16"}
        for r in records:
            if "R" not in r:
                continue
            c = fp16_by_shape.get((r["R"], r["K"]))
            r["pct_fp16_control"] = round(100 * r["gbps"] / c, 1) if c and r["arm"] != "fp16" else None
        if stack_blobs is not None:
            stack = B.stack(stack_blobs, args.stack_layers, pool)
            del stack_blobs

    cpu = None
    if not args.no_cpu:
        t0 = time.perf_counter()
        cpu = cpu_baseline(d, x, [(1, 1536, 1536), (3, 4096, 4096), (3, 12288, 4096),
                                  (3, 1024, 4096)])
        head["oracle_us_1core"] = cpu["oracle_us_1core"]
        head["oracle_us_ncores"] = cpu["oracle_us_ncores"]
        head["ncores"] = cpu["cores"]
        log("cpu baseline done in %.1fs" % (time.perf_counter() - t0))

    us = head["us_median"]
    value = head["bytes_weights"] / (us * 1e-6) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "Leech GEMV 4096x12288 (down_proj-shaped), batch 1, "
                               "shells 2..6 with P(m)~2^-m, LP3 layout 4.668 b/w",
                   "rows": ROWS, "cols": COLS, "batch": 1, "copies": head["copies"],
                   "trials": args.trials, "device": props.name, "arch": arch,
                   "torch": torch.__version__, "hip": getattr(torch.version, "hip", None)},
        "roofline": {"bound": "hbm", "achieved": round(value, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(value / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profile()},
        "cpu_baseline": cpu,
        "records": records,
        "stack": stack,
        # the summary last, so that the end of the line (what a log tail
        # shows) carries the gate's verdict and the headline's context
        "us_per_gemv": us,
        "us_per_gemv_graph": getattr(B, "graph_us", None),
        "us_noweights": head["us_noweights"],
        "pct_stream_ceiling": head["pct_stream_ceiling"],
        "cpu_cores_used": cpu["cores"] if cpu else None,
        "cpu_cores_available": cpu["cores_available"] if cpu else None,
        "timing_trials_redone": Timed.redone,
        "parity_checks": len(leg.ratios),
        "parity_max_ratio_all_records": leg.worst(),
        "bitexact": head.get("bitexact"),
        "parity_max_ratio": head.get("parity_max_ratio"),
    }
    return out


if __name__ == "__main__":
    main()
