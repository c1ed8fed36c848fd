"""R-SWA benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload ragged_mix]

One step is one whole job of the workload through the C ABI: causal prefill
of every request in every layer (RoPE + cache write + attention), the
staggered pre-roll that puts requests at different ring phases, then the
measured decode steps (per layer one launch: ring write, split-KV decode and
the cross-split merge; the step's last layer also advances the ring state).
Inputs are synthetic and already resident in HBM when timing starts.  The
timed steps carry no per-launch instrumentation; kernel durations for the
roofline come from one more job with event pairs around each launch.
Prints one JSON line.

value = decode KV-read GB/s over the measured decode steps: per request,
layer and step the method must read 4 * H * D * L bytes of bf16 keys and
values, L = prefill_len + min(t + 1, W).  Prefill TFLOP/s counts
4 * H * D * P (P + 1) / 2 per request and layer.
"""

from __future__ import annotations

import argparse
import dataclasses
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from kv_cache_management_amd import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
METRIC = "R-SWA decode KV-read GB/s (% HBM peak), decode steps/s; prefill TFLOP/s"
PROFILE_DIR = os.path.join(ROOT, "profiles")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def visible_keys(p: int, t: int, window: int, attention: str = "rswa") -> int:
    """Keys the decode step of a request with prefill p and t generated
    tokens before it attends to: P + min(t + 1, W) for R-SWA, the newest
    min(W, P + t + 1) positions for the standard-window baseline."""
    if attention == "swa":
        return min(window, p + t + 1)
    return p + min(t + 1, window)


def kv_bytes_per_layer_step(w: W.Workload, t_before, attention: str = "rswa"):
    """Algorithmic K+V bytes one layer's decode reads for the active requests,
    given each request's generated count before the step."""
    eb = w.elem_bytes
    return sum(2 * w.heads * w.head_dim * eb * visible_keys(p, t, w.window, attention)
               for p, t in zip(w.prefill_lens, t_before))


def prefill_flops(w: W.Workload):
    return sum(4 * w.heads * w.head_dim * p * (p + 1) // 2 for p in w.prefill_lens) * w.layers


class Job:
    """Device-resident inputs and the cache for one workload."""

    def __init__(self, w: W.Workload, decode_steps: int, seed: int = 0, fused: bool = True,
                 attention: str = "rswa", input_steps: int = 0):
        import torch
        from kv_cache_management_amd import rswa

        self.torch = torch
        self.R = rswa
        self.lib = rswa.load()
        self.w = w
        self.steps = decode_steps
        self.fused = fused
        dev = torch.device("cuda", torch.cuda.current_device())
        tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        n, H, D, L = w.batch, w.heads, w.head_dim, w.layers
        self.cache = rswa.RSWACache(L, H, D, w.window, max_requests=n, num_slots=w.pool_rows(),
                                    dtype=w.dtype, max_positions=w.max_positions,
                                    rope_base=w.rope_base, slot_table=w.slot_table(),
                                    max_prefill_tokens=sum(w.prefill_lens), attention=attention)
        self.h = self.cache.handle
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed)
        total = sum(w.prefill_lens)

        def rnd(shape):
            t = torch.empty(shape, device=dev, dtype=tdt)
            t.normal_(0.0, w.input_std, generator=gen)
            return t

        self.pf = [[rnd((total, H, D)) for _ in range(3)] for _ in range(L)]
        self.pf_out = torch.empty((total, H, D), device=dev, dtype=tdt)
        starts = w.starts()
        self.pre = max(starts)
        self.starts = starts
        self.schedule = []
        for g in range(self.pre):
            act = [r for r in range(n) if starts[r] > self.pre - 1 - g]
            self.schedule.append(act)
        g_total = self.pre + decode_steps
        # Distinct decode-input steps; step g reads block g mod this (the
        # launches, and the bytes they read, do not depend on the values).
        self.input_steps = min(g_total, input_steps) if input_steps > 0 else g_total
        log(f"allocating decode inputs: {self.input_steps} steps x {L} layers x 3 x {n} x {H} x {D}")
        self.dec = rnd((self.input_steps, L, 3, n, H, D))
        self.dec_out = torch.empty((L, n, H, D), device=dev, dtype=tdt)
        # raw pointers for the hot loop
        self.ids = np.arange(n, dtype=np.int32)
        self.plen = np.array(w.prefill_lens, dtype=np.int32)
        self.base = w.slot_bases().astype(np.int64)
        self.c_ids = self.ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        self.c_plen = self.plen.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        self.c_base = self.base.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        row = n * H * D * self.dec.element_size()
        self.dec_ptr0 = self.dec.data_ptr()
        self.row_bytes = row
        self.out_ptr = [self.dec_out[l].data_ptr() for l in range(L)]
        self.stream = torch.cuda.current_stream(dev)
        self.sptr = self.stream.cuda_stream
        # measured-step KV bytes (all layers)
        self.kv_bytes = 0
        for s in range(decode_steps):
            self.kv_bytes += L * kv_bytes_per_layer_step(w, [st + s for st in starts], attention)
        self.kv_launches = L * decode_steps
        ev = lambda: torch.cuda.Event(enable_timing=True)
        self.ev = {k: ev() for k in ("p0", "p1", "d0", "d1")}
        self.step_ev = None
        self.scratch = None
        self.graph_k = 0
        self.graph = None

    def enable_graph(self, k: int):
        """Measured decode steps replay one captured graph of k whole steps
        (every layer's fused decode, then advance).  Each replay reuses the
        inputs of the first k measured steps; the kernels read and advance
        the per-request state on the device, so positions and ring slots move
        on as in eager steps."""
        if self.steps % k:
            raise ValueError(f"decode steps ({self.steps}) must be a multiple of --graph {k}")
        self.graph_k = k

    def enable_step_events(self, cold: bool):
        """One event pair around every measured decode step; with cold, a
        1 GiB scratch write before each step (outside its pair) evicts the
        L2 and the 256 MB infinity cache."""
        torch = self.torch
        ev = lambda: torch.cuda.Event(enable_timing=True)
        self.step_ev = [(ev(), ev()) for _ in range(self.steps)]
        if cold:
            self.scratch = torch.empty(1 << 30, dtype=torch.uint8, device=self.dec.device)

    def _check(self, st):
        if st != 0:
            raise self.R.RSWAError(st, self.R.rswa_last_error(self.h))

    def _set_batch(self, act):
        ids = np.array(act, dtype=np.int32)
        self._check(self.lib.rswa_set_batch(self.h, len(ids),
                                            ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                            self.sptr))

    def _step(self, g, n_act):
        lib, h, s = self.lib, self.h, self.sptr
        L = self.w.layers
        for l in range(L):
            blk = self.dec_ptr0 + (((g % self.input_steps) * L + l) * 3) * self.row_bytes
            q, k, v = blk, blk + self.row_bytes, blk + 2 * self.row_bytes
            if self.fused:
                st = lib.rswa_decode_step_fused(h, l, q, k, v, self.out_ptr[l], s)
                if st:
                    self._check(st)
                continue
            st = lib.rswa_ring_write(h, l, k, v, s)
            if st:
                self._check(st)
            st = lib.rswa_decode_step(h, l, q, self.out_ptr[l], s)
            if st:
                self._check(st)
        st = lib.rswa_advance(h, s)
        if st:
            self._check(st)

    def run(self, profile_kernels: bool = False):
        lib, h, s, w = self.lib, self.h, self.sptr, self.w
        n = w.batch
        self._set_batch([])
        self.ev["p0"].record(self.stream)
        lib.rswa_profile_enable(h, 1 if profile_kernels else 0)
        for l in range(w.layers):
            q, k, v = (t.data_ptr() for t in self.pf[l])
            self._check(lib.rswa_prefill(h, l, n, self.c_ids, self.c_plen, self.c_base, q, k, v,
                                         self.pf_out.data_ptr(), s))
        lib.rswa_profile_enable(h, 0)
        self.ev["p1"].record(self.stream)
        current = None
        for g, act in enumerate(self.schedule):
            if act != current:
                self._set_batch(act)
                current = act
            self._step(g, len(act))
        if current != list(range(n)):
            self._set_batch(list(range(n)))
        if self.graph_k:
            self._run_graph()
            return
        self.ev["d0"].record(self.stream)
        lib.rswa_profile_enable(h, 1 if profile_kernels else 0)
        if self.step_ev is None:
            for i in range(self.steps):
                self._step(self.pre + i, n)
        else:
            for i in range(self.steps):
                if self.scratch is not None:
                    self.scratch.fill_(i & 255)
                a, b = self.step_ev[i]
                a.record(self.stream)
                self._step(self.pre + i, n)
                b.record(self.stream)
        lib.rswa_profile_enable(h, 0)
        self.ev["d1"].record(self.stream)

    def _run_graph(self):
        torch, lib, h = self.torch, self.lib, self.h
        k = self.graph_k
        # A graph holds the batch plan of its capture, and every job sets the
        # batch again after its pre-roll: capture afresh on a side stream.
        # The capture calls count as enqueuing the first replay's k steps.
        self.graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(self.stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(self.graph, stream=side):
                sptr = side.cuda_stream
                L = self.w.layers
                for i in range(k):
                    g = self.pre + i
                    for l in range(L):
                        blk = self.dec_ptr0 + (((g % self.input_steps) * L + l) * 3) * self.row_bytes
                        self._check(lib.rswa_decode_step_fused(
                            h, l, blk, blk + self.row_bytes, blk + 2 * self.row_bytes,
                            self.out_ptr[l], sptr))
                    self._check(lib.rswa_advance(h, sptr))
        self.stream.wait_stream(side)
        self.ev["d0"].record(self.stream)
        for j in range(self.steps // k):
            if j > 0:
                self._check(lib.rswa_note_steps(h, k))
            self.graph.replay()
        self.ev["d1"].record(self.stream)

    def times_ms(self):
        """(prefill ms, decode ms) of the last run; decode is one bracket
        around all measured steps, or with the cold protocol the sum of the
        per-step pairs (the scratch writes between them excluded)."""
        e = self.ev
        e["d1"].synchronize()
        dec = e["d0"].elapsed_time(e["d1"])
        if self.scratch is not None:
            dec = float(sum(self.step_times_ms()))
        return e["p0"].elapsed_time(e["p1"]), dec

    def step_times_ms(self):
        return [a.elapsed_time(b) for a, b in self.step_ev]

    def kernel_time(self, kernel):
        st, ms, cnt = self.R.rswa_profile_read(self.h, kernel, self.sptr)
        self._check(st)
        return ms, cnt


def traffic_from_profile(workload: str):
    """HBM traffic per decode launch from the committed PMC summary of this
    workload, taken on the current kernel source: the record (HBM bytes per
    launch of the profiled launches, their own algorithmic bytes and the
    ratio), or (None, reason)."""
    path = os.path.join(PROFILE_DIR, f"decode_split_{workload}_pmc.md")
    if not os.path.exists(path):
        return None, f"no {os.path.basename(path)}"
    from kv_cache_management_amd.profsummary import kernel_source_sha

    rec = None
    for line in open(path):
        if line.startswith("<!-- traffic "):
            rec = json.loads(line[len("<!-- traffic "):].rsplit("-->", 1)[0])
    if not rec:
        return None, "no traffic record"
    if rec.get("kernel_source_sha256_16") != kernel_source_sha("decode_split"):
        return None, "decode kernel changed since the counters were taken"
    return rec, None


def measured_peaks(torch, rswa, read_gib: int = 4):
    """What this GPU reaches on its own: a streaming read of a 4 GiB buffer
    with the decode kernel's load instruction (rswa_measure_read), a large
    bf16 GEMM through the vendor library (torch.matmul -> hipBLASLt), and the
    prefill kernel's MFMA alone on random and on zero operands
    (rswa_measure_mfma)."""
    dev = torch.device("cuda", torch.cuda.current_device())
    stream = torch.cuda.current_stream(dev)
    nbytes = read_gib << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(7)
    sink = torch.empty(rswa.RSWA_MEASURE_SINK_WORDS, dtype=torch.int32, device=dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    for _ in range(2):
        st = rswa.rswa_measure_read(buf.data_ptr(), nbytes, sink.data_ptr(), stream.cuda_stream)
        assert st == 0, st
    a, b = ev(), ev()
    reps = 10
    a.record(stream)
    for _ in range(reps):
        rswa.rswa_measure_read(buf.data_ptr(), nbytes, sink.data_ptr(), stream.cuda_stream)
    b.record(stream)
    b.synchronize()
    read_gbs = nbytes * reps / (a.elapsed_time(b) / 1e3) / 1e9
    del buf
    # A plain device copy (torch): the ceiling for the prefill cache write,
    # which reads k and v and writes them into the pool.
    src = torch.empty(1 << 29, dtype=torch.int16, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    a.record(stream)
    reps = 20
    for _ in range(reps):
        dst.copy_(src)
    b.record(stream)
    b.synchronize()
    copy_gbs = 2 * src.numel() * 2 * reps / (a.elapsed_time(b) / 1e3) / 1e9
    del src, dst
    n = 8192
    x = torch.randn((n, n), device=dev, dtype=torch.bfloat16)
    y = torch.randn((n, n), device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        z = torch.matmul(x, y)
    a.record(stream)
    reps = 20
    for _ in range(reps):
        z = torch.matmul(x, y)
    b.record(stream)
    b.synchronize()
    gemm_tflops = 2 * n ** 3 * reps / (a.elapsed_time(b) / 1e3) / 1e12
    del x, y, z
    # Matrix-core rate with the prefill kernel's MFMA alone, on N(0, 1) bf16
    # operands and on zeros: the gap is the clock the matrix cores lose to
    # the power their random operands draw.
    mfma = {}
    sink = torch.empty(512, dtype=torch.float32, device=dev)
    for kind in ("random", "zeros"):
        ops = (torch.randn if kind == "random" else torch.zeros)(
            (rswa.RSWA_MEASURE_MFMA_FRAGMENTS, 8), device=dev, dtype=torch.float32).to(torch.bfloat16)
        st = rswa.rswa_measure_mfma(ops.data_ptr(), 300_000, sink.data_ptr(), stream.cuda_stream)
        assert st == 0, st
        iters = 1_500_000
        a.record(stream)
        rswa.rswa_measure_mfma(ops.data_ptr(), iters, sink.data_ptr(), stream.cuda_stream)
        b.record(stream)
        b.synchronize()
        mfma[kind] = rswa.RSWA_MEASURE_MFMA_FLOPS_PER_ITER * iters / (a.elapsed_time(b) / 1e3) / 1e12
        del ops
    torch.cuda.empty_cache()
    return {"hbm_read_GBps": round(read_gbs, 1), "hbm_read": f"rswa_measure_read over {read_gib} GiB",
            "device_copy_GBps": round(copy_gbs, 1),
            "device_copy": "torch copy_ of 1 GiB, read + write bytes",
            "bf16_gemm_TFLOPs": round(gemm_tflops, 1),
            "bf16_gemm": f"torch.matmul {n}x{n}x{n} bf16",
            "bf16_mfma_random_TFLOPs": round(mfma["random"], 1),
            "bf16_mfma_zeros_TFLOPs": round(mfma["zeros"], 1),
            "bf16_mfma": "rswa_measure_mfma, 32x32x16 bf16 MFMA only, 2 waves/SIMD, ~0.3 s per figure"}


def prefill_main(runs: int = 3):
    """Prefill attention kernel on the 100-page document (4 x 25728 tokens,
    one layer): the configuration whose prefill is the main TFLOP/s
    datapoint, measured beside any --workload with the same kernel events."""
    from kv_cache_management_amd import rswa

    w = W.DOC100
    job = Job(w, 1)
    job.run(profile_kernels=False)
    for _ in range(runs):
        job.run(profile_kernels=True)
    job.times_ms()
    ms, cnt = job.kernel_time(rswa.RSWA_KERNEL_PREFILL_ATTENTION)
    job.cache.close()
    avg_s = ms / cnt / 1e3
    per_launch = prefill_flops(w) / w.layers
    tf = per_launch / avg_s / 1e12
    return {"workload": w.name, "requests": w.batch, "prefill_len": w.prefill_lens[0],
            "bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "avg_launch_us": round(avg_s * 1e6, 1), "launches": cnt}


def power_clock(torch, rswa, secs: float = 6.0):
    """Socket power and graphics clock while one load runs back to back:
    idle, the 100-page prefill (4 x 25728 tokens, one layer), the MFMA-only
    loop on zero and then on random bf16 operands, the streaming read.
    amd-smi is sampled from a thread (`amd-smi metric -p -c --json`, about
    every 0.1 s) and each phase reports the median of its samples.  It shows
    which figures the board's power limit holds down: the matrix cores on
    random operands run at the power cap with the clock lowered, while zero
    operands and HBM streaming keep the full clock."""
    import statistics
    import subprocess
    import threading
    import time

    cmd = ["amd-smi", "metric", "-p", "-c", "--json"]
    dev = torch.device("cuda", torch.cuda.current_device())
    stream = torch.cuda.current_stream(dev)

    def sample():
        r = subprocess.run(cmd, capture_output=True, text=True)
        try:
            j = json.loads(r.stdout)
            g = j["gpu_data"][0] if isinstance(j, dict) else j[0]
            watts = float(g["power"]["socket_power"]["value"])
            clks = [v["clk"]["value"] for k, v in g["clock"].items()
                    if k.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict)]
            return watts, statistics.mean(clks)
        except (ValueError, KeyError, IndexError, TypeError):
            return None

    if sample() is None:
        return {"error": "amd-smi gave no power / clock reading", "sampler": " ".join(cmd)}
    job = Job(W.DOC100, 1)
    job.run()
    sink = torch.empty(rswa.RSWA_MEASURE_SINK_WORDS, dtype=torch.int32, device=dev)
    ops = {k: (torch.randn if k == "random" else torch.zeros)(
        (rswa.RSWA_MEASURE_MFMA_FRAGMENTS, 8), device=dev, dtype=torch.float32).to(torch.bfloat16)
        for k in ("random", "zeros")}
    buf = torch.empty(4 << 30, dtype=torch.uint8, device=dev).fill_(7)
    torch.cuda.synchronize()
    samples, stop = [], [False]

    def poll():
        while not stop[0]:
            t0 = time.time()
            v = sample()
            if v:
                samples.append((t0, time.time(), v))

    th = threading.Thread(target=poll, daemon=True)
    th.start()
    loads = [
        ("idle", lambda: time.sleep(0.05)),
        ("prefill_doc100", lambda: job.run()),
        ("idle", lambda: time.sleep(0.05)),
        ("mfma_zeros", lambda: rswa.rswa_measure_mfma(ops["zeros"].data_ptr(), 1_500_000, sink.data_ptr(),
                                                      stream.cuda_stream)),
        ("idle", lambda: time.sleep(0.05)),
        ("mfma_random", lambda: rswa.rswa_measure_mfma(ops["random"].data_ptr(), 1_500_000,
                                                       sink.data_ptr(), stream.cuda_stream)),
        ("idle", lambda: time.sleep(0.05)),
        ("hbm_read", lambda: rswa.rswa_measure_read(buf.data_ptr(), buf.numel(), sink.data_ptr(),
                                                    stream.cuda_stream)),
    ]
    phases = []
    for name, fn in loads:
        log(f"power: {name}")
        t0, calls = time.time(), 0
        while time.time() - t0 < (secs / 2 if name == "idle" else secs):
            fn()
            torch.cuda.synchronize()
            calls += 1
        phases.append((name, t0, time.time(), calls))
    stop[0] = True
    th.join()
    job.cache.close()
    out = []
    for name, t0, t1, calls in phases:
        # samples wholly inside the phase, after its first second (the clock settles)
        v = [x for a, b, x in samples if a >= t0 + 1.0 and b <= t1]
        if not v:
            continue
        out.append({"phase": name, "samples": len(v), "calls": calls,
                    "socket_power_W": statistics.median(x[0] for x in v),
                    "gfx_clock_MHz": round(statistics.median(x[1] for x in v))})
    return {"sampler": " ".join(cmd), "phase_seconds": secs, "phases": out}


def ngram_ban_timing(torch, rswa, requests=64, vocab=129280, ngram=35, window=128, reps=200):
    """Time of one rswa_ngram_ban call at the page's sizes: 64 requests,
    129,280-token vocabulary, n = 35 inside a 128-token window, bf16 logits.
    Token rows repeat a short block so bans occur.  The kernel reads each
    window (512 B per request) and writes only the banned logits: it is
    launch-latency bound, so the figure reported is microseconds per call."""
    dev = torch.device("cuda", torch.cuda.current_device())
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    stride = 512
    period = torch.randint(1, 61, (requests, 1), device=dev, generator=g)
    block = torch.randint(0, vocab, (requests, 64), device=dev, generator=g)
    idx = torch.arange(stride, device=dev)[None, :] % period
    tokens = torch.gather(block, 1, idx).to(torch.int32).contiguous()
    lengths = torch.randint(ngram, stride + 1, (requests,), device=dev, generator=g).to(torch.int32)
    logits = torch.randn((requests, vocab), device=dev, generator=g).to(torch.bfloat16)
    for _ in range(5):
        rswa.ngram_ban(tokens, lengths, logits, ngram=ngram, window=window)
    stream = torch.cuda.current_stream(dev)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        rswa.ngram_ban(tokens, lengths, logits, ngram=ngram, window=window)
    b.record(stream)
    b.synchronize()
    banned = int(torch.isneginf(logits.float()).sum().item())
    return {"avg_us_per_call": round(a.elapsed_time(b) * 1e3 / reps, 2), "requests": requests,
            "vocab": vocab, "ngram": ngram, "window": window, "logits": "bf16",
            "banned_entries": banned, "bound": "launch latency"}


def serve(torch, rswa, args):
    """Serving loop over the library: requests queue up, are admitted into
    the pool while rows are free (rswa_admit), prefilled in varlen chunks of
    at most --chunk tokens per iteration across requests
    (rswa_prefill_chunk, every layer), decoded together once fully
    prefilled (rswa_decode_step_fused per layer, rswa_advance) up to
    --max-batch at a time, and retired after --gen tokens (rswa_retire),
    which frees their rows for the queue.  Synthetic inputs; the whole loop
    is bracketed by one event pair.  Prints one JSON line."""
    dev = torch.device("cuda", torch.cuda.current_device())
    stream = torch.cuda.current_stream(dev)
    L, H, D, Wn = 12, 10, 128, W.WINDOW
    rng = np.random.default_rng(0)
    plens = [int(p) for p in rng.integers(272, 8257, args.requests)]
    rows = int(args.pool_requests * (np.mean(plens) + Wn))
    table = np.random.default_rng(1).permutation(rows).astype(np.int32)
    cache = rswa.RSWACache(L, H, D, Wn, max_requests=args.requests, num_slots=rows,
                           max_prefill_tokens=args.chunk, slot_table=table,
                           max_splits=max(16384, 4 * args.requests))
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    pf_in = [torch.randn((3, args.chunk, H, D), device=dev, generator=g).to(torch.bfloat16)
             for _ in range(L)]
    pf_out = torch.empty((args.chunk, H, D), device=dev, dtype=torch.bfloat16)
    dec_in = torch.randn((L, 3, args.max_batch, H, D), device=dev, generator=g).to(torch.bfloat16)
    dec_out = torch.empty((L, args.max_batch, H, D), device=dev, dtype=torch.bfloat16)
    queue = list(range(args.requests))
    base, done_rows, gen = {}, {}, {}
    admitted, batch = [], []
    finished = 0
    it = pf_tokens = dec_tokens = 0
    peak_rows = 0
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record(stream)
    while finished < args.requests:
        it += 1
        # admission while rows are free
        while queue:
            r = queue[0]
            st, bs = rswa.rswa_admit(cache.handle, r, plens[r])
            if st == rswa.RSWA_E_CAPACITY:
                break
            cache._check(st)
            base[r], done_rows[r], gen[r] = bs, 0, 0
            admitted.append(queue.pop(0))
        peak_rows = max(peak_rows, rows - cache.free_rows())
        # one varlen prefill call per layer over the next chunks
        part, budget = [], args.chunk
        for r in admitted:
            if budget == 0:
                break
            left = plens[r] - done_rows[r]
            if left > 0:
                ln = min(left, budget)
                part.append((r, done_rows[r], ln))
                budget -= ln
        if part:
            ids = [r for r, _, _ in part]
            tot = sum(ln for _, _, ln in part)
            for l in range(L):
                q, k, v = (x[:tot] for x in pf_in[l])
                cache.prefill_chunk(l, ids, [plens[r] for r in ids], [base[r] for r in ids],
                                    [s0 for _, s0, _ in part], [ln for _, _, ln in part],
                                    q, k, v, pf_out[:tot])
            for r, s0, ln in part:
                done_rows[r] = s0 + ln
            pf_tokens += tot
        # one decode step for up to max_batch fully prefilled requests
        ready = [r for r in admitted if done_rows[r] == plens[r]][: args.max_batch]
        if not part and not ready:
            raise RuntimeError(f"serving loop stalled at iteration {it}: request {queue[:1]} "
                               f"does not fit the pool of {rows} rows")
        if ready:
            if ready != batch:
                cache.set_batch(ready)
                batch = ready
            n = len(batch)
            for l in range(L):
                cache.decode_step_fused(l, dec_in[l, 0, :n], dec_in[l, 1, :n], dec_in[l, 2, :n],
                                        dec_out[l, :n])
            cache.advance()
            dec_tokens += n
            done = []
            for r in batch:
                gen[r] += 1
                if gen[r] == args.gen:
                    done.append(r)
            if done:
                batch = [r for r in batch if r not in done]
                cache.set_batch(batch)
                cache.retire(done)
                admitted = [r for r in admitted if r not in done]
                finished += len(done)
    b.record(stream)
    b.synchronize()
    gpu_s = a.elapsed_time(b) / 1e3
    wall = time.perf_counter() - t0
    cache.close()
    return {
        "metric": "R-SWA serving loop: generated tokens/s with chunked prefill, admission and retirement",
        "value": round(dec_tokens / gpu_s, 1), "unit": "generated tokens/s", "n_gpus": 1,
        "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "serve_mix", "requests": args.requests, "layers": L, "heads": H,
                   "head_dim": D, "window": Wn, "prefill_len": "U{272..8256}, seed 0",
                   "generated_per_request": args.gen, "max_batch": args.max_batch,
                   "chunk_tokens": args.chunk, "pool_rows": rows, "kv_layout": "page-size-1 slot table"},
        "iterations": it, "prefill_tokens": pf_tokens, "generated_tokens": dec_tokens,
        "gpu_seconds": round(gpu_s, 3), "wall_seconds": round(wall, 3),
        "prefill_tokens_per_s": round(pf_tokens / gpu_s, 1),
        "peak_reserved_rows": int(peak_rows),
    }


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w: W.Workload, budget_s: float = 16.0, attention: str = "rswa"):
    """The oracle, as it stands, timed on this host's cores on a bounded sample
    of the same workload (decode of sampled requests in steady state)."""
    from kv_cache_management_amd import synth
    from oracle import rswa_oracle as O

    # Every core this process may run on, with the BLAS pool set to match.
    cores = len(os.sched_getaffinity(0))
    blas = None
    limiter = None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limiter = threadpool_limits(limits=cores, user_api="blas")
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            blas = {"library": info[0].get("internal_api"), "version": info[0].get("version"),
                    "threads": info[0].get("num_threads"), "arch": info[0].get("architecture")}
    except Exception:
        pass
    try:
        np_cfg = np.show_config(mode="dicts")
        np_build = {"blas": np_cfg.get("Build Dependencies", {}).get("blas", {}).get("name"),
                    "lapack": np_cfg.get("Build Dependencies", {}).get("lapack", {}).get("name"),
                    "simd": np_cfg.get("SIMD Extensions", {}).get("found")}
    except Exception:
        np_build = None
    n = w.batch
    reqs = sorted(set(np.linspace(0, n - 1, min(8, n)).round().astype(int).tolist()))
    starts = w.starts()
    layer = 0
    kv = 0
    steps_done = 0
    t_dec = 0.0
    per_req_budget = budget_s * 0.8 / len(reqs)
    for r in reqs:
        p = w.prefill_lens[r]
        pk = synth.draw(w.seed, w.wid, layer, synth.K_PREFILL, r, (p, w.heads, w.head_dim),
                        w.input_std, w.dtype)
        pv = synth.draw(w.seed, w.wid, layer, synth.V_PREFILL, r, (p, w.heads, w.head_dim),
                        w.input_std, w.dtype)
        rc = O.RingCache(p, w.window, w.heads, w.head_dim, w.rope_base)
        rc.load_prefill(pk, pv)
        s0 = starts[r] + w.window   # steady state: ring full
        nmax = 4096
        nmax = min(nmax, w.max_positions - p - s0)
        dq, dk, dv = (synth.draw(w.seed, w.wid, layer, kind, r, (s0 + nmax, w.heads, w.head_dim),
                                 w.input_std, w.dtype) for kind in (3, 4, 5))
        for s in range(s0):           # fill the ring (untimed)
            rc.write(dk[s], dv[s])
            rc.s += 1
        t0 = time.perf_counter()
        for i in range(nmax):
            s = s0 + i
            rc.step(dq[s], dk[s], dv[s], attention)
            kv += 2 * w.heads * w.head_dim * w.elem_bytes * visible_keys(p, s, w.window, attention)
            steps_done += 1
            if time.perf_counter() - t0 > per_req_budget:
                break
        t_dec += time.perf_counter() - t0
    # prefill: one request, full causal attention by definition
    rp = reqs[len(reqs) // 2]
    p = min(w.prefill_lens[rp], 2048)
    q, k, v = (synth.draw(w.seed, w.wid, layer, kind, rp, (p, w.heads, w.head_dim),
                          w.input_std, w.dtype) for kind in (0, 1, 2))
    t0 = time.perf_counter()
    O.prefill(q, k, v, w.rope_base)
    t_pf = time.perf_counter() - t0
    pf_flops = O.prefill_flops(p, w.heads, w.head_dim)
    if limiter is not None:
        limiter.restore_original_limits()
    return {
        "value": round(kv / t_dec / 1e9, 4),
        "unit": "GB/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle (RingCache.step): {steps_done} steady-state decode steps of "
                   f"requests {reqs} in layer {layer} ({kv / 1e9:.3f} GB of algorithmic KV reads "
                   f"in {t_dec:.2f} s); prefill: one request, first {p} tokens, layer {layer}"),
        "cpu": cpu_model(),
        "cores_source": "len(os.sched_getaffinity(0)); BLAS threads set to it",
        "blas": blas,
        "numpy_build": np_build,
        "decode_steps_per_s_per_request_layer": round(steps_done / t_dec, 3),
        "prefill_gflops": round(pf_flops / t_pf / 1e9, 3),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="ragged_mix", choices=sorted(W.ALL))
    ap.add_argument("--decode-steps", type=int, default=None,
                    help="measured decode steps per job (default: the workload's)")
    ap.add_argument("--input-steps", type=int, default=0,
                    help="distinct decode-input steps, cycled (default: one per step); for "
                         "profiler runs that cannot hold the full input set")
    ap.add_argument("--unfused", action="store_true",
                    help="separate rswa_ring_write + rswa_decode_step calls instead of "
                         "rswa_decode_step_fused")
    ap.add_argument("--no-kernel-events", action="store_true",
                    help="do not time kernels with event pairs inside the timed steps")
    ap.add_argument("--attention", choices=("rswa", "swa"), default="rswa",
                    help="swa: the standard sliding-window baseline (prefill keys cut)")
    ap.add_argument("--window", type=int, default=None,
                    help="override the workload's W (a W of at least the decode steps is the "
                         "growing full-cache baseline)")
    ap.add_argument("--graph", type=int, default=0, metavar="K",
                    help="replay a captured graph of K whole decode steps (fused call; the "
                         "graph reuses the first K steps' inputs)")
    ap.add_argument("--cold", action="store_true",
                    help="cold-cache protocol: a 1 GiB scratch write before every measured "
                         "decode step, outside that step's event pair")
    ap.add_argument("--no-step-times", action="store_true",
                    help="no per-step event pairs (no step-time percentiles)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured read / GEMM peaks")
    ap.add_argument("--serve", action="store_true",
                    help="serving loop with chunked prefill, admission and retirement (own JSON line)")
    ap.add_argument("--requests", type=int, default=96)
    ap.add_argument("--gen", type=int, default=256, help="tokens generated per request (--serve)")
    ap.add_argument("--max-batch", type=int, default=32)
    ap.add_argument("--chunk", type=int, default=8192, help="prefill tokens per iteration (--serve)")
    ap.add_argument("--pool-requests", type=float, default=40.0,
                    help="pool sized for this many average requests (--serve)")
    ap.add_argument("--no-prefill-main", action="store_true",
                    help="skip the prefill-kernel timing on the 100-page document")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=16.0)
    ap.add_argument("--power", action="store_true",
                    help="only sample socket power and clock during prefill, MFMA-only and HBM loads")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (torch) for counter calibration")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the R-SWA path here is single-GPU "
              f"(requested --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(int(os.environ.get("LOCAL_RANK", "0")))
    from kv_cache_management_amd import rswa

    if args.copy_calibration:
        # A plain copy kernel of known size: reads 1 GiB and writes 1 GiB.
        src = torch.empty(1 << 29, dtype=torch.int16, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 2, "copy_bytes_written": dst.numel() * 2,
                          "launches": 3}))
        return

    if args.serve:
        print(json.dumps(serve(torch, rswa, args)), flush=True)
        return

    if args.power:
        print(json.dumps(power_clock(torch, rswa)), flush=True)
        return

    w = W.ALL[args.workload]
    steps = args.decode_steps or w.decode_steps
    if args.window:
        w = dataclasses.replace(w, window=args.window)
    log(f"workload {w.name}: {w.batch} requests x {w.layers} layers, sum P = {sum(w.prefill_lens)}, "
        f"{steps} decode steps")
    job = Job(w, steps, fused=not args.unfused, attention=args.attention, input_steps=args.input_steps)
    if args.graph:
        if args.unfused or args.cold:
            sys.exit("--graph captures fused steps with warm caches only")
        job.enable_graph(args.graph)
    elif args.cold or not args.no_step_times:
        job.enable_step_events(cold=args.cold)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        t0 = time.perf_counter()
        job.run(profile_kernels=False)
        torch.cuda.synchronize()
        log(f"warmup {i}: {time.perf_counter() - t0:.2f} s")
    prof = not args.no_kernel_events
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    pf_ms, dec_ms = [], []
    # The timed steps carry no per-launch events (only the bracket, and with
    # --cold one pair per decode step).
    for i in range(args.steps):
        job.run(profile_kernels=False)
        a, b = job.times_ms()   # events of this step: synchronizes on them
        pf_ms.append(a)
        dec_ms.append(b)
        log(f"step {i}: prefill {a:.2f} ms, decode {b:.2f} ms")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_stats = None
    if job.step_ev is not None:
        st_ms = np.array(job.step_times_ms())
        q = max(1, len(st_ms) // 4)
        # step time against output length: median of 16 steps around each mark
        marks = sorted(set(int(x) for x in np.linspace(0, len(st_ms) - 1, 5)))
        by_t = {str(m): round(float(np.median(st_ms[max(0, m - 8): m + 8])), 4) for m in marks}
        step_stats = {"p50_ms": round(float(np.percentile(st_ms, 50)), 4),
                      "ms_at_measured_step": by_t,
                      "p99_ms": round(float(np.percentile(st_ms, 99)), 4),
                      "max_ms": round(float(st_ms.max()), 4),
                      "last_quarter_over_first_quarter": round(float(st_ms[-q:].mean() / st_ms[:q].mean()), 4),
                      "steps": int(len(st_ms)), "run": "last measured job"}
    k_dec = k_pf = (None, 0)
    if prof:
        # Kernel durations: one more job of the same work with an event pair
        # around every decode and prefill-attention launch (eager calls).
        log("kernel-timing job")
        graph_k, job.graph_k = job.graph_k, 0
        job.run(profile_kernels=True)
        job.times_ms()
        job.graph_k = graph_k
        k_dec = job.kernel_time(rswa.RSWA_KERNEL_DECODE_SPLIT)
        k_pf = job.kernel_time(rswa.RSWA_KERNEL_PREFILL_ATTENTION)

    dec_s = sum(dec_ms) / 1e3
    kv_total = job.kv_bytes * args.steps
    value = kv_total / dec_s / 1e9
    pf_flops = prefill_flops(w)
    pf_tflops = pf_flops * args.steps / (sum(pf_ms) / 1e3) / 1e12
    roofline = None
    if prof and k_dec[1]:
        per_launch_bytes = job.kv_bytes / job.kv_launches
        avg_s = k_dec[0] / k_dec[1] / 1e3
        achieved = per_launch_bytes / avg_s / 1e9
        trec, why = traffic_from_profile(w.name)
        # The PMC record is paired with the algorithmic bytes of the launches
        # it profiled (a shorter run of this workload), never with this line's.
        roofline = {"bound": "hbm", "kernel": "decode_split_kernel", "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": trec["hbm_bytes_per_launch"] if trec else None,
                    "traffic_algorithmic_bytes_per_launch":
                        trec["algorithmic_bytes_per_launch"] if trec else None,
                    "traffic_over_algorithmic": (round(trec["hbm_bytes_per_launch"] /
                                                       trec["algorithmic_bytes_per_launch"], 4)
                                                 if trec else None),
                    "traffic_note": (f"profiles/decode_split_{w.name}_pmc.md: {trec['launches_note']}"
                                     if trec else why),
                    "algorithmic_bytes_per_launch": int(per_launch_bytes),
                    "avg_launch_us": round(avg_s * 1e6, 2), "launches": k_dec[1],
                    "timing": "HIP event pair per launch, in a separate job after the timed steps"}
    prefill_kernel = None
    if prof and k_pf[1]:
        avg_s = k_pf[0] / k_pf[1] / 1e3
        per_launch = pf_flops / w.layers
        prefill_kernel = {"bound": "mfma", "achieved": round(per_launch / avg_s / 1e12, 2),
                          "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "frac": round(per_launch / avg_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                          "avg_launch_us": round(avg_s * 1e6, 1), "launches": k_pf[1]}
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "requests": w.batch, "layers": w.layers, "heads": w.heads,
                   "head_dim": w.head_dim, "window": w.window, "decode_steps": steps,
                   "prefill_tokens": sum(w.prefill_lens),
                   "kv_layout": "page-size-1 slot table" if w.paged else "contiguous",
                   "decode_input_steps": job.input_steps,
                   "decode_call": "rswa_ring_write + rswa_decode_step" if args.unfused
                   else (f"rswa_decode_step_fused, replayed as a graph of {args.graph} steps"
                         if args.graph else "rswa_decode_step_fused"),
                   "attention": "standard sliding window (baseline)" if args.attention == "swa"
                   else ("R-SWA" if w.window < steps + max(w.starts()) else
                         "growing full cache (W >= generated tokens)")},
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "decode_algorithmic_bytes_per_launch": int(job.kv_bytes / job.kv_launches),
        "decode_steps_per_s": round(steps * args.steps / dec_s, 2),
        "decode_ms_per_step": round(dec_s * 1e3 / (steps * args.steps), 4),
        "prefill_tflops": round(pf_tflops, 2),
        "prefill_mfma_frac": round(pf_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "decode_cache": "cold (1 GiB scratch write before each step)" if args.cold else "warm",
        "decode_step_times": step_stats,
        "roofline": roofline,
        "prefill_kernel": prefill_kernel,
        "prefill_main": None,
        "ngram_ban": None,
        "measured_peak": None,
        "cpu_baseline": None,
    }
    out["ngram_ban"] = ngram_ban_timing(torch, rswa)
    if prefill_kernel and w.name == W.DOC100.name:
        out["prefill_main"] = dict(prefill_kernel, workload=w.name)
    elif not args.no_prefill_main and not args.no_kernel_events:
        log("timing the prefill kernel on the 100-page document")
        out["prefill_main"] = prefill_main()
    if not args.no_peaks:
        log("measuring the read, GEMM and MFMA peaks")
        mp = measured_peaks(torch, rswa)
        out["measured_peak"] = mp
        if roofline:
            roofline["frac_of_measured_read"] = round(roofline["achieved"] / mp["hbm_read_GBps"], 4)
        if prefill_kernel:
            prefill_kernel["frac_of_measured_gemm"] = round(prefill_kernel["achieved"] / mp["bf16_gemm_TFLOPs"], 4)
            prefill_kernel["frac_of_measured_mfma"] = round(
                prefill_kernel["achieved"] / mp["bf16_mfma_random_TFLOPs"], 4)
        if out["prefill_main"]:
            out["prefill_main"]["frac_of_measured_mfma"] = round(
                out["prefill_main"]["achieved"] / mp["bf16_mfma_random_TFLOPs"], 4)
    if not args.no_cpu_baseline and int(os.environ.get("RANK", "0")) == 0:
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_budget, args.attention)
    job.cache.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
