#!/usr/bin/env python3
"""Benchmark: DF11 block decode on one MI355X.

One step = one df11_decode_block launch over a whole transformer block (the
Llama-3.1-8B-shaped block by default: q,k,v,o,gate,up,down, 218,103,808
weights, one shared codebook), inputs resident in HBM, with the caches
flushed before it: a read of 1 GiB of unrelated data pushes the block out of
the L2s and the 256 MB Infinity Cache, as a model's other work does between
two block decodes.  Flush and decode pairs are enqueued back to back with no
host synchronisation; each decode is timed with HIP events as the difference
of (flush, decode) and (flush) each between one event pair (an event recorded
between the two kernels would delay the decode's start; see ColdSchedule).
The launches rotate over device copies of the block.  Prints one JSON line.

  value      decoded BF16 GB/s = 2 * weights / mean decode time
  roofline   algorithmic HBM bytes per launch (compressed sections read +
             BF16 written) / mean decode time, vs 8 TB/s; frac_rotated is the
             same for launches back to back over the copies without flushes
  bandwidth_reference  streaming kernels of the library that move the
             decode's bytes without decoding (its memory skeleton, and a plain
             stream of the same bytes), and the stream's writes alone and
             reads alone, timed in both schedules
  cpu_baseline  the oracle's unit-parallel bit-serial decode of the same block
             on this host's cores (rank 0, N=1 only)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
INFINITY_CACHE_BYTES = 256 << 20  # MI355X last-level (Infinity) cache
KERNEL_SRC = os.path.join(ROOT, "huffman_decode_block_amd", "csrc", "df11_decode.hip")
# the headers of this package that the decode kernel's code includes
KERNEL_HEADERS = [os.path.join(ROOT, "huffman_decode_block_amd", "csrc", h) for h in ("df11_wave.h", "df11_internal.h")] \
    + [os.path.join(ROOT, "include", "df11.h")]
COUNTERS = os.path.join(ROOT, "profiles", "df11_decode_kernel_c3_hbm_counters.json")


from huffman_decode_block_amd.build import code_tokens  # noqa: E402  (re-exported for the tests)


def kernel_hash() -> str:
    """Identity of the decode kernel's code: its source and the package headers
    it includes (comments and layout excluded)."""
    parts = []
    for path in [KERNEL_SRC] + KERNEL_HEADERS:
        with open(path, encoding="utf-8") as f:
            parts.append(code_tokens(f.read()))
    return hashlib.sha256("\n".join(parts).encode()).hexdigest()[:16]


def algorithmic_bytes(s, with_counts: bool = False) -> dict:
    """Bytes one decode must move: the compressed payload read once plus the
    BF16 output written once (padding excluded)."""
    rd = ((s.total_bits + 7) // 8          # encoded exponents
          + s.n_total                      # sign/mantissa bytes
          + (5 * s.n_windows + 7) // 8     # 5-bit gaps
          + 8 * (s.n_units + 1)            # unit positions
          + s.raw.tables_bytes             # decode tables
          + (s.n_windows if with_counts else 0)  # per-window counts (counting-free variant)
          + 2 * (s.n_units if s.unit_end is not None else 0))  # unit ends (aligned-units layout)
    wr = 2 * s.n_total
    return {"read": int(rd), "write": int(wr), "total": int(rd + wr)}


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on this workload and the current kernel code; else None."""
    if not os.path.exists(COUNTERS):
        return None
    with open(COUNTERS) as f:
        c = json.load(f)
    if c.get("kernel_code_sha256_16") != kernel_hash() or not c.get("workload", "").startswith(workload + ":"):
        return None
    return c.get("hbm_bytes_per_launch")


# Sections read between two launches on the same copy, in Infinity Caches:
# the cache keeps part of what a launch read for longer than one cache's worth
# of later reads (C3 back to back over 2 copies, 600 MB of sections: the memory
# skeleton took 124.6 us, over 4 copies 135.2, over 8 copies 136.2, after a
# 1 GiB read 134.9), so the rotation covers several of them.
ROTATION_CACHES = 6


def rotation_copies(read_bytes: int, cap: int = 64) -> int:
    """Device copies of a block that the timed launches rotate over: enough
    that their sections add up to ROTATION_CACHES times the Infinity Cache, at
    least 2, at most `cap` (blocks so small that the cap binds stay cached
    whatever the count)."""
    need = ROTATION_CACHES * INFINITY_CACHE_BYTES
    return int(min(cap, max(2, -(-need // max(int(read_bytes), 1)))))


def progress(msg: str) -> None:
    """A progress line on stderr (stdout carries only the result line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def pctl(v, q: float) -> float:
    """The q-quantile of a list (nearest rank)."""
    v = sorted(v)
    return v[min(len(v) - 1, int(q * len(v)))]


class ColdSchedule:
    """Steps that each start with the caches flushed: a read of 1 GiB of
    unrelated data (an int64 sum, which torch runs on its input as it is; a
    write would leave dirty lines whose write-back competes with the step)
    pushes everything out of the L2s and the 256 MB Infinity Cache, then the
    launch runs.

    A HIP event recorded between two kernels delays the second kernel's start
    by ~5.6 us (kernel traces: no gap from the flush to the launch without an
    event between them, 5.6 us with one), so an event pair around each launch
    would time that delay too.  Instead each step is timed twice, both times
    with the event pair outside the kernels: leg A records (event, flush,
    launch, event), leg B (event, flush, event, launch).  Both intervals hold
    the same marker delay and a flush that follows a launch; the launch's
    duration is A - B (per launch: A_i minus B's mean), which the kernel trace
    of the same command confirms to within 0.2 %.  Steps are enqueued back to
    back with no host synchronisation, so the GPU never idles and its clocks
    stay up; one synchronize at the end of each leg."""

    FLUSH_BYTES = 1 << 30
    # What runs before each step ("read" is the schedule described above; the
    # others attribute what a cold step pays): a read of 256 MiB (the Infinity
    # Cache's size), or a sweep that reads one 8-byte element per 64 KiB over
    # 4 GiB, which touches 65,536 pages but moves only ~4 MB, so that it evicts
    # address translations and leaves the caches' contents as they were.
    FLUSH_KINDS = ("read", "read-256mib", "touch-pages")

    def __init__(self, dev, stream, kind: str = "read"):
        import torch
        if kind not in self.FLUSH_KINDS:
            raise ValueError(f"flush kind must be one of {self.FLUSH_KINDS}")
        self.torch = torch
        self.stream = stream
        n = (4 << 30) if kind == "touch-pages" else (256 << 20) if kind == "read-256mib" else self.FLUSH_BYTES
        self.scratch = torch.ones(n // 8, dtype=torch.int64, device=dev)
        # one element per 64 KiB row for the sweep, the whole buffer otherwise
        self.flush_view = self.scratch.view(-1, 8192)[:, 0] if kind == "touch-pages" else self.scratch
        self.flush_s = None  # leg B's mean of the last run (flush only), seconds

    def _leg(self, launch, k: int, start: int, inside: bool) -> list:
        torch = self.torch
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(k)]
        for i in range(k):
            ev[i][0].record(self.stream)
            self.flush_view.sum()
            if inside:
                launch(start + i)
            ev[i][1].record(self.stream)
            if not inside:
                launch(start + i)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) * 1e-3 for a, b in ev]

    def run(self, launch, k: int) -> list:
        """k cold steps of launch(i) (and k more for leg B, i = k .. 2k-1);
        returns each leg-A launch's duration in seconds, A_i - mean(B)."""
        a = self._leg(launch, k, 0, True)
        b = self._leg(launch, k, k, False)
        self.flush_s = sum(b) / len(b)
        return [t - self.flush_s for t in a]


def back_to_back(launch, k: int, stream, start: int = 0) -> float:
    """k launches back to back between one pair of HIP events on `stream`;
    returns the average launch duration in seconds."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(k):
        launch(start + i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e-3 / k


def cpu_model() -> str:
    """The host CPU's model name (Linux), or the platform's processor string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(sections, x, min_seconds: float, threads: int | None = None) -> dict:
    """The oracle's unit-parallel bit-serial decode of the whole block, repeated
    for at least min_seconds, on `threads` host threads (default: the cores this
    process may use, capped at 16, its share of the machine)."""
    import numpy as np

    import oracle
    if threads is None:
        threads = min(len(os.sched_getaffinity(0)), int(os.environ.get("OMP_NUM_THREADS") or 16))
    enc = oracle.Encoded(n=int(sections.n_total), total_bits=int(sections.total_bits),
                         n_windows=int(sections.n_windows), n_units=int(sections.n_units),
                         code_len=sections.code_len, stream=sections.stream,
                         sign_mant=sections.sign_mant, gaps=sections.gaps,
                         unit_pos=sections.unit_pos, max_len=int(sections.max_code_len))
    out = np.empty(enc.n, dtype=np.uint16)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.decode_units(enc, threads=threads, out=out)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    ok = bool(np.array_equal(out, x))
    split = f"units split over {threads} threads" if threads > 1 else "one thread"
    return {"value": round(2.0 * enc.n * reps / el / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"whole block ({enc.n} weights) decoded {reps}x by the oracle's bit-serial "
                      f"tree walk, {split}; {el:.1f} s; output == input: {ok}"}


def gpu_encode_bench(args, dev) -> None:
    """The GPU-side encoder on one block: histogram on the device, code lengths
    on the host, offsets and packing on the device.  value = BF16 input bytes
    encoded per second by the device passes (histogram + encode)."""
    import numpy as np
    import torch

    import df11_inputs as di
    import huffman_decode_block_amd as hdb

    wl = di.WORKLOADS[args.workload]
    x = di.generate(args.workload)
    xd = torch.from_numpy(x.view(np.int16)).to(dev)
    stream = torch.cuda.current_stream(dev)
    g = hdb.gpu_encode(xd)  # allocates the sections once; checked below
    s_host = hdb.df11_encode_block(di.split(args.workload, x)).sections
    ok = (np.array_equal(g.section("stream")[:g.plan.stream_bytes], s_host.stream)
          and np.array_equal(g.section("sign_mant")[:g.plan.sign_mant_bytes], s_host.sign_mant)
          and np.array_equal(g.section("gaps")[:g.plan.gaps_bytes], s_host.gaps)
          and np.array_equal(g.section("unit_pos").view(np.uint64), s_host.unit_pos))
    if not ok:
        raise SystemExit("GPU encoding differs from the host encoder; refusing to report a number")
    t = g.tensors
    hist = torch.empty(256, dtype=torch.int64, device=dev)

    # the steps rotate over device copies of the input, as for the decode, so
    # that no step finds the previous step's input in the Infinity Cache
    xds = [xd] + [xd.clone() for _ in range(rotation_copies(2 * int(x.size)) - 1)]
    step = [0]

    def encode_once():
        xi = xds[step[0] % len(xds)]
        step[0] += 1
        hdb.df11_gpu_histogram(xi, hist, t["chunk_hist"], stream)
        hdb.df11_gpu_encode(g.plan, xi, t["chunk_hist"], t["stream"], t["sign_mant"], t["gaps"], t["unit_pos"],
                            None, t["workspace"], stream)

    t_pre = time.perf_counter()
    while (time.perf_counter() - t_pre) * 1e3 < args.prewarm_ms:
        for _ in range(10):
            encode_once()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        encode_once()
    torch.cuda.synchronize()
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    t0 = time.perf_counter()
    ev[0].record(stream)
    for _ in range(args.steps):
        encode_once()
    ev[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = ev[0].elapsed_time(ev[1]) * 1e-3 / args.steps
    ok = (np.array_equal(g.section("stream")[:g.plan.stream_bytes], s_host.stream)
          and np.array_equal(g.section("sign_mant")[:g.plan.sign_mant_bytes], s_host.sign_mant)
          and np.array_equal(g.section("gaps")[:g.plan.gaps_bytes], s_host.gaps)
          and np.array_equal(g.section("unit_pos").view(np.uint64), s_host.unit_pos))
    if not ok:
        raise SystemExit("GPU encoding differs from the host encoder after timing; refusing to report a number")
    del xds
    n = int(x.size)
    out_bytes = int(s_host.raw.stream_bytes + s_host.raw.sign_mant_bytes + s_host.raw.gaps_bytes
                    + 8 * (s_host.n_units + 1))
    algo = 2 * n + out_bytes  # the input read once, the sections written once
    # CPU baselines: the library's host encoder (all cores of this process, at
    # most 16) and the oracle's encoder (one thread); whole block, timed once
    threads = min(len(os.sched_getaffinity(0)), int(os.environ.get("OMP_NUM_THREADS") or 16))
    c0 = time.perf_counter()
    hdb.df11_encode_block(di.split(args.workload, x), n_threads=threads)
    t_host = time.perf_counter() - c0
    cpu = {"value": round(2.0 * n / t_host / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "host encoder",
           "sample": f"whole block ({n} weights) encoded once by the library's host encoder, {threads} threads"}
    if not args.no_cpu_baseline:
        import oracle
        c0 = time.perf_counter()
        oracle.encode(x)
        t_or = time.perf_counter() - c0
        cpu_oracle = {"value": round(2.0 * n / t_or / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
                      "sample": f"whole block ({n} weights) encoded once by the oracle (bit-serial, one thread)"}
    else:
        cpu_oracle = None
    res = {
        "metric": "GPU-side DF11 encode of one transformer block (BF16 input GB/s)",
        "value": round(2.0 * n / per / 1e9, 2), "unit": "GB/s", "higher_is_better": True,
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 4),
        "data": "synthetic", "dtype": "u32",
        "config": {"workload": f"{args.workload}: {wl.description}", "weights": n},
        "encode_us": round(per * 1e6, 2),
        "roofline": {"bound": "hbm", "achieved": round(algo / per / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(algo / per / 1e9 / PEAK_HBM_GBS, 4), "algorithmic_bytes_per_step": algo,
                     "note": "the device passes read the input twice (histogram, pack)"},
        "cpu_baseline": cpu,
        "cpu_baseline_oracle": cpu_oracle,
    }
    print(json.dumps(res), flush=True)


def overlap_bench(args, dev) -> None:
    """Exposed decode time per block when block i+1 is decoded on a side stream
    while block i's seven GEMMs (torch F.linear, BF16, synthetic activations of
    `batch` tokens) run: the pages' decompress-just-before-use schedule.  Also
    the serial order (each block decoded on the GEMMs' stream right before
    them) and DecodeAhead's "auto" mode, which times both once per batch size
    and keeps the faster."""
    import numpy as np
    import torch
    import torch.nn.functional as F

    import df11_inputs as di
    import huffman_decode_block_amd as hdb
    from huffman_decode_block_amd.overlap import DecodeAhead

    wl = di.WORKLOADS[args.workload]
    x = di.generate(args.workload)
    enc = hdb.df11_encode_block(di.split(args.workload, x))
    blk = hdb.DeviceBlock.from_encoded(enc, device=dev)
    # device copies of the block in turn, so that no decode finds the
    # sections of an earlier one in the Infinity Cache (as with different
    # blocks)
    n_copies = rotation_copies(algorithmic_bytes(enc.sections)["read"])
    blks = [blk] + [hdb.DeviceBlock.from_encoded(enc, device=dev) for _ in range(n_copies - 1)]
    shapes = [(m.rows, m.cols) for m in wl.mats]
    nb = args.overlap_blocks
    ahead = DecodeAhead([blks[i % n_copies] for i in range(nb)], [shapes] * nb, device=dev)
    ref = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    ref_views = hdb.matrix_views(ref, blk, shapes)
    stream = torch.cuda.current_stream(dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def timed(fn, reps=3):
        best = None
        for _ in range(reps):
            torch.cuda.synchronize()
            a, b = ev(), ev()
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            t = a.elapsed_time(b) * 1e-3
            best = t if best is None else min(best, t)
        return best

    for bs in [int(v) for v in args.overlap.split(",") if v]:
        g = torch.Generator(device=dev).manual_seed(bs)
        acts = {c: torch.randn(bs, c, device=dev, generator=g).to(torch.bfloat16)
                for c in sorted({c for _, c in shapes})}

        def consume(i, views):
            for v in views:
                F.linear(acts[v.shape[1]], v)

        # the GEMMs alone read the weights from the two decode buffers in
        # turn, as every schedule below does (the same weights for every block
        # would stay partly in the Infinity Cache from one block to the next)
        buf_views = []
        for b in range(2):
            hdb.df11_decode_block(blks[b], out=ahead.bufs[b][: blk.n_total], stream=stream)
            buf_views.append(hdb.matrix_views(ahead.bufs[b][: blk.n_total], blk, shapes))
        torch.cuda.synchronize()
        for b in range(2):
            for v, r in zip(buf_views[b], ref_views):
                assert torch.equal(v.view(torch.int16), r.view(torch.int16))

        def gemms_only():
            for i in range(nb):
                consume(i, buf_views[i % 2])

        def decodes_only():
            for i in range(nb):
                hdb.df11_decode_block(blks[i % n_copies], out=ahead.bufs[i % 2][: blk.n_total], stream=stream)

        for f in (gemms_only, decodes_only):  # warm up (clocks, GEMM algorithm choice)
            for _ in range(3):
                f()
        torch.cuda.synchronize()
        # The ahead-decode's footprint: the whole GPU, or a capped number of
        # workgroups (it then streams on fewer CUs and leaves the rest to the
        # GEMMs, which matters once they are compute-bound).
        per_launch = {}
        ahead.mode = "ahead"
        for wv, mg in ((0, 0), (0, 256), (8, 0), (8, 512), (4, 0), (4, 1024), (4, 512), (2, 0)):
            ahead.launch = None if (wv, mg) == (0, 0) else (wv, mg, 0, 0)
            for _ in range(2):
                ahead.run(consume, stream=stream)
            per_launch[(wv, mg)] = timed(lambda: ahead.run(consume, stream=stream)) / nb
        best = min(per_launch, key=per_launch.get)
        t_p = per_launch[best]
        # auto: both schedules timed once for this batch (the ahead decode with
        # the best launch found above), the faster kept
        ahead.launch = None if best == (0, 0) else (best[0], best[1], 0, 0)
        ahead.mode = "auto"
        picked = ahead.calibrate(consume, stream=stream, key=bs)
        auto_launch = ahead.launch

        def serial():
            # the same blocks decoded inline, on the consumer's stream right
            # before each consumer (the serial order, default launch)
            ahead.mode = "inline"
            ahead.run(consume, stream=stream)

        def auto():
            ahead.launch, ahead.mode = auto_launch, "auto"
            ahead.run(consume, stream=stream, key=bs)

        for f in (serial, auto):
            for _ in range(2):
                f()
        # the four compared schedules timed in turn, round after round, each
        # keeping its best, so that a drift of the clocks or of the GEMMs'
        # speed during the run does not favour whichever was timed last
        t_g = t_d = t_s = t_a = float("inf")
        for _ in range(5):
            t_g = min(t_g, timed(gemms_only, reps=1) / nb)
            t_d = min(t_d, timed(decodes_only, reps=1) / nb)
            t_s = min(t_s, timed(serial, reps=1) / nb)
            t_a = min(t_a, timed(auto, reps=1) / nb)
        ahead.launch = None
        name = lambda k: f"{k[0] or 'default'} waves/group, " + (f"{k[1]} groups" if k[1] else "default grid")  # noqa: E731
        res = {
            "metric": "exposed decode time per block, next block decoded on a side stream during this block's GEMMs",
            "value": round((t_p - t_g) * 1e6, 2), "unit": "us", "higher_is_better": False,
            "batch_tokens": bs, "blocks": nb, "workload": f"{args.workload}: {wl.description}",
            "device_copies_rotated": n_copies,
            "gemms_only_us_per_block": round(t_g * 1e6, 2),
            "decode_only_us_per_block": round(t_d * 1e6, 2),
            "pipelined_us_per_block": round(t_p * 1e6, 2),
            "serial_us_per_block": round(t_s * 1e6, 2),
            "auto_schedule": picked,
            "auto_calibration_us_per_block": {k: round(v / nb * 1e6, 2) for k, v in ahead.timings[bs].items()},
            "auto_us_per_block": round(t_a * 1e6, 2),
            "auto_over_serial": round(t_a / t_s, 3),
            "pipelined_over_bf16": round(t_p / t_g, 3),
            "decode_launch": name(best),
            "pipelined_us_by_decode_launch": {name(k): round(v * 1e6, 2) for k, v in per_launch.items()},
        }
        print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="C3", choices=["C1", "C2", "C3", "C4", "C5", "E8"],
                    help="C3 is the headline workload; E8 is a single embedding/LM-head-shaped matrix")
    ap.add_argument("--waves", type=int, default=0, help="waves per workgroup (0 = library default)")
    ap.add_argument("--max-groups", type=int, default=0)
    ap.add_argument("--oversubscribe", type=int, default=0,
                    help="workgroups per resident workgroup slot (0 = library default)")
    ap.add_argument("--variant", type=int, default=0,
                    help="1 = one code per lookup, 2 = multi-code lookups (0 = library default), "
                         "3 = multi-code with stored per-window counts (a format variant)")
    ap.add_argument("--aligned-units", action="store_true",
                    help="encode with the aligned-units layout (a format variant: units start on "
                         "32-weight boundaries)")
    ap.add_argument("--prewarm-ms", type=float, default=500.0,
                    help="untimed decodes before the warmup steps, for this long (the GPU's clocks ramp up "
                         "over the first ~10 ms of load after host-side work)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline (cold) schedule: no back-to-back, same-block or "
                         "bandwidth-reference legs (for profiler runs, whose per-kernel averages then "
                         "cover the headline launches only)")
    ap.add_argument("--schedule", default="cold", choices=["cold", "rotated"],
                    help="the headline leg: cold = caches flushed before every launch, each launch timed by its "
                         "own event pair; rotated = launches back to back over the device copies, one event pair "
                         "around all of them")
    ap.add_argument("--flush", default="read", choices=list(ColdSchedule.FLUSH_KINDS),
                    help="what runs before each cold launch: read = 1 GiB of unrelated data (the headline "
                         "schedule); read-256mib = 256 MiB; touch-pages = one 8-byte element per 64 KiB over "
                         "4 GiB (address translations evicted, cache contents kept)")
    ap.add_argument("--copies", type=int, default=0,
                    help="device copies of the block the launches rotate over (0 = enough that their sections "
                         "cover several Infinity Caches)")
    ap.add_argument("--kernel", default="decode", choices=["decode", "skeleton", "stream"],
                    help="what the headline leg times: the decode, or one of the library's bandwidth references "
                         "(the line then reports that kernel, not the decode)")
    ap.add_argument("--out-offset-bytes", type=int, default=0, choices=[0, 16, 32, 48],
                    help="place each output this many bytes past a 64-byte boundary")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--overlap", default="",
                    help="comma-separated batch sizes: instead of the main line, measure the decode of block i+1 "
                         "on a side stream overlapped with block i's GEMMs (one JSON line per batch)")
    ap.add_argument("--overlap-blocks", type=int, default=12)
    ap.add_argument("--gpu-encode", action="store_true",
                    help="instead of the main line, measure the GPU-side encoder on the workload")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for counter calibration)")
    args = ap.parse_args()
    if args.copies < 0:
        raise SystemExit("--copies must be 0 (automatic) or a positive count")

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the decode needs no cross-GPU exchange and "
              "this build measures a single MI355X (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import df11_inputs as di
    import huffman_decode_block_amd as hdb

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)
        return

    if args.overlap:
        overlap_bench(args, dev)
        return
    if args.gpu_encode:
        gpu_encode_bench(args, dev)
        return

    wl = di.WORKLOADS[args.workload]
    t_gen = time.perf_counter()
    x = di.generate(args.workload)
    progress(f"{args.workload}: {x.size:,} weights generated in {time.perf_counter() - t_gen:.1f} s")
    with_counts = args.variant == hdb.DF11_VARIANT_COUNTS
    t_enc = time.perf_counter()
    enc = hdb.df11_encode_block(di.split(args.workload, x), window_counts=with_counts,
                                aligned_units=args.aligned_units)
    s = enc.sections
    progress(f"encoded on the host in {time.perf_counter() - t_enc:.1f} s")
    launch = (args.waves, args.max_groups, args.variant, args.oversubscribe) \
        if (args.waves or args.max_groups or args.variant or args.oversubscribe) else None
    stream = torch.cuda.current_stream(dev)
    ab = algorithmic_bytes(s, with_counts)
    n = int(s.n_total)
    off = args.out_offset_bytes // 2

    def new_output():
        # torch's allocations start on 512-byte boundaries
        return torch.empty(n + off, dtype=torch.bfloat16, device=dev)[off:]

    # A model decodes a different block each time.  The launches rotate over
    # device copies of the block (each with its own sections and output) whose
    # sections together cover ROTATION_CACHES times the 256 MiB Infinity Cache.
    n_copies = args.copies or rotation_copies(ab["read"])
    copies = [(hdb.DeviceBlock.from_encoded(enc, device=dev), new_output()) for _ in range(n_copies)]

    def decode(i):
        b, o = copies[i % n_copies]
        hdb.df11_decode_block(b, out=o, stream=stream, launch=launch)

    # Correctness of what is timed, checked first: the copy it needs would
    # leave the GPU idle (and its clocks falling) right before the timed steps.
    xd = torch.from_numpy(x.view(np.int16)).to(dev)
    for i in range(n_copies):
        decode(i)
        if not torch.equal(copies[i][1].view(torch.int16), xd):
            raise SystemExit("decode is not bit-exact; refusing to report a number")
    del xd
    progress(f"decode checked bit-exact on {n_copies} device copies of the block; timing")

    # The launches that can be timed: the decode and the two bandwidth
    # references (same copies and outputs; the references write the weights
    # with their exponent fields zero).
    ref_launch = None if launch is None else (args.waves, args.max_groups, 0, args.oversubscribe)

    def reference(kind):
        def run(i):
            b, o = copies[i % n_copies]
            hdb.df11_bandwidth_reference(b, o, kind, stream=stream, launch=ref_launch)
        return run

    kernels = {"decode": decode}
    if not args.aligned_units and not with_counts:
        kernels["skeleton"] = reference(hdb.DF11_REFERENCE_SKELETON)
        kernels["stream"] = reference(hdb.DF11_REFERENCE_STREAM)
        kernels["writes"] = reference(hdb.DF11_REFERENCE_WRITES)
        kernels["reads"] = reference(hdb.DF11_REFERENCE_READS)
    if args.kernel not in kernels:
        raise SystemExit("the bandwidth references cover the pages' format only")
    cold = ColdSchedule(dev, stream, args.flush)
    pos = [0]

    def leg(name, schedule, k):
        """k timed launches of kernel `name` in `schedule`: per-launch times
        (cold) or the region average (rotated), in seconds."""
        fn, start = kernels[name], pos[0]
        pos[0] += 2 * k
        if schedule == "cold":
            return cold.run(lambda j: fn(start + j), k)
        return [back_to_back(fn, k, stream, start)]

    # The headline leg: untimed pre-warm in the same schedule until the
    # clocks have ramped, then W warmup steps, then K timed steps.
    t_pre = time.perf_counter()
    while (time.perf_counter() - t_pre) * 1e3 < args.prewarm_ms:
        leg(args.kernel, args.schedule, 20)
    leg(args.kernel, args.schedule, max(args.warmup, 1))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    kt = leg(args.kernel, args.schedule, args.steps)
    wall = time.perf_counter() - t0
    k_head = sum(kt) / len(kt)

    other = "rotated" if args.schedule == "cold" else "cold"
    times = {(args.kernel, args.schedule): k_head}
    if not args.headline_only:
        if args.kernel != "decode":
            t = leg("decode", args.schedule, args.steps)
            times[("decode", args.schedule)] = sum(t) / len(t)
        leg("decode", other, 20)
        t = leg("decode", other, args.steps)
        times[("decode", other)] = sum(t) / len(t)
        # The same copy over and over: for blocks that fit the Infinity
        # Cache (C1, C2) this is the hot number.
        times[("decode", "same")] = back_to_back(lambda k: decode(0), args.steps, stream)
    # every copy's last decode is still bit-exact (when the decode ran last)
    xd = torch.from_numpy(x.view(np.int16)).to(dev)
    if args.kernel == "decode" or not args.headline_only:
        if args.kernel != "decode":
            for j in range(n_copies):
                decode(j)
        for b, o in copies:
            if not torch.equal(o.view(torch.int16), xd):
                raise SystemExit("decode is not bit-exact after timing; refusing to report a number")
    refs = {}
    if len(kernels) > 1:
        for name in ("skeleton", "stream", "writes", "reads"):
            if not args.headline_only:
                for sched in ("cold", "rotated"):
                    if (name, sched) in times:
                        continue
                    leg(name, sched, 20)
                    t = leg(name, sched, args.steps)
                    times[(name, sched)] = sum(t) / len(t)
            if args.headline_only and name != args.kernel:
                continue
            # skeleton and stream write each weight with its exponent field
            # zero, writes zeros, reads nothing (the outputs keep the values
            # the references before it wrote)
            expect = (torch.zeros_like(xd) if name == "writes"
                      else torch.bitwise_and(xd, torch.tensor(-32641, dtype=torch.int16, device=dev)))  # 0x807F
            if name == "reads":
                for j in range(n_copies):
                    kernels["stream"](j)
            for j in range(n_copies):
                kernels[name](j)
            for b, o in copies:
                if not torch.equal(o.view(torch.int16), expect):
                    raise SystemExit(f"bandwidth reference {name} wrote wrong values; refusing to report a number")
            del expect
            refs[name] = {f"{sched}_us": round(times[(name, sched)] * 1e6, 2)
                          for sched in ("cold", "rotated") if (name, sched) in times}
    del xd, copies, cold
    torch.cuda.empty_cache()
    k_cold = times.get(("decode", "cold"))
    k_rot = times.get(("decode", "rotated"))
    # the committed counters were taken on the default (multi-code) kernel
    traffic = measured_traffic(args.workload) if args.kernel == "decode" and args.variant in (0, 2) \
        and not args.aligned_units else None
    if traffic is None:
        progress("roofline.traffic is null: no committed HBM counter summary matches this kernel code, "
                 "workload and variant")
    ref_bytes = ab["total"] - int(s.raw.tables_bytes)  # the references do not read the decode tables
    head_bytes = ab["total"] if args.kernel == "decode" else ref_bytes
    achieved = head_bytes / k_head / 1e9
    frac = lambda t, nb=ab["total"]: round(nb / t / 1e9 / PEAK_HBM_GBS, 4) if t else None  # noqa: E731
    out_bytes = 2 * n
    for name, r in refs.items():
        nb = {"writes": out_bytes, "reads": ref_bytes - out_bytes}.get(name, ref_bytes)
        r["bytes"] = nb
        for sched in ("cold", "rotated"):
            if f"{sched}_us" in r:
                r[f"GBps_{sched}"] = round(nb / r[f"{sched}_us"] / 1e3, 1)
                kd = times.get(("decode", sched))
                if kd and name in ("skeleton", "stream"):
                    r[f"decode_over_reference_{sched}"] = round(ab["total"] / kd / 1e9 / r[f"GBps_{sched}"], 3)
    us = lambda v: round(v * 1e6, 2) if v else None  # noqa: E731
    kernel_name = {"decode": "df11_decode_kernel", "skeleton": "df11_skeleton_kernel",
                   "stream": "df11_stream_kernel"}[args.kernel]
    res = {
        "metric": "decoded BF16 GB/s and % HBM roofline per transformer block, 1 MI355X" if args.kernel == "decode"
        else f"bandwidth reference '{args.kernel}' (moves the decode's bytes without decoding; not the decode)",
        "value": round(2.0 * n / k_head / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(k_head * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "step": ("one launch over the whole block with the caches flushed before it (a 1 GiB read); value and "
                 "ms_per_step from HIP events: (flush, launch) timed between one event pair, minus (flush) timed "
                 "the same way with the launch after its pair, so that the flush and the event marker's dispatch "
                 "delay cancel (wall_ms_per_step: both legs, flushes included)") if args.schedule == "cold" else
                ("one launch over the whole block, launches back to back over device copies of the block; "
                 "value and ms_per_step from one HIP event pair around the timed launches"),
        "wall_ms_per_step": round(wall / args.steps * 1e3, 4),
        "config": {
            "workload": f"{args.workload}: {wl.description}",
            "weights": n,
            "matrices": len(wl.mats),
            "codebook": "shared per block" if wl.shared_codebook else "per matrix",
            "seed": wl.seed,
            "compressed_bytes": int(s.compressed_bytes),
            "bits_per_weight": round(8 * ab["read"] / n, 3),
            "mean_code_len_bits": round(s.mean_code_len_bits, 4),
            "exp_entropy_bits": round(s.exp_entropy_bits, 4),
            "max_code_len": int(s.max_code_len),
            "decode_tables": int(s.n_tables),
            "launch": {"kernel": args.kernel, "schedule": args.schedule, "flush": args.flush,
                       "waves_per_group": args.waves or "default", "max_groups": args.max_groups or "auto",
                       "oversubscribe": args.oversubscribe or "default",
                       "variant": {0: "default (multi-code)", 1: "one code per lookup",
                                   2: "multi-code",
                                   3: "multi-code with stored per-window counts (format variant)"}[args.variant],
                       "layout": "aligned units (format variant)" if args.aligned_units else "the pages' format",
                       "out_offset_bytes": args.out_offset_bytes},
        },
        "gweights_per_s": round(n / k_head / 1e9, 2),
        "pct_hbm_roofline": round(100.0 * achieved / PEAK_HBM_GBS, 2),
        "kernel_us": {args.schedule: ({"mean": us(k_head), "p10": us(pctl(kt, .1)), "p50": us(pctl(kt, .5)),
                                       "p90": us(pctl(kt, .9)), "launches": len(kt)}
                                      if args.schedule == "cold" else {"mean": us(k_head), "launches": args.steps}),
                      "decode_cold": us(k_cold), "decode_rotated": us(k_rot),
                      "decode_same_block_back_to_back": us(times.get(("decode", "same"))),
                      "device_copies_rotated": n_copies},
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "schedule": args.schedule,
            "frac_cold": frac(k_cold),
            "frac_rotated": frac(k_rot),
            "algorithmic_bytes_per_launch": head_bytes,
            "kernel": kernel_name,
        },
        "bandwidth_reference": refs or None,
        "library_stamp": hdb.library_stamp(),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        progress("timing the oracle on the host (cpu_baseline)")
        res["cpu_baseline"] = cpu_baseline(s, x, args.cpu_seconds)
        res["cpu_baseline_1thread"] = cpu_baseline(s, x, args.cpu_seconds / 3, threads=1)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
