#!/usr/bin/env python3
"""Benchmark: DF11 block decode on one MI355X.

One step = one df11_decode_block launch over a whole transformer block (the
Llama-3.1-8B-shaped block by default: q,k,v,o,gate,up,down, 218,103,808
weights, one shared codebook), inputs resident in HBM.  The timed launches
rotate over device copies of the block, as a model decodes a different block
each time (no launch finds the previous one's sections in the caches).
Prints one JSON line.

  value      decoded BF16 GB/s = 2 * weights * steps / timed seconds
  roofline   algorithmic HBM bytes per launch (compressed sections read +
             BF16 written) / average kernel time from HIP events, vs 8 TB/s
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


def code_tokens(src: str) -> str:
    """The source with comments removed and whitespace runs collapsed, so that
    a change of comments alone keeps the kernel's identity."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if src.startswith("//", i):
            i = src.find("\n", i)
            i = n if i < 0 else i
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


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


def rotation_copies(read_bytes: int, cap: int = 64) -> int:
    """Device copies of a block that the timed launches rotate over: enough
    that their sections add up to twice the Infinity Cache, at least 2, at most
    `cap` (blocks so small that the cap binds stay cached whatever the count)."""
    return int(min(cap, max(2, -(-2 * INFINITY_CACHE_BYTES // max(int(read_bytes), 1)))))


def progress(msg: str) -> None:
    """A progress line on stderr (stdout carries only the result line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def copy_context(n_bytes: int, dev, reps: int = 20) -> dict:
    """A plain device-to-device copy that moves the same HBM bytes as one
    decode (half read, half written), timed the same way: the achievable
    streaming rate on this GPU, reported as context for the decode's rate."""
    import torch
    half = max(16, n_bytes // 2 // 16 * 16)
    src = torch.empty(half, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream(dev)
    for _ in range(5):
        dst.copy_(src)
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    ev[0].record(stream)
    for _ in range(reps):
        dst.copy_(src)
    ev[1].record(stream)
    torch.cuda.synchronize()
    t = ev[0].elapsed_time(ev[1]) * 1e-3 / reps
    del src, dst
    return {"bytes": 2 * half, "copy_us": round(t * 1e6, 2), "copy_GBps": round(2 * half / t / 1e9, 1)}


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
    `batch` tokens) run: the pages' decompress-just-before-use schedule."""
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
    # two device copies of the block in turn, so that no decode finds the
    # previous one's sections in the Infinity Cache (as with different blocks)
    blks = [blk, hdb.DeviceBlock.from_encoded(enc, device=dev)]
    shapes = [(m.rows, m.cols) for m in wl.mats]
    nb = args.overlap_blocks
    ahead = DecodeAhead([blks[i % 2] for i in range(nb)], [shapes] * nb, device=dev)
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

        def gemms_only():
            for i in range(nb):
                consume(i, ref_views)

        def decodes_only():
            for i in range(nb):
                hdb.df11_decode_block(blks[i % 2], out=ahead.bufs[i % 2][: blk.n_total], stream=stream)

        for f in (gemms_only, decodes_only):  # warm up (clocks, GEMM algorithm choice)
            for _ in range(3):
                f()
        torch.cuda.synchronize()
        t_g, t_d = timed(gemms_only) / nb, timed(decodes_only) / nb
        # The ahead-decode's footprint: the whole GPU, or a capped number of
        # workgroups (it then streams on fewer CUs and leaves the rest to the
        # GEMMs, which matters once they are compute-bound).
        per_launch = {}
        for wv, mg in ((0, 0), (0, 256), (8, 0), (8, 512), (4, 0), (4, 1024), (4, 512), (2, 0)):
            ahead.launch = None if (wv, mg) == (0, 0) else (wv, mg, 0, 0)
            for _ in range(2):
                ahead.run(consume, stream=stream)
            per_launch[(wv, mg)] = timed(lambda: ahead.run(consume, stream=stream)) / nb
        ahead.launch = None
        best = min(per_launch, key=per_launch.get)
        t_p = per_launch[best]
        name = lambda k: f"{k[0] or 'default'} waves/group, " + (f"{k[1]} groups" if k[1] else "default grid")  # noqa: E731
        res = {
            "metric": "exposed decode time per block, next block decoded on a side stream during this block's GEMMs",
            "value": round((t_p - t_g) * 1e6, 2), "unit": "us", "higher_is_better": False,
            "batch_tokens": bs, "blocks": nb, "workload": f"{args.workload}: {wl.description}",
            "gemms_only_us_per_block": round(t_g * 1e6, 2),
            "decode_only_us_per_block": round(t_d * 1e6, 2),
            "pipelined_us_per_block": round(t_p * 1e6, 2),
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
    ap.add_argument("--cold-launches", type=int, default=20,
                    help="single launches each after a read of 1 GiB of unrelated data (caches flushed)")
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
    blk = hdb.DeviceBlock.from_encoded(enc, device=dev)
    out = torch.empty(s.n_total, dtype=torch.bfloat16, device=dev)
    launch = (args.waves, args.max_groups, args.variant, args.oversubscribe) \
        if (args.waves or args.max_groups or args.variant or args.oversubscribe) else None
    stream = torch.cuda.current_stream(dev)
    ab = algorithmic_bytes(s, with_counts)

    # A model decodes a different block each time.  The timed launches rotate
    # over device copies of the block (each with its own sections and output)
    # whose sections together are at least twice the 256 MiB Infinity Cache,
    # so no launch finds what the one before it read still cached; decoding
    # one block over and over would find part of it there.
    n_copies = rotation_copies(ab["read"])
    copies = [(blk, out)] + [(hdb.DeviceBlock.from_encoded(enc, device=dev), torch.empty_like(out))
                             for _ in range(n_copies - 1)]

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
    region = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]

    # Untimed pre-warm until the clocks have ramped (not counted as steps),
    # then the W warmup steps, then the K timed steps with no idle between.
    t_pre = time.perf_counter()
    i = 0
    while (time.perf_counter() - t_pre) * 1e3 < args.prewarm_ms:
        for _ in range(50):
            decode(i)
            i += 1
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        decode(i)
        i += 1
    torch.cuda.synchronize()
    # The timed region: K launches back to back on the decode's stream, HIP
    # events at its two ends (the kernel's average launch duration is their
    # interval over K).
    t0 = time.perf_counter()
    region[0].record(stream)
    for k in range(args.steps):
        decode(i + k)
    region[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    k_avg = region[0].elapsed_time(region[1]) * 1e-3 / args.steps
    i += args.steps
    # Spread of single launches, from K more launches each between its own
    # pair of events (the event pair adds a few microseconds to each).
    for k in range(args.steps):
        starts[k].record(stream)
        decode(i + k)
        ends[k].record(stream)
    torch.cuda.synchronize()
    kt = sorted(a.elapsed_time(b) * 1e-3 for a, b in zip(starts, ends))
    # For comparison, K launches that decode the first copy over and over
    # (part of its sections is then still in the Infinity Cache).
    region[0].record(stream)
    for k in range(args.steps):
        decode(0)
    region[1].record(stream)
    torch.cuda.synchronize()
    k_same = region[0].elapsed_time(region[1]) * 1e-3 / args.steps
    # Cold single launches: before each, a read of 1 GiB of unrelated data
    # pushes the block's sections out of the L2 and the Infinity Cache, leaving
    # clean lines (not in any interval).  An int64 sum reads its input as it
    # is (a narrower type would first be copied, i.e. written, to int64).
    scratch = torch.ones(1 << 27, dtype=torch.int64, device=dev)
    cold = []
    ce = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    for k in range(args.cold_launches):
        flush = scratch.sum()
        ce[0].record(stream)
        decode(0)
        ce[1].record(stream)
        torch.cuda.synchronize()
        cold.append(ce[0].elapsed_time(ce[1]) * 1e-3)
    del scratch, flush
    cold.sort()
    xd = torch.from_numpy(x.view(np.int16)).to(dev)  # and of every copy's last decode
    for b, o in copies:
        if not torch.equal(o.view(torch.int16), xd):
            raise SystemExit("decode is not bit-exact after timing; refusing to report a number")
    del xd, copies

    n = int(s.n_total)
    achieved = ab["total"] / k_avg / 1e9
    value = 2.0 * n * args.steps / wall / 1e9
    # the committed counters were taken on the default (multi-code) kernel
    traffic = measured_traffic(args.workload) if args.variant in (0, 2) and not args.aligned_units else None
    if traffic is None:
        progress("roofline.traffic is null: no committed HBM counter summary matches this kernel code, "
                 "workload and variant")
    cc = copy_context(ab["total"], dev)
    cc["decode_over_copy"] = round(achieved / cc["copy_GBps"], 3)
    res = {
        "metric": "decoded BF16 GB/s and % HBM roofline per transformer block, 1 MI355X",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
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
            "launch": {"waves_per_group": args.waves or "default", "max_groups": args.max_groups or "auto",
                       "oversubscribe": args.oversubscribe or "default",
                       "variant": {0: "default (multi-code)", 1: "one code per lookup",
                                   2: "multi-code",
                                   3: "multi-code with stored per-window counts (format variant)"}[args.variant],
                       "layout": "aligned units (format variant)" if args.aligned_units else "the pages' format"},
        },
        "gweights_per_s": round(n * args.steps / wall / 1e9, 2),
        "pct_hbm_roofline": round(100.0 * ab["total"] * args.steps / wall / 1e9 / PEAK_HBM_GBS, 2),
        "kernel_us": {"avg": round(k_avg * 1e6, 2),
                      "single_launch": {"p10": round(kt[len(kt) // 10] * 1e6, 2),
                                        "p50": round(kt[len(kt) // 2] * 1e6, 2),
                                        "p90": round(kt[(9 * len(kt)) // 10] * 1e6, 2)},
                      "cold_single_launch": {"p10": round(cold[len(cold) // 10] * 1e6, 2),
                                             "p50": round(cold[len(cold) // 2] * 1e6, 2),
                                             "p90": round(cold[(9 * len(cold)) // 10] * 1e6, 2),
                                             "launches": len(cold)} if cold else None,
                      "same_block_back_to_back": round(k_same * 1e6, 2),
                      "device_copies_rotated": n_copies},
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": ab["total"],
            "kernel": "df11_decode_kernel",
        },
        "copy_context": cc,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        progress("timing the oracle on the host (cpu_baseline)")
        res["cpu_baseline"] = cpu_baseline(s, x, args.cpu_seconds)
        res["cpu_baseline_1thread"] = cpu_baseline(s, x, args.cpu_seconds / 3, threads=1)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
