"""Decode the next transformer block while the current one is consumed.

The pages decompress a block's weights just before its matrix multiplications
and drop them after, so that only one block is resident in BF16 at a time and
the decode cost does not grow with the batch (hada.io summary of the DFloat11
paper, sections "Decompression par bloc transformer" and "Noyau GPU en deux
etapes et metadonnees auxiliaires").  This module schedules that with two BF16
buffers: block i+1 is decoded on a side stream into one buffer while the
caller's stream consumes block i from the other, and HIP events order the two
streams (decode i+1 waits until block i-1's consumer released its buffer; the
consumer of block i waits for its decode).  Overlap is not always a gain: a
consumer that already keeps every compute unit busy only shares them with the
decode, so the same blocks can also be decoded inline, on the consumer's own
stream right before use, and an "auto" mode times both once per key (say, a
batch size) and keeps the faster.  It only enqueues launches: every step of
the decode runs in the library's kernel.
"""
from __future__ import annotations

from typing import Callable, Sequence

from . import DeviceBlock, df11_decode_block, matrix_views


class DecodeAhead:
    """Double-buffered block decode, ahead on a side stream or inline.

    blocks  encoded blocks already in device memory (``DeviceBlock``)
    shapes  per block, the (rows, cols) of its matrices in storage order
    mode    "ahead": block i+1 is decoded on the side stream while block i is
            consumed; "inline": each block is decoded on the consumer's stream
            right before its consumer (no overlap, nothing competes with the
            consumer); "auto": the first run for a given `key` times both
            schedules and every later run with that key uses the faster one.
            Overlap pays when the consumer leaves memory bandwidth or compute
            units idle, and costs when it does not (a compute-bound consumer
            at large batch shares its units with the decode).
    launch  launch geometry of the side-stream decodes (as for
            ``df11_decode_block``), e.g. a capped grid that leaves compute
            units to the consumer; None for the library's default.  Inline
            decodes share the GPU with nothing and always use the default.
    """

    MODES = ("ahead", "inline", "auto")

    def __init__(self, blocks: Sequence[DeviceBlock], shapes: Sequence[Sequence[tuple]], device=None,
                 side_stream=None, launch=None, mode: str = "ahead"):
        import torch
        if len(blocks) != len(shapes):
            raise ValueError("one shape list per block")
        if mode not in self.MODES:
            raise ValueError(f"mode must be one of {self.MODES}")
        self.torch = torch
        self.blocks = list(blocks)
        self.shapes = [list(s) for s in shapes]
        self.device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        n_max = max((int(b.raw.n_total) for b in self.blocks), default=0)
        self.bufs = [torch.empty(n_max, dtype=torch.bfloat16, device=self.device) for _ in range(2)]
        # default priority: streams of other priorities are not used here
        self.side = side_stream if side_stream is not None else torch.cuda.Stream(self.device)
        for t in self.bufs:  # the allocator must not reuse them before the side stream is done
            t.record_stream(self.side)
        self.launch = launch
        self.mode = mode
        self.choice = {}    # key -> "ahead" | "inline", filled by calibrate()
        self.timings = {}   # key -> {schedule: seconds per run}
        # per buffer: event after its last consumer, kept across run() calls so
        # that the next call's first decodes wait for the previous call's last
        # consumers (in either schedule)
        self._released = [None, None]

    # overlap is kept only when it beats the inline order by more than this
    # fraction: closer than that, run-to-run noise (2-3 % on GEMM-heavy
    # consumers) decides, and the inline order is the serial order itself
    # (nothing competes with the consumer)
    MARGIN = 0.03

    def calibrate(self, consume: Callable[[int, list], None], stream=None, order: Sequence[int] | None = None,
                  key=None, reps: int = 5) -> str:
        """Times both schedules on this consumer (each run `reps` times after
        one untimed run, alternating between the two, HIP events on
        `stream`; synchronizes; the median time of each), keeps the faster one
        for `key` (the inline order unless overlap wins by more than MARGIN)
        and returns it.  `consume` is called by every run, so it must be safe
        to repeat."""
        torch = self.torch
        stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        runs = {"inline": [], "ahead": []}
        for sched in runs:
            self._run(consume, stream, order, sched)
        for _ in range(reps):
            for sched in runs:
                torch.cuda.synchronize(self.device)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                self._run(consume, stream, order, sched)
                b.record(stream)
                torch.cuda.synchronize(self.device)
                runs[sched].append(a.elapsed_time(b) * 1e-3)
        med = {sched: sorted(v)[len(v) // 2] for sched, v in runs.items()}
        self.timings[key] = med
        self.choice[key] = "ahead" if med["ahead"] < med["inline"] * (1.0 - self.MARGIN) else "inline"
        return self.choice[key]

    def run(self, consume: Callable[[int, list], None], stream=None, order: Sequence[int] | None = None,
            key=None) -> str:
        """For each block index in `order` (default: all, in order), call
        ``consume(i, views)`` with that block's decoded matrices; ``consume``
        must enqueue its work on `stream` (default: the current stream).
        Returns the schedule used; once everything is enqueued (nothing is
        synchronized, except for the calibration of a new key in "auto"
        mode)."""
        torch = self.torch
        stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        sched = self.mode
        if sched == "auto":
            sched = self.choice.get(key) or self.calibrate(consume, stream, order, key)
        self._run(consume, stream, order, sched)
        return sched

    def _run(self, consume, stream, order, sched):
        torch = self.torch
        order = list(range(len(self.blocks))) if order is None else list(order)
        for t in self.bufs:
            t.record_stream(stream)
        released = self._released

        def decode(k, on):
            i, b = order[k], k % 2
            if released[b] is not None and on is not stream:  # the consumer of block k-2 is done with it
                on.wait_event(released[b])
            buf = self.bufs[b][: int(self.blocks[i].raw.n_total)]
            df11_decode_block(self.blocks[i], out=buf, stream=on, launch=self.launch if on is not stream else None)
            if on is stream:
                return buf, None
            ev = torch.cuda.Event()
            ev.record(on)
            return buf, ev

        if sched == "inline":
            for k, i in enumerate(order):
                buf, _ = decode(k, stream)  # stream order puts it after the consumer of block k-2
                consume(i, matrix_views(buf, self.blocks[i], self.shapes[i]))
                # Only the last consumer of each buffer needs an event (for a
                # later run that decodes ahead on the side stream): an event
                # recorded between two kernels delays the next one's start by
                # several microseconds.
                if k >= len(order) - 2:
                    ev = torch.cuda.Event()
                    ev.record(stream)
                    released[k % 2] = ev
            return
        pending = decode(0, self.side) if order else None
        for k, i in enumerate(order):
            buf, ready = pending
            if k + 1 < len(order):
                pending = decode(k + 1, self.side)  # runs on the side stream while block k is consumed
            stream.wait_event(ready)
            consume(i, matrix_views(buf, self.blocks[i], self.shapes[i]))
            ev = torch.cuda.Event()
            ev.record(stream)
            released[k % 2] = ev
