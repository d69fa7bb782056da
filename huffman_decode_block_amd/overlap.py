"""Decode the next transformer block while the current one is consumed.

The pages decompress a block's weights just before its matrix multiplications
and drop them after, so that only one block is resident in BF16 at a time and
the decode cost does not grow with the batch (hada.io summary of the DFloat11
paper, sections "Decompression par bloc transformer" and "Noyau GPU en deux
etapes et metadonnees auxiliaires").  This module schedules that with two BF16
buffers: block i+1 is decoded on a side stream into one buffer while the
caller's stream consumes block i from the other, and HIP events order the two
streams (decode i+1 waits until block i-1's consumer released its buffer; the
consumer of block i waits for its decode).  It only enqueues launches: every
step of the decode runs in the library's kernel.
"""
from __future__ import annotations

from typing import Callable, Sequence

from . import DeviceBlock, df11_decode_block, matrix_views


class DecodeAhead:
    """Double-buffered block decode on a side stream.

    blocks  encoded blocks already in device memory (``DeviceBlock``)
    shapes  per block, the (rows, cols) of its matrices in storage order
    """

    def __init__(self, blocks: Sequence[DeviceBlock], shapes: Sequence[Sequence[tuple]], device=None,
                 side_stream=None, launch=None):
        import torch
        if len(blocks) != len(shapes):
            raise ValueError("one shape list per block")
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
        # per buffer: event after its last consumer, kept across run() calls so
        # that the next call's first decodes wait for the previous call's last
        # consumers
        self._released = [None, None]

    def run(self, consume: Callable[[int, list], None], stream=None, order: Sequence[int] | None = None):
        """For each block index in `order` (default: all, in order), call
        ``consume(i, views)`` with that block's decoded matrices; ``consume``
        must enqueue its work on `stream` (default: the current stream).
        Returns once everything is enqueued (nothing is synchronized)."""
        torch = self.torch
        stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        order = list(range(len(self.blocks))) if order is None else list(order)
        for t in self.bufs:
            t.record_stream(stream)
        released = self._released

        def decode(k):
            i, b = order[k], k % 2
            if released[b] is not None:  # the consumer of block k-2 is done with this buffer
                self.side.wait_event(released[b])
            buf = self.bufs[b][: int(self.blocks[i].raw.n_total)]
            df11_decode_block(self.blocks[i], out=buf, stream=self.side, launch=self.launch)
            ev = torch.cuda.Event()
            ev.record(self.side)
            return buf, ev

        pending = decode(0) if order else None
        for k, i in enumerate(order):
            buf, ready = pending
            if k + 1 < len(order):
                pending = decode(k + 1)  # runs on the side stream while block k is consumed
            stream.wait_event(ready)
            consume(i, matrix_views(buf, self.blocks[i], self.shapes[i]))
            ev = torch.cuda.Event()
            ev.record(stream)
            released[k % 2] = ev
