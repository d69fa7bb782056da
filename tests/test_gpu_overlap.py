"""GPU: decode-ahead pipelining (block i+1 decoded on a side stream while block
i is consumed).  The weights each consumer sees must be bit-exact; the GEMM
outputs are compared with the same GEMMs on the original weights."""
import numpy as np
import pytest

import df11_inputs as di
import huffman_decode_block_amd as hdb
from huffman_decode_block_amd.overlap import DecodeAhead

pytestmark = pytest.mark.gpu

SHAPES = [(512, 1024), (256, 1024), (1024, 512)]


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "the GPU tests need a GPU"
    return t


def _blocks(torch, n_blocks):
    blocks, originals = [], []
    for b in range(n_blocks):
        mats = [di.random_normal(r * c, 0.02 * (1 + b), 900 + 10 * b + k) for k, (r, c) in enumerate(SHAPES)]
        enc = hdb.df11_encode_block(mats)
        blocks.append(hdb.DeviceBlock.from_encoded(enc))
        originals.append([torch.from_numpy(m.view(np.int16)).to("cuda").view(torch.bfloat16).view(r, c)
                          for m, (r, c) in zip(mats, SHAPES)])
    return blocks, originals


@pytest.mark.parametrize("mode", ["ahead", "inline"])
@pytest.mark.parametrize("order", [[0, 1, 2], [0, 1, 2, 0, 1, 2], [2], [1, 1, 0]])
def test_decode_ahead_feeds_exact_weights(torch, order, mode):
    import torch.nn.functional as F
    print(f"[gpu-test] decode-ahead order={order} mode={mode}", flush=True)
    blocks, originals = _blocks(torch, 3)
    gen = torch.Generator(device="cuda").manual_seed(7)
    xs = {c: torch.randn(64, c, device="cuda", generator=gen).to(torch.bfloat16) for c in (512, 1024)}
    ahead = DecodeAhead(blocks, [SHAPES] * 3, mode=mode)
    stream = torch.cuda.current_stream()
    seen, outs = [], []

    def consume(i, views):
        seen.append((i, [v.clone() for v in views]))
        outs.append((i, [F.linear(xs[v.shape[1]], v) for v in views]))

    ahead.run(consume, stream=stream, order=order)
    torch.cuda.synchronize()
    assert [i for i, _ in seen] == order
    for (i, ws), (_, ys) in zip(seen, outs):
        for w, ref, y in zip(ws, originals[i], ys):
            assert torch.equal(w.view(torch.int16), ref.view(torch.int16)), f"block {i} weights differ"
            y_ref = F.linear(xs[ref.shape[1]], ref)
            # same operands; the GEMM library may pick its algorithm by pointer alignment
            torch.testing.assert_close(y, y_ref, rtol=1e-2, atol=1e-3)


def test_consecutive_runs_do_not_overwrite_a_buffer_still_in_use(torch):
    # the first run's last consumer of each buffer is held back on its stream
    # (a bounded spin) while the second run starts decoding into the same
    # buffers: the second run's decodes must wait for it
    print("[gpu-test] decode-ahead: two runs back to back", flush=True)
    blocks, originals = _blocks(torch, 3)
    ahead = DecodeAhead(blocks, [SHAPES] * 3)
    stream = torch.cuda.current_stream()
    seen = []

    def slow(i, views):
        torch.cuda._sleep(20_000_000)  # about 10 ms of GPU time on the consumer stream
        seen.append((i, [v.clone() for v in views]))

    def quick(i, views):
        seen.append((i, [v.clone() for v in views]))

    ahead.run(slow, stream=stream, order=[0, 1])
    ahead.run(quick, stream=stream, order=[2, 2, 1])
    torch.cuda.synchronize()
    assert [i for i, _ in seen] == [0, 1, 2, 2, 1]
    for i, ws in seen:
        for w, ref in zip(ws, originals[i]):
            assert torch.equal(w.view(torch.int16), ref.view(torch.int16)), f"block {i} weights differ"


def test_auto_mode_picks_a_schedule_per_key_and_mixed_runs_stay_exact(torch):
    """"auto" times both schedules for a new key (calling the consumer), keeps
    the faster, and later runs with that key use it; runs in different
    schedules on the same buffers, back to back, still feed exact weights."""
    print("[gpu-test] decode-ahead: auto mode", flush=True)
    blocks, originals = _blocks(torch, 3)
    ahead = DecodeAhead(blocks, [SHAPES] * 3, mode="auto")
    stream = torch.cuda.current_stream()
    seen = []

    def record(i, views):
        seen.append((i, [v.clone() for v in views]))

    used = ahead.run(record, stream=stream, order=[0, 1, 2], key="k")
    assert used in ("ahead", "inline") and ahead.choice["k"] == used
    assert set(ahead.timings["k"]) == {"ahead", "inline"}
    calls = len(seen)
    assert calls == 3 * (1 + 5) * 2 + 3  # untimed + 5 timed runs per schedule, then the run itself
    assert ahead.run(record, stream=stream, order=[2, 0], key="k") == used
    assert len(seen) == calls + 2
    # explicit schedules alternating on the same buffers
    ahead.mode = "inline"
    ahead.run(record, stream=stream, order=[1, 2])
    ahead.mode = "ahead"
    ahead.run(record, stream=stream, order=[0, 1, 2])
    torch.cuda.synchronize()
    for i, ws in seen:
        for w, ref in zip(ws, originals[i]):
            assert torch.equal(w.view(torch.int16), ref.view(torch.int16)), f"block {i} weights differ"


def test_launch_geometry_applies_to_side_stream_decodes_only(torch, monkeypatch):
    """A capped launch is for decodes that share the GPU with the consumer:
    the side-stream decodes take it, inline decodes use the library default;
    the consumers still see exact weights in both schedules."""
    import huffman_decode_block_amd.overlap as ov
    print("[gpu-test] decode-ahead launch geometry per schedule", flush=True)
    blocks, originals = _blocks(torch, 3)
    stream = torch.cuda.current_stream()
    calls = []
    real = ov.df11_decode_block

    def recording(blk, out=None, stream=None, launch=None):
        calls.append((stream, launch))
        return real(blk, out=out, stream=stream, launch=launch)

    monkeypatch.setattr(ov, "df11_decode_block", recording)
    capped = (8, 512, 0, 0)
    ahead = DecodeAhead(blocks, [SHAPES] * 3, launch=capped)
    for mode in ("ahead", "inline"):
        ahead.mode = mode
        calls.clear()
        seen = []
        ahead.run(lambda i, views: seen.append((i, [v.clone() for v in views])), stream=stream)
        torch.cuda.synchronize()
        assert len(calls) == 3
        for on, launch in calls:
            if mode == "ahead":
                assert on is ahead.side and launch == capped
            else:
                assert on is stream and launch is None
        for i, ws in seen:
            for w, ref in zip(ws, originals[i]):
                assert torch.equal(w.view(torch.int16), ref.view(torch.int16)), f"{mode}: block {i} weights differ"
