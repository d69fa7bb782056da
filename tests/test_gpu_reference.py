"""GPU checks of the bandwidth references (df11_bandwidth_reference): the
two streaming kernels that move a decode's HBM bytes without decoding write
out[i] = weight i with its exponent field zero, for every i, the writes-only
one zeros, the reads-only one nothing, and none writes outside the output,
for any size, output offset and launch geometry."""
import numpy as np
import pytest

import df11_inputs as di
import huffman_decode_block_amd as hdb

pytestmark = pytest.mark.gpu

GUARD = 64
KINDS = {"skeleton": hdb.DF11_REFERENCE_SKELETON, "stream": hdb.DF11_REFERENCE_STREAM,
         "writes": hdb.DF11_REFERENCE_WRITES, "reads": hdb.DF11_REFERENCE_READS}
FILL = 0x5A5A


def expected(kname, x):
    """What a reference leaves in an output pre-filled with FILL."""
    if kname == "writes":
        return np.zeros_like(x)
    if kname == "reads":
        return np.full_like(x, FILL)
    return x & np.uint16(0x807F)


def say(msg):
    print(f"[gpu-test] {msg}", flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "the GPU tests need a GPU"
    return t


def run_guarded(torch, blk, n, kind, lead=GUARD, launch=None):
    buf = torch.full((n + lead + GUARD,), FILL, dtype=torch.int16, device="cuda")
    hdb.df11_bandwidth_reference(blk, buf[lead:lead + n], kind, launch=launch)
    torch.cuda.synchronize()
    h = buf.cpu().numpy().view(np.uint16)
    assert (h[:lead] == FILL).all(), "write below the output"
    assert (h[lead + n:] == FILL).all(), "write past the output"
    return h[lead:lead + n]


def check(torch, x, name, lead=GUARD, launch=None):
    blk = hdb.DeviceBlock.from_encoded(hdb.df11_encode_block([x]))
    for kname, kind in KINDS.items():
        say(f"{name}: {kname} n={x.size} lead={lead} launch={launch}")
        y = run_guarded(torch, blk, x.size, kind, lead, launch)
        np.testing.assert_array_equal(y, expected(kname, x))


@pytest.mark.parametrize("n", [1, 7, 8, 4095, 4096, 4097, 65_535, 1_000_003])
def test_reference_sizes(torch, n):
    check(torch, di.random_normal(n, 0.02, 300 + n), f"n{n}")


@pytest.mark.parametrize("offset_bytes", [16, 32, 48])
def test_reference_output_offsets(torch, offset_bytes):
    check(torch, di.random_normal(500_001, 0.02, 7), f"off{offset_bytes}", lead=GUARD + offset_bytes // 2)


@pytest.mark.parametrize("launch", [(1, 0, 0, 0), (4, 7, 0, 0), (16, 0, 0, 1), (8, 1, 0, 0), (2, 0, 0, 64)])
def test_reference_launch_geometry(torch, launch):
    check(torch, di.random_normal(2_000_000, 0.01, 8), "geometry", launch=launch)


def test_reference_edge_inputs(torch):
    check(torch, di.all_bf16_patterns(3), "all_patterns")
    check(torch, di.single_exponent(4097, 255, 3), "single_4097")
    check(torch, di.fibonacci_exponents(), "fibonacci34")


def test_reference_full_c3(torch):
    """The headline workload at full size, as the benchmark runs it."""
    x = di.generate("C3")
    enc = hdb.df11_encode_block(di.split("C3", x))
    blk = hdb.DeviceBlock.from_encoded(enc)
    xd = torch.from_numpy(x.view(np.int16)).to("cuda")
    expect = torch.bitwise_and(xd, torch.tensor(-32641, dtype=torch.int16, device="cuda"))
    out = torch.empty(x.size, dtype=torch.int16, device="cuda")
    for kname, kind in KINDS.items():
        say(f"C3: {kname}")
        out.fill_(FILL)
        hdb.df11_bandwidth_reference(blk, out, kind)
        torch.cuda.synchronize()
        want = {"writes": torch.zeros_like(out), "reads": torch.full_like(out, FILL)}.get(kname, expect)
        assert torch.equal(out, want)


def test_reference_refuses_format_variants_and_unknown_kinds(torch):
    x = di.random_normal(10_000, 0.02, 9)
    out = torch.empty(x.size, dtype=torch.bfloat16, device="cuda")
    for kw in ({"window_counts": True}, {"aligned_units": True}):
        blk = hdb.DeviceBlock.from_encoded(hdb.df11_encode_block([x], **kw))
        with pytest.raises(hdb.DF11Error) as ei:
            hdb.df11_bandwidth_reference(blk, out, hdb.DF11_REFERENCE_SKELETON)
        assert ei.value.status == hdb.DF11_E_UNSUPPORTED
    blk = hdb.DeviceBlock.from_encoded(hdb.df11_encode_block([x]))
    with pytest.raises(hdb.DF11Error) as ei:
        hdb.df11_bandwidth_reference(blk, out, 7)
    assert ei.value.status == hdb.DF11_E_INVALID_ARG
    with pytest.raises(hdb.DF11Error) as ei:
        hdb.df11_bandwidth_reference(blk, out[:-1], hdb.DF11_REFERENCE_STREAM)
    assert ei.value.status == hdb.DF11_E_BUFFER_TOO_SMALL
