"""GPU parity of the aligned-units layout (DF11_ENCODE_ALIGNED_UNITS, a format
variant that is not the pages'): every decode variant, through the C-ABI,
bit for bit against the input and the oracle's unit decode, from the oracle's
sections and from library blobs, with guard regions on both sides of the
output; and full-size C3."""
import numpy as np
import pytest

import df11_inputs as di
import huffman_decode_block_amd as hdb
import oracle

pytestmark = pytest.mark.gpu

GUARD = 64
VARIANTS = [hdb.DF11_VARIANT_SINGLE, hdb.DF11_VARIANT_MULTI, hdb.DF11_VARIANT_COUNTS]


def say(msg):
    print(f"[gpu-test] {msg}", flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "the GPU tests need a GPU"
    return t


def decode_guarded(torch, blk, n, launch):
    buf = torch.full((n + 2 * GUARD,), 0x5A5A, dtype=torch.int16, device="cuda")
    hdb.df11_decode_block(blk, out=buf[GUARD:GUARD + n], launch=launch)
    torch.cuda.synchronize()
    h = buf.cpu().numpy().view(np.uint16)
    assert (h[:GUARD] == 0x5A5A).all() and (h[GUARD + n:] == 0x5A5A).all(), "write outside the output"
    return h[GUARD:GUARD + n].copy()


def cyclic8(n):
    i = np.arange(n)
    return ((120 + (i % 8)) << 7 | (i & 0x7F)).astype(np.uint16)


CASES = {
    "cyclic8": lambda: cyclic8(3 * 1344 + 100),
    "c1": lambda: di.generate("C1"),
    "ragged": lambda: di.random_normal(100_003, 0.02, 5),
    "skew_steep": lambda: di.skewed(200_000, 12, 2.5, 9),
    "skew_flat": lambda: di.skewed(200_000, 256, 0.3, 8),
    "single": lambda: di.single_exponent(100_000, 127, 1),
    "high": lambda: di.high_exponents(100_003, 7),
    "fib34": lambda: di.fibonacci_exponents()[:1_000_000],
    "all_patterns": lambda: di.all_bf16_patterns(3),
    "many_subtables": lambda: di.many_subtables(),
    "tiny": lambda: di.random_normal(5, 0.02, 3),
    "one": lambda: di.random_normal(1, 0.02, 3),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_oracle_sections(torch, case):
    x = CASES[case]()
    o = oracle.encode_aligned_units(x)
    expect = oracle.decode_units(o)
    np.testing.assert_array_equal(expect, x)
    blk = hdb.DeviceBlock.from_parts(code_len=o.code_len, stream=o.stream, sign_mant=o.sign_mant, gaps=o.gaps,
                                     unit_pos=o.unit_pos, n_total=o.n, total_bits=o.total_bits,
                                     counts=oracle.window_counts(o, x), unit_end=o.unit_end)
    for v in VARIANTS:
        say(f"aligned {case}: oracle sections n={x.size} units={o.n_units} variant={v}")
        np.testing.assert_array_equal(decode_guarded(torch, blk, x.size, (0, 0, v)), expect)


@pytest.mark.parametrize("case", sorted(CASES))
def test_library_blob(torch, case):
    x = CASES[case]()
    enc = hdb.df11_encode_block([x], window_counts=True, aligned_units=True)
    blk = hdb.DeviceBlock.from_encoded(enc)
    for launch in [(0, 0, v) for v in VARIANTS] + [(1, 0, 2), (4, 0, 2), (16, 7, 2), (0, 0, 2, 1)]:
        say(f"aligned {case}: library blob n={x.size} launch={launch}")
        np.testing.assert_array_equal(decode_guarded(torch, blk, x.size, launch), x)


@pytest.mark.parametrize("workload", ["C2", "C3"])
def test_full_size(torch, workload):
    x = di.generate(workload)
    enc = hdb.df11_encode_block(di.split(workload, x), window_counts=True, aligned_units=True)
    s = enc.sections
    assert (s.unit_pos[:-1] % 32 == 0).all()
    blk = hdb.DeviceBlock.from_encoded(enc)
    out = torch.empty(x.size, dtype=torch.bfloat16, device="cuda")
    xd = torch.from_numpy(x.view(np.int16)).to("cuda")
    for v in VARIANTS:
        say(f"aligned {workload}: n={x.size} variant={v}")
        out.view(torch.int16).fill_(0x5A5A)
        hdb.df11_decode_block(blk, out=out, launch=(0, 0, v))
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), xd)
