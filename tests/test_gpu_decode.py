"""GPU parity: the HIP decode (through the C-ABI) against the oracle, element by
element, bit for bit.  Integer work: zero tolerance.

Every case decodes into a buffer poisoned on both sides (guard regions must
survive) and compares with the oracle's bit-serial decode of the same
sections, and with the input itself (the method is lossless).  Sections come
either from the oracle (the decode is checked independently of the library
encoder) or from the library encoder (the path the benchmark times)."""
import numpy as np
import pytest

import df11_inputs as di
import huffman_decode_block_amd as hdb
import oracle
from conftest import load_golden

pytestmark = pytest.mark.gpu

GUARD = 64  # guard elements on each side (keeps the payload 16-byte aligned)


def say(msg):
    print(f"[gpu-test] {msg}", flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "the GPU tests need a GPU"
    return t


def oracle_view(s):
    """The library's sections as the oracle's Encoded record (plain arrays)."""
    return oracle.Encoded(n=int(s.n_total), total_bits=int(s.total_bits), n_windows=int(s.n_windows),
                          n_units=int(s.n_units), code_len=s.code_len, stream=s.stream,
                          sign_mant=s.sign_mant, gaps=s.gaps, unit_pos=s.unit_pos,
                          max_len=int(s.max_code_len))


def decode_guarded(torch, blk, n, poison, launch=None, stream=None, lead=GUARD):
    """Decodes into a view `lead` elements into a poisoned buffer (torch's
    allocations start on 512-byte boundaries, so lead = GUARD puts the output
    on a 64-byte boundary, GUARD + 8k on a 16k-byte offset from one)."""
    buf = torch.full((n + lead + GUARD,), poison, dtype=torch.int16, device="cuda")
    view = buf[lead:lead + n]
    hdb.df11_decode_block(blk, out=view, stream=stream, launch=launch)
    torch.cuda.synchronize()
    h = buf.cpu().numpy().view(np.uint16)
    p = np.uint16(poison & 0xFFFF)
    assert (h[:lead] == p).all(), "write below the output"
    assert (h[lead + n:] == p).all(), "write past the output"
    return h[lead:lead + n].copy()


def check_oracle_sections(torch, x, name, variants=(0,)):
    o = oracle.encode(x)
    expect = oracle.decode(o)
    np.testing.assert_array_equal(expect, x)
    counts = oracle.window_counts(o, decoded=expect) if hdb.DF11_VARIANT_COUNTS in variants else None
    blk = hdb.DeviceBlock.from_parts(code_len=o.code_len, stream=o.stream, sign_mant=o.sign_mant,
                                     gaps=o.gaps, unit_pos=o.unit_pos, n_total=o.n,
                                     total_bits=o.total_bits, counts=counts)
    for variant in variants:
        for poison in (0x5A5A, -1):
            say(f"{name}: oracle sections n={x.size} max_len={o.max_len} variant={variant} "
                f"poison={poison & 0xFFFF:#x}")
            y = decode_guarded(torch, blk, x.size, poison, launch=(0, 0, variant))
            np.testing.assert_array_equal(y, expect)


VARIANTS = [hdb.DF11_VARIANT_SINGLE, hdb.DF11_VARIANT_MULTI, hdb.DF11_VARIANT_COUNTS]


def check_library_blob(torch, x, name, mats=None, launch=None):
    with_counts = launch is not None and len(launch) > 2 and launch[2] == hdb.DF11_VARIANT_COUNTS
    enc = hdb.df11_encode_block(mats if mats is not None else [x], window_counts=with_counts)
    s = enc.sections
    blk = hdb.DeviceBlock.from_encoded(enc)
    say(f"{name}: library blob n={x.size} tables={s.n_tables} max_len={s.max_code_len} launch={launch}")
    y = decode_guarded(torch, blk, x.size, 0x5A5A, launch=launch)
    np.testing.assert_array_equal(y, oracle.decode(oracle_view(s)))
    np.testing.assert_array_equal(y, x)
    return enc, blk


EDGE = {
    "all_patterns": lambda: di.all_bf16_patterns(),
    "all_patterns_perm": lambda: di.all_bf16_patterns(5),
    "high_exponents": lambda: di.high_exponents(100_003, 7),
    "single_1": lambda: di.single_exponent(1, 127, 1),
    "single_5": lambda: di.single_exponent(5, 0, 2),
    "single_4097": lambda: di.single_exponent(4097, 255, 3),
    "single_300k": lambda: di.single_exponent(300_000, 119, 4),
    "fibonacci34_len32": lambda: di.fibonacci_exponents(),
    "many_subtables_global": lambda: di.many_subtables(),
    "skew_flat": lambda: di.skewed(400_000, 256, 0.3, 8),
    "skew_steep": lambda: di.skewed(400_000, 12, 2.5, 9),
    "c1": lambda: di.generate("C1"),
}


@pytest.mark.parametrize("name", ["v1_mixed_small", "v3_single_exponent", "v5_straddle_window",
                                  "v6_last_window_without_start"])
def test_golden_vectors(torch, name):
    check_oracle_sections(torch, np.array(load_golden(name)["x"], dtype=np.uint16), name, VARIANTS)


@pytest.mark.parametrize("n", [1, 2, 7, 63, 64, 65, 255, 4095, 4096, 4097, 8191, 262_143,
                               262_145, 1_000_003])
def test_ragged_sizes(torch, n):
    check_oracle_sections(torch, di.random_normal(n, 0.02, 500 + n), f"ragged_{n}", VARIANTS)


@pytest.mark.parametrize("case", sorted(EDGE))
def test_edge_inputs_oracle_sections(torch, case):
    check_oracle_sections(torch, EDGE[case](), case, VARIANTS)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("case", sorted(EDGE))
def test_edge_inputs_library_blob(torch, case, variant):
    check_library_blob(torch, EDGE[case](), case, launch=(0, 0, variant))


def test_empty_block_is_a_noop(torch):
    enc = hdb.df11_encode_block([np.zeros(0, np.uint16)])
    blk = hdb.DeviceBlock.from_encoded(enc)
    buf = torch.full((16,), 7, dtype=torch.int16, device="cuda")
    hdb.df11_decode_block(blk, out=buf[:0])
    torch.cuda.synchronize()
    assert (buf.cpu() == 7).all()


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("waves", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("max_groups,over", [(0, 0), (1, 0), (7, 0), (0, 1), (0, 64)])
def test_launch_geometry_does_not_change_the_output(torch, waves, max_groups, over, variant):
    x = di.generate("C1") if max_groups == 1 else di.random_normal(3_000_000, 0.02, 77)
    check_library_blob(torch, x, f"geometry_w{waves}_g{max_groups}_o{over}_v{variant}",
                       launch=(waves, max_groups, variant, over))


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("offset_bytes", [16, 32, 48])
def test_output_off_a_64_byte_boundary(torch, offset_bytes, variant):
    """Outputs that start 16, 32 or 48 bytes past a 64-byte boundary (a view
    such as big[8:]): the kernel finds the 64-byte sectors it shares with
    neighbouring units from the output's address, and the result is the
    same."""
    x = di.random_normal(1_000_003, 0.02, 90 + offset_bytes)
    enc = hdb.df11_encode_block([x], window_counts=True)
    blk = hdb.DeviceBlock.from_encoded(enc)
    say(f"output offset {offset_bytes} B, variant {variant}")
    y = decode_guarded(torch, blk, x.size, 0x5A5A, launch=(0, 0, variant), lead=GUARD + offset_bytes // 2)
    np.testing.assert_array_equal(y, x)


def test_workload_c2(torch):
    x = di.generate("C2")
    check_oracle_sections(torch, x, "C2", VARIANTS)
    for v in VARIANTS:
        check_library_blob(torch, x, "C2", launch=(0, 0, v))


def test_side_stream(torch):
    x = di.random_normal(2_000_000, 0.01, 5)
    enc = hdb.df11_encode_block([x])
    blk = hdb.DeviceBlock.from_encoded(enc)
    side = torch.cuda.Stream()
    out = torch.empty(x.size, dtype=torch.bfloat16, device="cuda")
    say("side stream decode")
    with torch.cuda.stream(side):
        hdb.df11_decode_block(blk, out=out, stream=side)
    side.synchronize()
    np.testing.assert_array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), x)


def test_device_side_errors(torch):
    x = di.random_normal(10_000, 0.02, 6)
    blk = hdb.DeviceBlock.from_encoded(hdb.df11_encode_block([x]))
    small = torch.empty(x.size - 1, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(hdb.DF11Error) as ei:
        hdb.df11_decode_block(blk, out=small)
    assert ei.value.status == hdb.DF11_E_BUFFER_TOO_SMALL
    big = torch.empty(x.size + 8, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(hdb.DF11Error) as ei:
        hdb.df11_decode_block(blk, out=big[1:])
    assert ei.value.status == hdb.DF11_E_INVALID_ARG
    # the counting-free variant needs a blob with window counts
    ok = torch.empty(x.size, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(hdb.DF11Error) as ei:
        hdb.df11_decode_block(blk, out=ok, launch=(0, 0, hdb.DF11_VARIANT_COUNTS))
    assert ei.value.status == hdb.DF11_E_INVALID_ARG


def _full_block(torch, key, variants=(0,)):
    say(f"{key}: generating")
    x = di.generate(key)
    mats = di.split(key, x)
    say(f"{key}: encoding {x.size} weights")
    enc = hdb.df11_encode_block(mats, window_counts=hdb.DF11_VARIANT_COUNTS in variants)
    s = enc.sections
    assert hdb.df11_validate(s) == hdb.DF11_OK
    blk = hdb.DeviceBlock.from_encoded(enc)
    out = torch.empty(x.size, dtype=torch.bfloat16, device="cuda")
    xd = torch.from_numpy(x.view(np.int16)).to("cuda")
    ref = None
    for variant in variants:
        out.view(torch.int16).fill_(0x5A5A)
        say(f"{key}: decoding units={s.n_units} tables={s.n_tables} max_len={s.max_code_len} "
            f"variant={variant}")
        hdb.df11_decode_block(blk, out=out, launch=(0, 0, variant))
        torch.cuda.synchronize()
        ident = bool(torch.equal(out.view(torch.int16), xd))
        say(f"{key}: identity {ident}; oracle decode of every unit")
        y = out.view(torch.int16).cpu().numpy().view(np.uint16)
        if ref is None:
            ref = oracle.decode_units(oracle_view(s), threads=16)
        np.testing.assert_array_equal(y, ref)
        assert ident
        del y
    del xd
    # per-matrix views
    wl = di.WORKLOADS[key]
    views = hdb.matrix_views(out, blk, [(m.rows, m.cols) for m in wl.mats])
    for v, m in zip(views, mats):
        assert tuple(v.shape) == (v.shape[0], v.shape[1]) and v.numel() == m.size
    return x, enc


def test_workload_c3_full(torch):
    x, enc = _full_block(torch, "C3", VARIANTS)
    # the library's sections equal the oracle's own encoding at full size
    say("C3: oracle encode for section parity")
    o = oracle.encode(x)
    s = enc.sections
    for a, b in [(s.stream, o.stream), (s.sign_mant, o.sign_mant), (s.gaps, o.gaps),
                 (s.unit_pos, o.unit_pos), (s.code_len, o.code_len)]:
        np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(s.counts[:s.n_windows], oracle.window_counts(o, decoded=x))


def test_workload_c4_full(torch):
    _full_block(torch, "C4", VARIANTS)


def test_workload_c5_full(torch):
    _full_block(torch, "C5", VARIANTS)


def test_workload_e8_full(torch):
    """A single large matrix with its own codebook: the token embedding / LM
    head of a Llama-3.1-8B-shaped model (128256 x 4096), one launch."""
    _full_block(torch, "E8", VARIANTS)
