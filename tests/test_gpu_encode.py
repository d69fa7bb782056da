"""GPU parity of the GPU-side encoder: every section byte for byte against
the host encoder (itself byte-for-byte equal to the oracle, see
test_encoder_parity.py) and, for a few inputs, the oracle directly; then the
GPU decode of the GPU-encoded block must give back the input."""
import numpy as np
import pytest

import df11_inputs as di
import huffman_decode_block_amd as hdb
import oracle
from conftest import load_golden

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-test] {msg}", flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "the GPU tests need a GPU"
    return t


def check(torch, x, name, counts=False, with_oracle=False):
    say(f"gpu encode {name}: n={x.size} counts={counts}")
    xd = torch.from_numpy(x.view(np.int16)).to("cuda")
    g = hdb.gpu_encode(xd, window_counts=counts)
    s = hdb.df11_encode_block([x], window_counts=counts).sections
    p = g.plan
    assert bytes(p.code_len) == bytes(s.code_len) and p.total_bits == s.total_bits
    np.testing.assert_array_equal(g.section("stream")[:p.stream_bytes], s.stream)
    np.testing.assert_array_equal(g.section("sign_mant")[:p.sign_mant_bytes], s.sign_mant)
    np.testing.assert_array_equal(g.section("gaps")[:p.gaps_bytes], s.gaps)
    np.testing.assert_array_equal(g.section("unit_pos").view(np.uint64), s.unit_pos)
    if counts:
        np.testing.assert_array_equal(g.section("counts"), s.counts)
    if with_oracle:
        o = oracle.encode(x)
        np.testing.assert_array_equal(g.section("stream")[:o.stream.size], o.stream)
        np.testing.assert_array_equal(g.section("gaps")[:o.gaps.size], o.gaps)
        np.testing.assert_array_equal(g.section("unit_pos").view(np.uint64), o.unit_pos)
    # round trip through the GPU decoder
    out = torch.empty(max(1, x.size), dtype=torch.bfloat16, device="cuda")
    variants = (hdb.DF11_VARIANT_MULTI, hdb.DF11_VARIANT_COUNTS) if counts else (hdb.DF11_VARIANT_MULTI,)
    for v in variants:
        out.view(torch.int16).fill_(0x5A5A)
        hdb.df11_decode_block(g.block, out=out[:x.size], launch=(0, 0, v))
        torch.cuda.synchronize()
        assert torch.equal(out[:x.size].view(torch.int16), xd), f"{name}: decode of the GPU encoding differs"
    return g


@pytest.mark.parametrize("name", ["v1_mixed_small", "v3_single_exponent", "v5_straddle_window",
                                  "v6_last_window_without_start"])
def test_golden_vectors(torch, name):
    check(torch, np.array(load_golden(name)["x"], dtype=np.uint16), name, counts=True, with_oracle=True)


@pytest.mark.parametrize("n", [1, 2, 15, 16, 17, 4095, 4096, 4097, 8193, 65_537, 262_145, 1_000_003])
def test_ragged_sizes(torch, n):
    check(torch, di.random_normal(n, 0.02, 700 + n), f"ragged_{n}", counts=(n % 2 == 1))


EDGE = {
    "all_patterns": lambda: di.all_bf16_patterns(),
    "all_patterns_perm": lambda: di.all_bf16_patterns(5),
    "high_exponents": lambda: di.high_exponents(100_003, 7),
    "single_300k": lambda: di.single_exponent(300_000, 119, 4),
    "fibonacci34_len32": lambda: di.fibonacci_exponents(),
    "many_subtables": lambda: di.many_subtables(),
    "skew_flat": lambda: di.skewed(400_000, 256, 0.3, 8),
    "skew_steep": lambda: di.skewed(400_000, 12, 2.5, 9),
    "c1": lambda: di.generate("C1"),
}


@pytest.mark.parametrize("case", sorted(EDGE))
def test_edge_inputs(torch, case):
    check(torch, EDGE[case](), case, counts=True, with_oracle=case in ("c1", "fibonacci34_len32"))


def test_histogram(torch):
    x = di.generate("C2")
    xd = torch.from_numpy(x.view(np.int16)).to("cuda")
    for n in (x.size, x.size - 3, 4096 * 37 + 1, 4095, 7, 0):
        h = torch.empty(256, dtype=torch.int64, device="cuda")
        nb = hdb.df11_gpu_chunk_hist_bytes(n)
        assert nb == 512 * ((n + 4095) // 4096)
        ch = torch.full((max(8, nb // 2),), -1, dtype=torch.int16, device="cuda")
        hdb.df11_gpu_histogram(xd[:n], h, ch)
        torch.cuda.synchronize()
        e = (x[:n] >> 7) & 0xFF
        np.testing.assert_array_equal(h.cpu().numpy(), np.bincount(e, minlength=256))
        got = ch.cpu().numpy().view(np.uint16)[:nb // 2].reshape(-1, 256)
        for c in range(got.shape[0]):
            np.testing.assert_array_equal(got[c], np.bincount(e[4096 * c:4096 * (c + 1)], minlength=256))
        h2 = torch.empty(256, dtype=torch.int64, device="cuda")
        hdb.df11_gpu_histogram(xd[:n], h2)  # without the per-chunk counts
        torch.cuda.synchronize()
        assert torch.equal(h, h2)


def test_histogram_when_the_exponent_mode_moves_between_chunks(torch):
    """The histogram pass counts a window of exponents around the previous
    chunk's most frequent one in per-lane counters and the rest with shared
    atomics: chunks whose distributions jump (small and large scales, one
    exponent, every exponent, exponents 0 and 255 at the edges of the range),
    in an order that moves the window up, down and to both ends, give the
    same counts as numpy, per chunk and in total."""
    rng = np.random.default_rng(21)
    parts = []
    for k, kind in enumerate(["n-2", "n-30", "single255", "all", "n-2", "single0", "t", "n-9", "all", "single128",
                              "n-2", "n-30"] * 4):
        if kind.startswith("n"):
            v = rng.normal(0, 2.0 ** int(kind[1:]), 4096 * (1 + k % 3)).astype(np.float32)
            parts.append((v.view(np.uint32) >> 16).astype(np.uint16))
        elif kind.startswith("single"):
            parts.append(di.single_exponent(4096 * (1 + k % 2), int(kind[6:]), k))
        elif kind == "all":
            parts.append(di.all_bf16_patterns(k)[:4096 * 3])
        else:
            v = (rng.standard_t(3, 4096) * 1e-3).astype(np.float32)
            parts.append((v.view(np.uint32) >> 16).astype(np.uint16))
    x = np.concatenate(parts)
    x = x[: x.size - 1234]  # a ragged last chunk
    xd = torch.from_numpy(x.view(np.int16)).to("cuda")
    h = torch.empty(256, dtype=torch.int64, device="cuda")
    nb = hdb.df11_gpu_chunk_hist_bytes(x.size)
    ch = torch.full((nb // 2,), -1, dtype=torch.int16, device="cuda")
    say(f"histogram with moving modes: n={x.size}")
    hdb.df11_gpu_histogram(xd, h, ch)
    torch.cuda.synchronize()
    e = (x >> 7) & 0xFF
    np.testing.assert_array_equal(h.cpu().numpy(), np.bincount(e, minlength=256))
    got = ch.cpu().numpy().view(np.uint16).reshape(-1, 256)
    want = np.stack([np.bincount(e[4096 * c:4096 * (c + 1)], minlength=256) for c in range(got.shape[0])])
    np.testing.assert_array_equal(got, want)
    # and the whole encoder on it
    check(torch, x, "moving modes", counts=True)


def test_histogram_window_follows_each_waves_chunks(torch):
    """With more chunks than histogram waves (3 workgroups of 4 waves per CU:
    3,072 on 256 CUs), each wave counts several chunks in turn and places
    each chunk's window from the one before: here the scale changes every
    2,048 chunks, so the chunks of one wave jump between scales, one exponent
    (0, 127, 255), every pattern and heavy tails, and the windows move up,
    down, to both ends and miss most weights; the block's last chunk is
    partial and is counted by the wave whose turn it is.  Counts per chunk
    and in total must still equal numpy's."""
    rng = np.random.default_rng(33)
    groups, chunk = 2048, 4096
    kinds = ["n-2", "n-30", "single255", "all", "n-9", "single0", "t", "n-2", "single127", "n-5"]
    parts = []
    for r, kind in enumerate(kinds):  # chunks r * 2048 .. r * 2048 + 2047
        m = groups * chunk
        if kind.startswith("n"):
            v = rng.normal(0, 2.0 ** int(kind[1:]), m).astype(np.float32)
            parts.append((v.view(np.uint32) >> 16).astype(np.uint16))
        elif kind.startswith("single"):
            parts.append(di.single_exponent(m, int(kind[6:]), r))
        elif kind == "all":
            parts.append(np.tile(di.all_bf16_patterns(r), m // 65536))
        else:
            v = (rng.standard_t(2, m) * 1e-2).astype(np.float32)
            parts.append((v.view(np.uint32) >> 16).astype(np.uint16))
    x = np.concatenate(parts)
    x = x[: x.size - 777]  # a ragged last chunk
    n_chunks = (x.size + chunk - 1) // chunk
    assert n_chunks > 4 * groups
    xd = torch.from_numpy(x.view(np.int16)).to("cuda")
    h = torch.empty(256, dtype=torch.int64, device="cuda")
    ch = torch.full((hdb.df11_gpu_chunk_hist_bytes(x.size) // 2,), -1, dtype=torch.int16, device="cuda")
    say(f"histogram, several chunks per wave: n={x.size}")
    hdb.df11_gpu_histogram(xd, h, ch)
    torch.cuda.synchronize()
    e = ((x >> 7) & 0xFF).astype(np.int64)
    np.testing.assert_array_equal(h.cpu().numpy(), np.bincount(e, minlength=256))
    want = np.bincount(np.arange(x.size) // chunk * 256 + e, minlength=n_chunks * 256).reshape(n_chunks, 256)
    got = ch.cpu().numpy().view(np.uint16).reshape(-1, 256)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("counts", [False, True])
def test_pack_paths_meet_at_chunk_boundaries(torch, counts):
    """Chunks of rare exponents (long codes, more bits than a wave's LDS frame
    holds) between chunks of common ones: the pack pass ORs the former's codes
    into HBM one by one and packs the latter in LDS, and the words and windows
    they share at their boundaries must come out as the host encoder's."""
    chunk = 4096
    x = di.random_normal(40 * chunk + 1000, 0.02, 41)
    rng = np.random.default_rng(42)
    rare = np.concatenate([np.arange(1, 100), np.arange(140, 255)]).astype(np.uint16)
    slow = (3, 4, 17, 38)
    for c in slow:
        e = rng.choice(rare, chunk)
        sm = rng.integers(0, 1 << 16, chunk, dtype=np.uint16) & np.uint16(0x807F)
        x[c * chunk:(c + 1) * chunk] = sm | (e << np.uint16(7))
    g = check(torch, x, f"paths_meet_counts{int(counts)}", counts=counts)
    lens = np.frombuffer(bytes(g.plan.code_len), dtype=np.uint8).astype(np.int64)
    bits = [int(lens[(x[c * chunk:(c + 1) * chunk] >> 7) & 0xFF].sum()) for c in range(40)]
    assert all(bits[c] > 32 * 1023 for c in slow), bits  # past the frame: the global path
    assert all(bits[c] < 32 * 1000 for c in range(40) if c not in slow), bits  # the LDS frame


def test_workload_c2(torch):
    check(torch, di.generate("C2"), "C2", counts=True)


def test_workload_c3_full(torch):
    x = di.generate("C3")
    g = check(torch, x, "C3", counts=True)
    assert g.plan.n_total == x.size


def test_round_trip_past_32_bit_sizes(torch):
    # 2.2 G weights (more than 2^31) and about 5.7 G stream bits (more than
    # 2^32), in more than 1,024 segments of 256 chunks, so each thread of the
    # one-workgroup offset scan sums several segments.  Generated, encoded and
    # decoded on the device (seeded); the decode is checked against the oracle
    # elsewhere, and every section enters it: a wrong offset, gap, position or
    # count would change the output.
    n = 2_200_000_001
    say(f"gpu encode round trip: n={n}")
    gen = torch.Generator(device="cuda").manual_seed(12)
    x = (torch.randn(n, device="cuda", generator=gen) * 0.02).to(torch.bfloat16).view(torch.int16)
    g = hdb.gpu_encode(x, window_counts=True)
    assert (g.plan.n_total + 4095) // 4096 > 1024 * 256 and g.plan.total_bits > 1 << 32 and n > 1 << 31
    out = torch.empty(n, dtype=torch.int16, device="cuda")
    for v in (hdb.DF11_VARIANT_MULTI, hdb.DF11_VARIANT_COUNTS):
        out.fill_(0x5A5A)
        hdb.df11_decode_block(g.block, out=out, launch=(0, 0, v))
        torch.cuda.synchronize()
        assert torch.equal(out, x), f"variant {v}: decode of the GPU encoding differs"
    del out, g, x
    torch.cuda.empty_cache()


def test_argument_errors(torch):
    x = di.random_normal(10_000, 0.02, 3)
    xd = torch.from_numpy(x.view(np.int16)).to("cuda")
    h = torch.empty(256, dtype=torch.int64, device="cuda")
    with pytest.raises(hdb.DF11Error) as ei:
        hdb.df11_gpu_histogram(xd[1:], h)  # not 16-byte aligned
    assert ei.value.status == hdb.DF11_E_INVALID_ARG
    ch = torch.empty(hdb.df11_gpu_chunk_hist_bytes(x.size) // 2 + 8, dtype=torch.int16, device="cuda")
    with pytest.raises(hdb.DF11Error) as ei:
        hdb.df11_gpu_histogram(xd, h, ch[1:])  # per-chunk counts not 16-byte aligned
    assert ei.value.status == hdb.DF11_E_INVALID_ARG
    hdb.df11_gpu_histogram(xd, h, ch)
    torch.cuda.synchronize()
    plan = hdb.df11_gpu_plan_build(np.bincount((x >> 7) & 0xFF, minlength=256).astype(np.uint64))
    buf = lambda n: torch.empty(max(16, n), dtype=torch.uint8, device="cuda")  # noqa: E731
    args = [buf(plan.stream_bytes), buf(plan.sign_mant_bytes), buf(plan.gaps_bytes),
            torch.empty(plan.n_units + 1, dtype=torch.int64, device="cuda")]
    with pytest.raises(hdb.DF11Error) as ei:  # counts given, but the plan has none
        hdb.df11_gpu_encode(plan, xd, ch, *args, buf(64 * plan.n_units), buf(plan.workspace_bytes))
    assert ei.value.status == hdb.DF11_E_INVALID_ARG
    shifted = torch.empty(x.size + 8, dtype=torch.int16, device="cuda")[1:x.size + 1]
    shifted.copy_(xd)
    with pytest.raises(hdb.DF11Error) as ei:  # misaligned input (the library refuses it)
        hdb.df11_gpu_encode(plan, shifted, ch, *args, None, buf(plan.workspace_bytes))
    assert ei.value.status == hdb.DF11_E_INVALID_ARG
    # tensors smaller than the plan's sections are refused before any launch
    with pytest.raises(ValueError):
        hdb.df11_gpu_encode(plan, xd, ch, buf(plan.stream_bytes - 1), *args[1:], None, buf(plan.workspace_bytes))
    with pytest.raises(ValueError):
        hdb.df11_gpu_encode(plan, xd[:-1], ch, *args, None, buf(plan.workspace_bytes))
    with pytest.raises(ValueError):
        hdb.df11_gpu_encode(plan, xd, ch, *args, None, buf(plan.workspace_bytes - 1))
    with pytest.raises(ValueError):
        hdb.df11_gpu_histogram(xd, h, ch[:8])
    with pytest.raises(TypeError):
        hdb.df11_gpu_histogram(xd, torch.empty(512, dtype=torch.int32, device="cuda"))
    with pytest.raises(TypeError):
        hdb.df11_gpu_histogram(xd.float(), h)
    with pytest.raises(hdb.DF11Error) as ei:  # no per-chunk counts
        hdb.df11_gpu_encode(plan, xd, None, *args, None, buf(plan.workspace_bytes))
    assert ei.value.status == hdb.DF11_E_INVALID_ARG
