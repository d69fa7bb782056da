"""GPU parity over seeded random blocks (`df11_inputs.random_block`: six value
families, log-uniform sizes, splits into 1 to 7 matrices).  Library blobs in
the pages' format (with window counts) and in the aligned-units layout are
decoded by every variant, each with a seeded launch geometry, into a buffer
guarded on both sides, and compared with the input bit for bit (the library's
sections equal the oracle's on the same blocks: test_random_blocks.py)."""
import numpy as np
import pytest

import df11_inputs as di
import huffman_decode_block_amd as hdb

pytestmark = pytest.mark.gpu

GUARD = 64
CASES = [(s, 1) for s in range(36)] + [(100 + s, 1 << 20) for s in range(6)]


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "the GPU tests need a GPU"
    return t


def geometry(seed, variant):
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([4241, seed, variant])))
    waves = int(g.choice([0, 1, 2, 4, 8, 16]))
    max_groups = int(g.choice([0, 0, 1, 3, 64]))
    over = int(g.choice([0, 0, 1, 2, 16]))
    return (waves, max_groups, variant, over)


@pytest.mark.parametrize("aligned", [False, True])
@pytest.mark.parametrize("seed,min_n", CASES)
def test_random_block_decodes_bit_exactly(torch, seed, min_n, aligned):
    x, mats, what = di.random_block(seed, max_n=max(min_n, 1 << 20) * 4, min_n=min_n)
    enc = hdb.df11_encode_block(mats, window_counts=True, aligned_units=aligned)
    blk = hdb.DeviceBlock.from_encoded(enc)
    n = x.size
    for variant in (hdb.DF11_VARIANT_SINGLE, hdb.DF11_VARIANT_MULTI, hdb.DF11_VARIANT_COUNTS):
        launch = geometry(seed, variant)
        print(f"[gpu-test] random block {seed}: {what}, aligned={aligned}, launch={launch}", flush=True)
        buf = torch.full((n + 2 * GUARD,), 0x5A5A, dtype=torch.int16, device="cuda")
        hdb.df11_decode_block(blk, out=buf[GUARD:GUARD + n], launch=launch)
        torch.cuda.synchronize()
        h = buf.cpu().numpy().view(np.uint16)
        assert (h[:GUARD] == 0x5A5A).all() and (h[GUARD + n:] == 0x5A5A).all(), (what, launch)
        np.testing.assert_array_equal(h[GUARD:GUARD + n], x, err_msg=f"{what} launch={launch}")


@pytest.mark.parametrize("seed,min_n", CASES[::2])
def test_random_block_gpu_encoding_equals_the_host_encoder(torch, seed, min_n):
    x, _, what = di.random_block(seed, max_n=max(min_n, 1 << 20) * 4, min_n=min_n)
    counts = seed % 2 == 0
    print(f"[gpu-test] gpu encode of random block {seed}: {what}, counts={counts}", flush=True)
    xd = torch.from_numpy(x.view(np.int16)).to("cuda")
    g = hdb.gpu_encode(xd, window_counts=counts)
    s = hdb.df11_encode_block([x], window_counts=counts).sections
    p = g.plan
    assert bytes(p.code_len) == bytes(s.code_len) and p.total_bits == s.total_bits, what
    np.testing.assert_array_equal(g.section("stream")[:p.stream_bytes], s.stream, err_msg=what)
    np.testing.assert_array_equal(g.section("sign_mant")[:p.sign_mant_bytes], s.sign_mant, err_msg=what)
    np.testing.assert_array_equal(g.section("gaps")[:p.gaps_bytes], s.gaps, err_msg=what)
    np.testing.assert_array_equal(g.section("unit_pos").view(np.uint64), s.unit_pos, err_msg=what)
    if counts:
        np.testing.assert_array_equal(g.section("counts"), s.counts, err_msg=what)


def _decodes_exactly(torch, x, blk, launch):
    n = x.size
    buf = torch.full((n + 2 * GUARD,), 0x5A5A, dtype=torch.int16, device="cuda")
    hdb.df11_decode_block(blk, out=buf[GUARD:GUARD + n], launch=launch)
    torch.cuda.synchronize()
    h = buf.cpu().numpy().view(np.uint16)
    return (h[:GUARD] == 0x5A5A).all() and (h[GUARD + n:] == 0x5A5A).all() and np.array_equal(h[GUARD:GUARD + n], x)


@pytest.mark.parametrize("first,last,min_n,max_n", [(1000, 1500, 1, 1 << 22), (2000, 2100, 1 << 20, 1 << 24)])
def test_wide_sweep(torch, first, last, min_n, max_n):
    # many more seeds than the cases above, checked in one test each: every
    # decode variant with its seeded launch geometry, both layouts
    bad = []
    for seed in range(first, last):
        x, mats, what = di.random_block(seed, max_n=max_n, min_n=min_n)
        for aligned in (False, True):
            blk = hdb.DeviceBlock.from_encoded(hdb.df11_encode_block(mats, window_counts=True, aligned_units=aligned))
            for variant in (hdb.DF11_VARIANT_SINGLE, hdb.DF11_VARIANT_MULTI, hdb.DF11_VARIANT_COUNTS):
                launch = geometry(seed, variant)
                if not _decodes_exactly(torch, x, blk, launch):
                    bad.append((seed, what, aligned, launch))
        if seed % 50 == 0:
            print(f"[gpu-test] wide sweep: seed {seed}, {len(bad)} mismatches so far", flush=True)
    assert not bad, bad[:5]
