"""GPU: a block whose section contents are corrupted on the device (after the
host-side checks), in the pages' format and the aligned-units layout,
decodes to garbage but never writes outside its output range, and decode
tables that would not advance make the multi-code kernels fall back to the
hierarchical tables (one code per lookup), so the output is still exact.
The kernel's own bounds are what is tested: stores go through
buffer ranges clamped to [0, n_total), sub-table indices are clamped, every
table step advances, and staging writes are bounded by the staging size."""
import ctypes

import numpy as np
import pytest

import df11_inputs as di
import huffman_decode_block_amd as hdb

pytestmark = pytest.mark.gpu

GUARD = 4096          # sentinel elements on each side of the output
SENTINEL = 0x5A5A
VARIANTS = [hdb.DF11_VARIANT_SINGLE, hdb.DF11_VARIANT_MULTI, hdb.DF11_VARIANT_COUNTS]


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "the GPU tests need a GPU"
    return t


@pytest.fixture(scope="module")
def sections():
    x = di.random_normal(200_003, 0.02, 41)
    return x, hdb.df11_encode_block([x], window_counts=True).sections


@pytest.fixture(scope="module")
def aligned_sections():
    x = di.random_normal(200_003, 0.02, 43)
    return x, hdb.df11_encode_block([x], window_counts=True, aligned_units=True).sections


class Block:
    """Device copies of every section, and the df11_device_block over them."""

    def __init__(self, torch, s):
        tables = hdb.df11_build_tables(s.code_len)
        _, n_tables = hdb.df11_tables_size(s.code_len)
        arrays = {"tables": tables, "stream": s.stream, "sign_mant": s.sign_mant, "gaps": s.gaps,
                  "unit_pos": np.ascontiguousarray(s.unit_pos, dtype=np.uint64), "counts": s.counts}
        if s.unit_end is not None:
            arrays["unit_end"] = np.ascontiguousarray(s.unit_end)
        self.t = {}
        for k, a in arrays.items():
            a = np.ascontiguousarray(a).view(np.uint8).reshape(-1)
            d = torch.empty(a.size, dtype=torch.uint8, device="cuda")
            d.copy_(torch.from_numpy(a))
            self.t[k] = d
        b = hdb.df11_device_block()
        b.tables, b.tables_bytes = self.t["tables"].data_ptr(), self.t["tables"].numel()
        b.stream, b.stream_bytes = self.t["stream"].data_ptr(), self.t["stream"].numel()
        b.sign_mant, b.sign_mant_bytes = self.t["sign_mant"].data_ptr(), self.t["sign_mant"].numel()
        b.gaps, b.gaps_bytes = self.t["gaps"].data_ptr(), self.t["gaps"].numel()
        b.unit_pos = self.t["unit_pos"].data_ptr()
        b.counts = self.t["counts"].data_ptr()
        b.unit_end = self.t["unit_end"].data_ptr() if "unit_end" in self.t else None
        b.n_total, b.total_bits = int(s.n_total), int(s.total_bits)
        b.n_windows, b.n_units = int(s.n_windows), int(s.n_units)
        b.max_unit_count = int(np.diff(s.unit_pos.astype(np.int64)).max())
        b.version = hdb.DF11_FORMAT_VERSION
        b.n_tables = n_tables
        self.raw = b
        self.n_hier = n_tables

    def decode(self, torch, variant):
        n = int(self.raw.n_total)
        full = torch.full((n + 2 * GUARD,), SENTINEL, dtype=torch.int16, device="cuda")
        out = full[GUARD:GUARD + n]
        L = hdb.df11_launch(0, 0, variant, 0)
        st = hdb.lib().df11_decode_block_ex(ctypes.byref(self.raw), out.data_ptr(), n,
                                            torch.cuda.current_stream().cuda_stream, ctypes.byref(L))
        assert st == hdb.DF11_OK, hdb.lib().df11_status_str(st)
        torch.cuda.synchronize()
        return full


def random_bytes(torch, t, seed):
    g = np.random.default_rng(seed)
    t.copy_(torch.from_numpy(g.integers(0, 256, t.numel(), dtype=np.uint8)))


def corrupt(torch, blk, case, seed):
    g = np.random.default_rng(seed)
    if case == "stream":
        random_bytes(torch, blk.t["stream"], seed)
    elif case == "gaps":
        random_bytes(torch, blk.t["gaps"], seed)
    elif case == "counts":
        random_bytes(torch, blk.t["counts"], seed)
    elif case == "unit_pos_random":
        nu = int(blk.raw.n_units) + 1
        v = g.integers(0, 2**63, nu, dtype=np.int64).astype(np.uint64)
        v[::3] = g.integers(0, int(blk.raw.n_total) + 10, len(v[::3]))
        blk.t["unit_pos"].copy_(torch.from_numpy(v.view(np.uint8)))
    elif case == "unit_pos_reversed":
        v = blk.t["unit_pos"].cpu().numpy().view(np.uint64)[::-1].copy()
        blk.t["unit_pos"].copy_(torch.from_numpy(v.view(np.uint8)))
    elif case == "unit_end":
        random_bytes(torch, blk.t["unit_end"], seed)
    elif case == "hier_tables":
        # the hierarchical tables only (the multi-code tables after them stay valid)
        t = blk.t["tables"][: blk.n_hier * 1024]
        random_bytes(torch, t, seed)
    else:
        raise ValueError(case)


SAFE_CASES = ["stream", "gaps", "counts", "unit_pos_random", "unit_pos_reversed", "hier_tables"]


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("case", SAFE_CASES)
def test_corrupt_contents_stay_inside_the_output(torch, sections, case, variant):
    x, s = sections
    print(f"[gpu-test] corrupt {case}, variant {variant}, n={x.size}", flush=True)
    blk = Block(torch, s)
    assert torch.equal(blk.decode(torch, variant)[GUARD:-GUARD].cpu(), torch.from_numpy(x.view(np.int16)))
    corrupt(torch, blk, case, 7)
    full = blk.decode(torch, variant).cpu().numpy()
    assert (full[:GUARD] == SENTINEL).all() and (full[-GUARD:] == SENTINEL).all()


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("case", ["unit_end", "stream", "unit_pos_random", "gaps"])
def test_corrupt_aligned_layout_stays_inside_the_output(torch, aligned_sections, case, variant):
    x, s = aligned_sections
    print(f"[gpu-test] corrupt aligned {case}, variant {variant}, n={x.size}", flush=True)
    blk = Block(torch, s)
    assert torch.equal(blk.decode(torch, variant)[GUARD:-GUARD].cpu(), torch.from_numpy(x.view(np.int16)))
    corrupt(torch, blk, case, 9)
    full = blk.decode(torch, variant).cpu().numpy()
    assert (full[:GUARD] == SENTINEL).all() and (full[-GUARD:] == SENTINEL).all()


@pytest.mark.parametrize("variant", [hdb.DF11_VARIANT_MULTI, hdb.DF11_VARIANT_COUNTS])
@pytest.mark.parametrize("table", ["count", "emit"])
def test_bad_multi_code_tables_fall_back_to_the_hierarchical_tables(torch, sections, table, variant):
    """A count or emit entry that would not advance is refused when the
    tables are loaded; the workgroups then decode one code per lookup through
    the hierarchical tables, which are intact here: every element is written
    and the output is still the input."""
    x, s = sections
    print(f"[gpu-test] bad {table} table, variant {variant}", flush=True)
    blk = Block(torch, s)
    base = blk.n_hier * 1024
    count_bytes = 4 << 10  # 1,024 entries of 4 bytes
    if table == "count":
        off = base + 4 * 37  # one count entry with a step of 0 bits that is not the escape
    else:
        off = base + count_bytes + 8 * 1001  # one emit entry taking 0 codes
    blk.t["tables"][off:off + 4].zero_()
    full = blk.decode(torch, variant).cpu()
    assert (full[:GUARD] == SENTINEL).all() and (full[-GUARD:] == SENTINEL).all()
    assert torch.equal(full[GUARD:-GUARD], torch.from_numpy(x.view(np.int16)))
    # the one-code-per-lookup kernel reads neither table and is unaffected
    out = blk.decode(torch, hdb.DF11_VARIANT_SINGLE)[GUARD:-GUARD].cpu()
    assert torch.equal(out, torch.from_numpy(x.view(np.int16)))
