"""Host-side pieces of bench.py: the code identity used to decide whether the
committed HBM counters still describe the kernel, the algorithmic byte count
the roofline fraction is priced on, and the refusal to run on several GPUs."""
import importlib.util
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import df11_inputs as di
import huffman_decode_block_amd as hdb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_code_tokens_ignore_comments_and_layout(bench):
    a = "int f(int x) {  // add one\n    return x + 1; /* the\n result */ }\n"
    b = "int f(int x)\n{\n  return x + 1;\n}\n"
    assert bench.code_tokens(a) == bench.code_tokens(b)
    # code changes are seen
    assert bench.code_tokens(a) != bench.code_tokens(a.replace("x + 1", "x + 2"))
    # comment markers inside literals are code
    s1 = 'const char *p = "a // b";\n'
    s2 = 'const char *p = "a";\n'
    assert bench.code_tokens(s1) != bench.code_tokens(s2)
    assert "a // b" in bench.code_tokens(s1)
    assert bench.code_tokens("char c = '\\'';// x\n") == "char c = '\\'';"


def test_kernel_hash_is_stable_under_comment_edits(bench, tmp_path, monkeypatch):
    src = open(bench.KERNEL_SRC).read()
    h = bench.kernel_hash()
    f = tmp_path / "k.hip"
    f.write_text("// a new header line\n" + src.replace("\n\n", "\n\n// note\n", 1))
    monkeypatch.setattr(bench, "KERNEL_SRC", str(f))
    assert bench.kernel_hash() == h
    f.write_text(src + "\nint extra_symbol;\n")
    assert bench.kernel_hash() != h
    # the included headers are part of the identity
    monkeypatch.setattr(bench, "KERNEL_SRC", str(tmp_path / "k.hip"))
    f.write_text(src)
    hdr = tmp_path / "w.h"
    hdr.write_text(open(bench.KERNEL_HEADERS[0]).read() + "\nint other;\n")
    monkeypatch.setattr(bench, "KERNEL_HEADERS", [str(hdr)])
    assert bench.kernel_hash() != h


def test_measured_traffic_only_for_matching_code_and_workload(bench, tmp_path, monkeypatch):
    counters = tmp_path / "c.json"
    counters.write_text(json.dumps({"kernel_code_sha256_16": bench.kernel_hash(), "workload": "C3: block",
                                    "hbm_bytes_per_launch": 123}))
    monkeypatch.setattr(bench, "COUNTERS", str(counters))
    assert bench.measured_traffic("C3") == 123
    assert bench.measured_traffic("C4") is None
    counters.write_text(json.dumps({"kernel_code_sha256_16": "0" * 16, "workload": "C3: block",
                                    "hbm_bytes_per_launch": 123}))
    assert bench.measured_traffic("C3") is None


def test_algorithmic_bytes_match_the_sections(bench):
    x = di.generate("C1")
    enc = hdb.df11_encode_block(di.split("C1", x), window_counts=True)
    s = enc.sections
    ab = bench.algorithmic_bytes(s)
    assert ab["write"] == 2 * x.size
    want_read = (s.total_bits + 7) // 8 + x.size + (5 * s.n_windows + 7) // 8 + 8 * (s.n_units + 1) \
        + s.raw.tables_bytes
    assert ab["read"] == want_read
    assert ab["total"] == ab["read"] + ab["write"]
    assert bench.algorithmic_bytes(s, with_counts=True)["read"] == want_read + s.n_windows
    # near the closed form of the format: 8 + L + 5L/64 bits per weight plus the tables
    bits = 8 * (ab["read"] - s.raw.tables_bytes) / x.size
    L = s.mean_code_len_bits
    assert abs(bits - (8 + L + 5 * L / 64)) < 0.05


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
    assert not r.stdout.strip().startswith("{")


def test_algorithmic_bytes_are_integers(bench):
    enc = hdb.df11_encode_block([np.zeros(1000, np.uint16)])
    ab = bench.algorithmic_bytes(enc.sections)
    assert all(isinstance(v, int) for v in ab.values())


def test_rotation_copies_cover_several_infinity_caches():
    import bench
    need = bench.ROTATION_CACHES * bench.INFINITY_CACHE_BYTES
    assert bench.ROTATION_CACHES >= 4                        # two caches' worth still left hits
    assert bench.rotation_copies(299_316_096) == 6          # a Llama-3.1-8B-shaped block's sections
    assert bench.rotation_copies(1_200_000_000) == 2        # a Llama-3.1-70B-shaped block's
    assert bench.rotation_copies(22_768_000) == 64          # one 4096 x 4096 matrix: the cap
    for read in (1_000_000, 22_768_000, 100_000_000, 299_316_096, 720_000_000, 4_000_000_000):
        k = bench.rotation_copies(read)
        assert k >= 2 and (k * read >= need or k == 64)
        assert k == 2 or (k - 1) * read < need              # no more copies than needed
    assert bench.rotation_copies(1) == 64 and bench.rotation_copies(0) == 64


def test_cold_schedule_rejects_an_unknown_flush(bench):
    # checked before anything is allocated
    with pytest.raises(ValueError):
        bench.ColdSchedule("cpu", None, "write-1gib")
    assert bench.ColdSchedule.FLUSH_KINDS[0] == "read"  # the headline schedule is the default


def test_committed_counters_describe_the_current_decode_kernel(bench):
    """The headline's roofline.traffic comes from the committed counter
    summary only while it was taken on the current decode kernel code (its
    source and the headers it includes): a change to any of them needs the
    counters taken again."""
    with open(bench.COUNTERS) as f:
        c = json.load(f)
    assert c["kernel_code_sha256_16"] == bench.kernel_hash(), \
        "the decode kernel's code changed since profiles/df11_decode_kernel_c3_hbm_counters.json was taken"
    assert bench.measured_traffic("C3") == c["hbm_bytes_per_launch"]
