import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")
    # build only what is missing (a fresh checkout); an existing build is used as is
    import oracle
    if not os.path.exists(oracle._LIB_PATH):
        oracle.build(force=True)
    lib = os.path.join(ROOT, "huffman_decode_block_amd", "libdf11.so")
    if not os.path.exists(lib):
        from huffman_decode_block_amd.build import build
        build()


def load_golden(name):
    import json
    with open(os.path.join(GOLDEN, name + ".json")) as f:
        return json.load(f)
