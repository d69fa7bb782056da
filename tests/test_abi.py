"""The C-ABI library loads and exports every function include/df11.h
declares; host-side argument checks and status codes behave as documented.
No GPU work is started here."""
import ctypes
import os
import re

import numpy as np

import huffman_decode_block_amd as hdb
from conftest import ROOT


def declared_functions():
    src = open(os.path.join(ROOT, "include", "df11.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(df11_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 11
    lib = ctypes.CDLL(hdb.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(hdb.EXPORTS) == names


def test_binding_has_the_c_names():
    for n in declared_functions():
        assert callable(getattr(hdb, n)), n


def test_status_strings():
    assert hdb.df11_status_str(hdb.DF11_OK) == "ok"
    for s in range(-6, 0):
        assert hdb.df11_status_str(s) not in ("ok", "unknown status")
    assert hdb.df11_status_str(-99) == "unknown status"
    assert hdb.df11_last_hip_error() == 0


def test_null_arguments_are_rejected():
    L = hdb.lib()
    assert L.df11_encode_block(None, 1, 0, None) == hdb.DF11_E_INVALID_ARG
    assert L.df11_encoded_sections(None, None) == hdb.DF11_E_INVALID_ARG
    L.df11_encoded_free(None)
    assert L.df11_validate(None) == hdb.DF11_E_INVALID_ARG
    assert L.df11_tables_size(None, None, None) == hdb.DF11_E_INVALID_ARG
    assert L.df11_decode_block(None, None, 0, None) == hdb.DF11_E_INVALID_ARG
    view = (hdb.df11_bf16_view * 1)()
    view[0].data = None
    view[0].numel = 5
    h = ctypes.c_void_p()
    assert L.df11_encode_block(view, 1, 0, ctypes.byref(h)) == hdb.DF11_E_INVALID_ARG


def test_decode_argument_checks_return_before_any_launch():
    x = np.arange(1000, dtype=np.uint16)
    enc = hdb.df11_encode_block([x])
    s = enc.sections
    # pretend device pointers: only the host-side checks run, nothing is dereferenced
    blk = hdb.df11_device_block_from_blob(s, 1 << 20)
    L = hdb.lib()
    assert L.df11_decode_block(ctypes.byref(blk), 1 << 24, 999, None) == hdb.DF11_E_BUFFER_TOO_SMALL
    assert L.df11_decode_block(ctypes.byref(blk), (1 << 24) + 2, 1000, None) == hdb.DF11_E_INVALID_ARG
    bad = hdb.df11_device_block.from_buffer_copy(blk)
    bad.version = 2
    assert L.df11_decode_block(ctypes.byref(bad), 1 << 24, 1000, None) == hdb.DF11_E_UNSUPPORTED
    bad = hdb.df11_device_block.from_buffer_copy(blk)
    bad.n_units += 1
    assert L.df11_decode_block(ctypes.byref(bad), 1 << 24, 1000, None) == hdb.DF11_E_INVALID_ARG
    bad = hdb.df11_device_block.from_buffer_copy(blk)
    bad.gaps_bytes = 8
    assert L.df11_decode_block(ctypes.byref(bad), 1 << 24, 1000, None) == hdb.DF11_E_INVALID_ARG
    bad = hdb.df11_device_block.from_buffer_copy(blk)
    bad.max_unit_count = 5000
    assert L.df11_decode_block(ctypes.byref(bad), 1 << 24, 1000, None) == hdb.DF11_E_INVALID_ARG
    # sizes that no encoder produces are refused before any size is derived
    # from them; every other field is made consistent with the bad one, so
    # that only this check can refuse
    for n_total, total_bits in ((1000, 33 * 1000), (1000, 999), (1000, (1 << 64) - 1), (1 << 50, 1 << 52)):
        bad = hdb.df11_device_block.from_buffer_copy(blk)
        bad.n_total, bad.total_bits = n_total, total_bits
        nw = ((total_bits + 63) % (1 << 64)) // 64  # wraps like uint64 arithmetic
        nu = (nw + 63) // 64
        bad.n_windows, bad.n_units = nw, nu
        bad.stream_bytes, bad.gaps_bytes = 512 * nu + 16, 40 * nu + 8
        bad.sign_mant_bytes = (n_total + 15) // 16 * 16
        got = L.df11_decode_block(ctypes.byref(bad), 1 << 24, n_total, None)
        assert got == hdb.DF11_E_INVALID_ARG, (n_total, total_bits, got)
    launch = hdb.df11_launch(3, 0)
    assert L.df11_decode_block_ex(ctypes.byref(blk), 1 << 24, 1000, None,
                                  ctypes.byref(launch)) == hdb.DF11_E_INVALID_ARG
    # an empty block is a no-op that needs no pointers
    empty = hdb.df11_encode_block([np.zeros(0, np.uint16)])
    eb = hdb.df11_device_block_from_blob(empty.sections, 1 << 20)
    assert L.df11_decode_block(ctypes.byref(eb), None, 0, None) == hdb.DF11_OK


def test_section_views_keep_their_blob_alive():
    import gc
    x = np.arange(100_000, dtype=np.uint16)
    stream = hdb.df11_encode_block([x]).sections.stream  # the Encoded is a temporary
    copy = stream.copy()
    gc.collect()
    junk = [np.full(1 << 16, 0xAB, np.uint8) for _ in range(64)]  # reuse freed memory, if any
    assert np.array_equal(stream, copy)
    del junk
