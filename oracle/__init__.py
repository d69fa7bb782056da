"""CPU oracle for DFloat11 exponent coding -- TEST INFRASTRUCTURE ONLY.

Plain, slow reference of what the GPU path computes: the DF11 encoder
(exponent histogram, Huffman code lengths, canonical codes, bit-serial
packing, gaps and unit positions) and a bit-serial Huffman decoder.  The
arithmetic lives in ``df11_oracle.c`` (plain C99, built with gcc); this module
only builds and loads it and marshals numpy arrays.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package.  It shares no code with ``huffman_decode_block_amd`` and
never imports it.

Sources: the hada.io summary of the DFloat11 paper, sections "Le format
DFloat11" (exponent-only Huffman coding, EncodedExponent and
PackedSignMantissa arrays) and "Noyau GPU en deux etapes et metadonnees
auxiliaires" (8-byte thread windows, 5-bit gaps, stored output positions).
Parity status: every function here is pinned by the not-gpu tests (round
trip on all BF16 patterns, Kraft equality, entropy bound, brute-force and
dynamic-programming optimality, hand-derived vectors, vectorised
re-derivation of gaps and positions, a bit-by-bit walk of each window for the
per-window counts; for the aligned-units variant a closed-form layout, the
round trip, its invariants and the gap rule re-applied to the pages' format).

Two format variants that are not on the pages are defined here in numpy
(`window_counts`, `encode_aligned_units`); everything else is the C file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "df11_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_df11.so")
_lib = None

CAP = 32


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into oracle/liboracle_df11.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-shared", "-fPIC", "-pthread",
             _SRC, "-o", tmp]
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    u64p = ctypes.POINTER(ctypes.c_uint64)
    u32p = ctypes.POINTER(ctypes.c_uint32)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    u64 = ctypes.c_uint64
    lib.orc_histogram.argtypes = [u16p, u64, u64p]
    lib.orc_histogram.restype = None
    lib.orc_code_lengths.argtypes = [u64p, u32p]
    lib.orc_code_lengths.restype = ctypes.c_int
    lib.orc_code_lengths_capped.argtypes = [u64p, ctypes.c_uint32, u32p]
    lib.orc_code_lengths_capped.restype = ctypes.c_int
    lib.orc_package_merge_lengths.argtypes = [u64p, ctypes.c_uint32, u32p]
    lib.orc_package_merge_lengths.restype = ctypes.c_int
    lib.orc_canonical_codes.argtypes = [u32p, u64p]
    lib.orc_canonical_codes.restype = None
    lib.orc_plan.argtypes = [u16p, u64, u32p, u64p]
    lib.orc_plan.restype = ctypes.c_int
    lib.orc_encode.argtypes = [u16p, u64, u32p, u8p, u64, u8p, u64, u8p, u64, u64p, u64, u64p]
    lib.orc_encode.restype = ctypes.c_int
    lib.orc_decode.argtypes = [u32p, u8p, u64, u8p, u64, u16p]
    lib.orc_decode.restype = ctypes.c_int
    lib.orc_decode_units.argtypes = [u32p, u8p, u64, u8p, u8p, u64p, u64, u64, u16p]
    lib.orc_decode_units.restype = ctypes.c_int
    lib.orc_decode_units_threads.argtypes = [u32p, u8p, u64, u8p, u8p, u64p, u64, u64, u16p,
                                             ctypes.c_int]
    lib.orc_decode_units_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _u16(x) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(x))
    if a.dtype != np.uint16:
        if a.dtype == np.int16:
            a = a.view(np.uint16)
        else:
            raise TypeError(f"expected raw BF16 bits as uint16, got {a.dtype}")
    return a.reshape(-1)


def histogram(x) -> np.ndarray:
    x = _u16(x)
    counts = np.zeros(256, dtype=np.uint64)
    _load().orc_histogram(_ptr(x, ctypes.c_uint16), x.size, _ptr(counts, ctypes.c_uint64))
    return counts


def code_lengths(counts, cap: int = CAP) -> np.ndarray:
    """Huffman lengths (reading R1), package-merge when longer than cap (R2)."""
    c = np.ascontiguousarray(np.asarray(counts, dtype=np.uint64).reshape(256))
    ln = np.zeros(256, dtype=np.uint32)
    rc = _load().orc_code_lengths_capped(_ptr(c, ctypes.c_uint64), cap, _ptr(ln, ctypes.c_uint32))
    if rc < 0:
        raise ValueError(f"orc_code_lengths_capped failed: {rc}")
    return ln


def package_merge_lengths(counts, cap: int) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(counts, dtype=np.uint64).reshape(256))
    ln = np.zeros(256, dtype=np.uint32)
    rc = _load().orc_package_merge_lengths(_ptr(c, ctypes.c_uint64), cap, _ptr(ln, ctypes.c_uint32))
    if rc < 0:
        raise ValueError(f"orc_package_merge_lengths failed: {rc}")
    return ln


def canonical_codes(lengths) -> np.ndarray:
    ln = np.ascontiguousarray(np.asarray(lengths, dtype=np.uint32).reshape(256))
    codes = np.zeros(256, dtype=np.uint64)
    _load().orc_canonical_codes(_ptr(ln, ctypes.c_uint32), _ptr(codes, ctypes.c_uint64))
    return codes


@dataclass
class Encoded:
    """Sections of one encoded block, as the oracle computes them."""
    n: int
    total_bits: int
    n_windows: int
    n_units: int
    code_len: np.ndarray      # uint8[256]
    stream: np.ndarray        # uint8[512*n_units + 16]
    sign_mant: np.ndarray     # uint8[round_up(n, 16)]
    gaps: np.ndarray          # uint8[40*n_units + 8]
    unit_pos: np.ndarray      # uint64[n_units + 1]
    max_len: int
    unit_end: np.ndarray | None = None  # aligned-units variant: uint16[n_units], bits of codes per unit


def encode(x) -> Encoded:
    x = _u16(x)
    lib = _load()
    ln = np.zeros(256, dtype=np.uint32)
    sizes = np.zeros(8, dtype=np.uint64)
    mx = lib.orc_plan(_ptr(x, ctypes.c_uint16), x.size, _ptr(ln, ctypes.c_uint32),
                      _ptr(sizes, ctypes.c_uint64))
    if mx < 0:
        raise ValueError(f"orc_plan failed: {mx}")
    n, total_bits, n_windows, n_units, sb, smb, gb, upe = (int(v) for v in sizes)
    stream = np.zeros(sb, dtype=np.uint8)
    sm = np.zeros(smb, dtype=np.uint8)
    gaps = np.zeros(gb, dtype=np.uint8)
    unit_pos = np.zeros(upe, dtype=np.uint64)
    tb = np.zeros(1, dtype=np.uint64)
    rc = lib.orc_encode(_ptr(x, ctypes.c_uint16), x.size, _ptr(ln, ctypes.c_uint32),
                        _ptr(stream, ctypes.c_uint8), sb, _ptr(sm, ctypes.c_uint8), smb,
                        _ptr(gaps, ctypes.c_uint8), gb, _ptr(unit_pos, ctypes.c_uint64), upe,
                        _ptr(tb, ctypes.c_uint64))
    if rc != 0:
        raise ValueError(f"orc_encode failed: {rc}")
    assert int(tb[0]) == total_bits
    return Encoded(n=n, total_bits=total_bits, n_windows=n_windows, n_units=n_units,
                   code_len=ln.astype(np.uint8), stream=stream, sign_mant=sm, gaps=gaps,
                   unit_pos=unit_pos, max_len=int(mx))


def decode(enc: Encoded) -> np.ndarray:
    """Bit-serial decode of the whole stream from bit 0."""
    ln = np.ascontiguousarray(enc.code_len.astype(np.uint32))
    out = np.zeros(enc.n, dtype=np.uint16)
    stream = np.ascontiguousarray(enc.stream)
    sm = np.ascontiguousarray(enc.sign_mant)
    rc = _load().orc_decode(_ptr(ln, ctypes.c_uint32), _ptr(stream, ctypes.c_uint8), stream.size,
                            _ptr(sm, ctypes.c_uint8), enc.n, _ptr(out, ctypes.c_uint16))
    if rc != 0:
        raise ValueError(f"orc_decode failed: {rc}")
    return out


def decode_units(enc: Encoded, u_begin: int = 0, u_end: int | None = None,
                 threads: int = 1, out: np.ndarray | None = None) -> np.ndarray:
    """Decode units [u_begin, u_end) independently from their gap and position.

    Writes into out[unit_pos[u_begin] : unit_pos[u_end]] (a full-size output
    array, allocated zeroed if not given) and returns it."""
    if u_end is None:
        u_end = enc.n_units
    ln = np.ascontiguousarray(enc.code_len.astype(np.uint32))
    if out is None:
        out = np.zeros(enc.n, dtype=np.uint16)
    stream = np.ascontiguousarray(enc.stream)
    sm = np.ascontiguousarray(enc.sign_mant)
    gaps = np.ascontiguousarray(enc.gaps)
    up = np.ascontiguousarray(enc.unit_pos)
    lib = _load()
    if threads == 1:
        rc = lib.orc_decode_units(_ptr(ln, ctypes.c_uint32), _ptr(stream, ctypes.c_uint8),
                                  stream.size, _ptr(sm, ctypes.c_uint8), _ptr(gaps, ctypes.c_uint8),
                                  _ptr(up, ctypes.c_uint64), u_begin, u_end,
                                  _ptr(out, ctypes.c_uint16))
    else:
        rc = lib.orc_decode_units_threads(_ptr(ln, ctypes.c_uint32), _ptr(stream, ctypes.c_uint8),
                                          stream.size, _ptr(sm, ctypes.c_uint8),
                                          _ptr(gaps, ctypes.c_uint8), _ptr(up, ctypes.c_uint64),
                                          u_begin, u_end, _ptr(out, ctypes.c_uint16), threads)
    if rc != 0:
        raise ValueError(f"orc_decode_units failed: {rc}")
    return out


UNIT_BITS = 4096   # 64 windows of 64 bits: one stored position per unit
GROUP = 32         # aligned-units variant: codes per group (64 output bytes)


def code_starts(enc: Encoded, decoded=None) -> np.ndarray:
    """Stream bit at which each weight's codeword starts: the lengths of the
    codes before it, plus, in the aligned-units variant, the filler bits before
    it (the layout rule of `aligned_layout`)."""
    x = decode_units(enc) if decoded is None else _u16(decoded)
    lengths = enc.code_len.astype(np.int64)[(x >> 7) & 0xFF]
    if enc.unit_end is not None:
        return aligned_layout(lengths)[0]
    if not x.size:
        return np.zeros(0, np.int64)
    return np.concatenate([np.zeros(1, np.int64), np.cumsum(lengths)[:-1]])


def aligned_layout(lengths) -> tuple:
    """Code starts of the aligned-units variant (ours, not the pages'): the
    codes are taken in groups of 32 consecutive weights, in order.  A group is
    placed right after the previous one unless one of its codes would then
    start in a later unit than its first code (a unit being 4,096 stream bits);
    in that case the rest of the current unit is left as zero filler and the
    group starts at the next unit's first bit.  So every unit but the last
    holds a whole number of groups, and the first weight of every unit is a
    multiple of 32.  Returns (starts int64[n], unit code ends int64[n_units]
    (absolute: the filler's first bit, the unit's end when it has none, and
    the stream's end for the last unit), total stream bits)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    n = lengths.size
    starts = np.zeros(n, np.int64)
    ends = {}  # unit -> absolute end of its codes, where a filler follows
    pos = 0
    for g0 in range(0, n, GROUP):
        glen = lengths[g0:g0 + GROUP]
        offs = np.concatenate([np.zeros(1, np.int64), np.cumsum(glen)[:-1]])
        u = pos // UNIT_BITS
        if pos + offs[-1] >= (u + 1) * UNIT_BITS:  # its last code would start in the next unit
            ends[u] = pos
            pos = (u + 1) * UNIT_BITS
        starts[g0:g0 + glen.size] = pos + offs
        pos += int(glen.sum())
    total_bits = pos
    n_units = ((total_bits + 63) // 64 + 63) // 64
    unit_end = np.array([ends.get(u, min((u + 1) * UNIT_BITS, total_bits)) for u in range(n_units)],
                        dtype=np.int64)
    return starts, unit_end, total_bits


def encode_aligned_units(x) -> Encoded:
    """The aligned-units format variant (ours, not the pages'): code lengths,
    codewords and sign/mantissa bytes as in `encode`; the codes laid out by
    `aligned_layout`, filler bits 0.  Gaps: for window w of unit u, the first
    code start at or after 64w, or the end of u's codes if none comes before
    it, minus 64w (0 for a window entirely past the end of u's codes).  Unit
    positions: the number of codes that start before the unit.  unit_end[u]:
    the end of u's codes minus the unit's first bit.  The first weight of
    every unit is then a multiple of 32, so a decoder's writes of consecutive
    units meet on 64-byte boundaries."""
    base = encode(x)
    xs = _u16(x)
    codes = canonical_codes(base.code_len.astype(np.uint32)).astype(np.int64)
    lengths = base.code_len.astype(np.int64)[(xs >> 7) & 0xFF]
    starts, ends_abs, total_bits = aligned_layout(lengths)
    n_windows = (total_bits + 63) // 64
    n_units = (n_windows + 63) // 64
    # stream: codeword bits MSB-first at their starts, everything else 0
    bits = np.zeros(8 * (512 * n_units + 16), dtype=np.uint8)
    if xs.size:
        cw = codes[(xs >> 7) & 0xFF]
        rep = np.repeat(np.arange(xs.size), lengths)
        j = np.arange(rep.size) - np.repeat(np.cumsum(lengths) - lengths, lengths)  # bit index in its code
        bits[starts[rep] + j] = ((cw[rep] >> (lengths[rep] - 1 - j)) & 1).astype(np.uint8)
    stream = np.packbits(bits)
    # gaps
    w = np.arange(n_windows, dtype=np.int64)
    end_w = ends_abs[w // 64]
    if starts.size:
        nxt = np.searchsorted(starts, 64 * w)  # first code starting at or after 64w
        first = np.where(nxt < starts.size, starts[np.minimum(nxt, starts.size - 1)], total_bits)
    else:
        first = np.full(n_windows, total_bits, dtype=np.int64)
    gap = np.where(64 * w >= end_w, 0, np.minimum(first, end_w) - 64 * w)
    assert (gap >= 0).all() and (gap <= 31).all()
    gbits = np.zeros(8 * (40 * n_units + 8), dtype=np.uint8)  # 5-bit fields, MSB-first
    for k in range(5):
        gbits[5 * w + k] = (gap >> (4 - k)) & 1
    gaps = np.packbits(gbits)[:40 * n_units + 8]
    unit_pos = np.zeros(n_units + 1, dtype=np.uint64)
    unit_pos[:n_units] = np.searchsorted(starts, UNIT_BITS * np.arange(n_units, dtype=np.int64))
    unit_pos[n_units] = xs.size
    unit_end = (ends_abs - UNIT_BITS * np.arange(n_units, dtype=np.int64)).astype(np.uint16)
    return Encoded(n=xs.size, total_bits=int(total_bits), n_windows=int(n_windows), n_units=int(n_units),
                   code_len=base.code_len, stream=stream, sign_mant=base.sign_mant, gaps=gaps,
                   unit_pos=unit_pos, max_len=base.max_len, unit_end=unit_end)


def window_counts(enc: Encoded, decoded=None) -> np.ndarray:
    """Per-window code counts of a format variant that is not on the pages:
    for each 64-bit window w, the number of codewords whose first bit lies in
    [64w, 64w + 64).  As no codeword starts in [64w, 64w + gap_w) (definition
    of the gap, hada.io summary, section "Noyau GPU en deux etapes et
    metadonnees auxiliaires"), this is exactly the count of codes starting in
    [64w + gap_w, min(64w + 64, total_bits)), the number that the decoder's
    first phase computes for the window.  Code starts come from the oracle's
    own decode of the stream (or `decoded`, its result, when already at hand)
    through `code_starts`.  Returns n_windows uint8 values (each at most 64)."""
    starts = code_starts(enc, decoded)
    counts = np.bincount(starts >> 6, minlength=enc.n_windows)[:enc.n_windows]
    return counts.astype(np.uint8)


def exponent_entropy_bits(counts) -> float:
    """Shannon entropy of the exponent distribution, in bits per weight."""
    c = np.asarray(counts, dtype=np.float64)
    tot = c.sum()
    if tot == 0:
        return 0.0
    p = c[c > 0] / tot
    return float(-(p * np.log2(p)).sum())
