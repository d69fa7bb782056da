"""Python binding of libdf11 (include/df11.h): DFloat11 block encoding on the
host and block decoding on an MI355X.

Argument marshalling only: every step of the encoder runs in the library's
C++ code and every step of the decode runs in its HIP kernel.  PyTorch is used
for device memory and streams.  The functions keep the C names; a few small
classes (Encoded, DeviceBlock) own the memory behind them.

The library must be built first (``python -m huffman_decode_block_amd.build``
or ``__graft_entry__.build()``); the first call into the package raises
ImportError when it is missing.  There is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdf11.so")

DF11_OK = 0
DF11_E_INVALID_ARG = -1
DF11_E_NOMEM = -2
DF11_E_FORMAT = -3
DF11_E_BUFFER_TOO_SMALL = -4
DF11_E_UNSUPPORTED = -5
DF11_E_HIP = -6
DF11_FORMAT_VERSION = 1

_u64 = ctypes.c_uint64
_u32 = ctypes.c_uint32
_vp = ctypes.c_void_p


class df11_bf16_view(ctypes.Structure):
    _fields_ = [("data", _vp), ("numel", _u64)]


class df11_sections(ctypes.Structure):
    _fields_ = [
        ("version", _u32), ("n_mats", _u32), ("n_symbols", _u32), ("max_code_len", _u32),
        ("n_tables", _u32), ("reserved", _u32),
        ("n_total", _u64), ("total_bits", _u64), ("n_windows", _u64), ("n_units", _u64),
        ("max_unit_count", _u64),
        ("code_len", _vp), ("mat_offset", _vp),
        ("stream", _vp), ("stream_bytes", _u64),
        ("sign_mant", _vp), ("sign_mant_bytes", _u64),
        ("gaps", _vp), ("gaps_bytes", _u64),
        ("unit_pos", _vp),
        ("tables", _vp), ("tables_bytes", _u64),
        ("blob", _vp), ("blob_bytes", _u64),
        ("off_code_len", _u64), ("off_mat_offset", _u64), ("off_stream", _u64),
        ("off_sign_mant", _u64), ("off_gaps", _u64), ("off_unit_pos", _u64), ("off_tables", _u64),
        ("exp_entropy_bits", ctypes.c_double), ("mean_code_len_bits", ctypes.c_double),
        ("counts", _vp), ("counts_bytes", _u64), ("off_counts", _u64),
        ("unit_end", _vp), ("unit_end_bytes", _u64), ("off_unit_end", _u64),
    ]


class df11_device_block(ctypes.Structure):
    _fields_ = [
        ("tables", _vp), ("tables_bytes", _u64),
        ("stream", _vp), ("stream_bytes", _u64),
        ("sign_mant", _vp), ("sign_mant_bytes", _u64),
        ("gaps", _vp), ("gaps_bytes", _u64),
        ("unit_pos", _vp),
        ("n_total", _u64), ("total_bits", _u64), ("n_windows", _u64), ("n_units", _u64),
        ("max_unit_count", _u64),
        ("version", _u32), ("n_tables", _u32),
        ("counts", _vp),
        ("unit_end", _vp),
    ]


class df11_gpu_plan(ctypes.Structure):
    _fields_ = [
        ("code_len", ctypes.c_uint8 * 256),
        ("n_symbols", _u32), ("max_code_len", _u32), ("n_tables", _u32), ("flags", _u32),
        ("n_total", _u64), ("total_bits", _u64), ("n_windows", _u64), ("n_units", _u64),
        ("stream_bytes", _u64), ("sign_mant_bytes", _u64), ("gaps_bytes", _u64), ("unit_pos_bytes", _u64),
        ("counts_bytes", _u64), ("tables_bytes", _u64), ("workspace_bytes", _u64),
    ]


class df11_launch(ctypes.Structure):
    _fields_ = [("waves_per_group", _u32), ("max_groups", _u32), ("variant", _u32), ("oversubscribe", _u32)]


DF11_VARIANT_SINGLE = 1
DF11_VARIANT_MULTI = 2
DF11_VARIANT_COUNTS = 3
DF11_ENCODE_WINDOW_COUNTS = 1
DF11_ENCODE_ALIGNED_UNITS = 2


class DF11Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {df11_status_str(status)} ({status})")


_lib = None

EXPORTS = [
    "df11_encode_block", "df11_encode_block_ex", "df11_encoded_sections", "df11_encoded_free", "df11_validate",
    "df11_tables_size", "df11_build_tables", "df11_device_block_from_blob", "df11_decode_block",
    "df11_decode_block_ex", "df11_status_str", "df11_last_hip_error", "df11_hip_error_name",
    "df11_gpu_chunk_hist_bytes", "df11_gpu_histogram", "df11_gpu_plan_build", "df11_gpu_encode",
    "df11_bandwidth_reference", "df11_gpu_encode_noalloc",
]

DF11_REFERENCE_SKELETON = 1
DF11_REFERENCE_STREAM = 2
DF11_REFERENCE_WRITES = 3
DF11_REFERENCE_READS = 4


def lib():
    """The loaded libdf11 (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with python -m huffman_decode_block_amd.build")
    from .build import built_stamp, source_stamp
    have, want = built_stamp(), source_stamp()
    if have != want:
        raise ImportError(f"{LIB_PATH} was built from other sources (stamp {have}, sources {want}): "
                          "rebuild it with python -m huffman_decode_block_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    L.df11_encode_block.argtypes = [P(df11_bf16_view), _u32, _u32, P(_vp)]
    L.df11_encode_block.restype = ctypes.c_int32
    L.df11_encode_block_ex.argtypes = [P(df11_bf16_view), _u32, _u32, _u32, P(_vp)]
    L.df11_encode_block_ex.restype = ctypes.c_int32
    L.df11_encoded_sections.argtypes = [_vp, P(df11_sections)]
    L.df11_encoded_sections.restype = ctypes.c_int32
    L.df11_encoded_free.argtypes = [_vp]
    L.df11_encoded_free.restype = None
    L.df11_validate.argtypes = [P(df11_sections)]
    L.df11_validate.restype = ctypes.c_int32
    L.df11_tables_size.argtypes = [_vp, P(_u64), P(_u32)]
    L.df11_tables_size.restype = ctypes.c_int32
    L.df11_build_tables.argtypes = [_vp, _vp, _u64]
    L.df11_build_tables.restype = ctypes.c_int32
    L.df11_device_block_from_blob.argtypes = [P(df11_sections), _vp, P(df11_device_block)]
    L.df11_device_block_from_blob.restype = ctypes.c_int32
    L.df11_decode_block.argtypes = [P(df11_device_block), _vp, _u64, _vp]
    L.df11_decode_block.restype = ctypes.c_int32
    L.df11_gpu_chunk_hist_bytes.argtypes = [_u64]
    L.df11_gpu_chunk_hist_bytes.restype = _u64
    L.df11_gpu_histogram.argtypes = [_vp, _u64, _vp, _vp, _vp]
    L.df11_gpu_histogram.restype = ctypes.c_int32
    L.df11_gpu_plan_build.argtypes = [_vp, _u32, P(df11_gpu_plan)]
    L.df11_gpu_plan_build.restype = ctypes.c_int32
    L.df11_gpu_encode.argtypes = [P(df11_gpu_plan), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    L.df11_gpu_encode.restype = ctypes.c_int32
    L.df11_decode_block_ex.argtypes = [P(df11_device_block), _vp, _u64, _vp, P(df11_launch)]
    L.df11_decode_block_ex.restype = ctypes.c_int32
    L.df11_gpu_encode_noalloc.argtypes = [P(df11_gpu_plan), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    L.df11_gpu_encode_noalloc.restype = ctypes.c_int32
    L.df11_bandwidth_reference.argtypes = [P(df11_device_block), _vp, _u64, _u32, _vp, P(df11_launch)]
    L.df11_bandwidth_reference.restype = ctypes.c_int32
    L.df11_status_str.argtypes = [ctypes.c_int32]
    L.df11_status_str.restype = ctypes.c_char_p
    L.df11_last_hip_error.argtypes = []
    L.df11_last_hip_error.restype = ctypes.c_int32
    L.df11_hip_error_name.argtypes = [ctypes.c_int32]
    L.df11_hip_error_name.restype = ctypes.c_char_p
    _lib = L
    return L


def library_stamp() -> str:
    """The source stamp of the loaded library (see the build module)."""
    lib()
    from .build import built_stamp
    return built_stamp()


def df11_status_str(status: int) -> str:
    return lib().df11_status_str(int(status)).decode()


def df11_last_hip_error() -> int:
    return int(lib().df11_last_hip_error())


def df11_hip_error_name(code: int) -> str:
    return lib().df11_hip_error_name(int(code)).decode()


def _check(status: int, what: str):
    if status != DF11_OK:
        if status == DF11_E_HIP:
            code = df11_last_hip_error()
            what = f"{what} [HIP error {code}: {df11_hip_error_name(code)}]"
        raise DF11Error(status, what)


def _as_u16(m) -> np.ndarray:
    """Raw BF16 bits of a host array / CPU tensor as a contiguous uint16 array."""
    try:
        import torch
        if isinstance(m, torch.Tensor):
            if m.is_cuda:
                raise ValueError("the encoder takes host tensors")
            if m.dtype == torch.bfloat16:
                m = m.contiguous().view(torch.int16)
            return m.contiguous().numpy().view(np.uint16).reshape(-1)
    except ImportError:
        pass
    a = np.ascontiguousarray(m)
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError(f"expected BF16 bits (uint16/int16 or torch.bfloat16), got {a.dtype}")
    return a.reshape(-1)


def _np_view(ptr: int, count: int, dtype, owner=None) -> np.ndarray:
    """A numpy view of library memory; it keeps `owner` (the object that frees
    that memory) alive for as long as the view, or any view of it, exists."""
    if count == 0:
        return np.zeros(0, dtype=dtype)
    ctype = np.ctypeslib.as_ctypes_type(dtype)
    arr = (ctype * count).from_address(ptr)
    arr._owner = owner
    return np.ctypeslib.as_array(arr)


class Sections:
    """Numpy views of one encoded blob.  Every view keeps the blob's Encoded
    alive; only an explicit Encoded.free() ends them early."""

    def __init__(self, owner, s: df11_sections):
        self._owner = owner
        self.raw = s
        self.version = s.version
        self.n_mats = s.n_mats
        self.n_symbols = s.n_symbols
        self.max_code_len = s.max_code_len
        self.n_tables = s.n_tables
        self.n_total = s.n_total
        self.total_bits = s.total_bits
        self.n_windows = s.n_windows
        self.n_units = s.n_units
        self.max_unit_count = s.max_unit_count
        self.exp_entropy_bits = s.exp_entropy_bits
        self.mean_code_len_bits = s.mean_code_len_bits
        self.code_len = _np_view(s.code_len, 256, np.uint8, owner)
        self.mat_offset = _np_view(s.mat_offset, s.n_mats + 1, np.uint64, owner)
        self.stream = _np_view(s.stream, s.stream_bytes, np.uint8, owner)
        self.sign_mant = _np_view(s.sign_mant, s.sign_mant_bytes, np.uint8, owner)
        self.gaps = _np_view(s.gaps, s.gaps_bytes, np.uint8, owner)
        self.unit_pos = _np_view(s.unit_pos, s.n_units + 1, np.uint64, owner)
        self.tables = _np_view(s.tables, s.tables_bytes, np.uint8, owner)
        self.blob = _np_view(s.blob, s.blob_bytes, np.uint8, owner)
        # optional per-window code counts (64 * n_units bytes), else None
        self.counts = _np_view(s.counts, s.counts_bytes, np.uint8, owner) if s.counts_bytes else None
        # aligned-units layout: where each unit's codes end, from its first bit; else None
        self.unit_end = _np_view(s.unit_end, s.n_units, np.uint16, owner) if s.unit_end_bytes else None

    @property
    def compressed_bytes(self) -> int:
        """Bytes a decode reads: stream, sign/mantissa, gaps, positions, tables
        (and the unit ends of the aligned-units layout)."""
        return int(self.raw.stream_bytes + self.raw.sign_mant_bytes + self.raw.gaps_bytes
                   + 8 * (self.n_units + 1) + self.raw.tables_bytes + self.raw.unit_end_bytes)


class Encoded:
    """Owner of a df11_encoded blob (host memory allocated by the library)."""

    def __init__(self, handle: int):
        self._h = handle
        s = df11_sections()
        _check(lib().df11_encoded_sections(handle, ctypes.byref(s)), "df11_encoded_sections")
        self.sections = Sections(self, s)

    def free(self):
        if self._h:
            lib().df11_encoded_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.free()


def df11_encode_block(mats, n_threads: int = 0, window_counts: bool = False, aligned_units: bool = False) -> Encoded:
    """Encode a list of BF16 matrices (host) as one block with one codebook;
    window_counts adds the per-window code counts and aligned_units lays the
    codes out so that units start on 32-weight boundaries (df11_encode_block_ex
    with DF11_ENCODE_WINDOW_COUNTS / DF11_ENCODE_ALIGNED_UNITS)."""
    flags = (DF11_ENCODE_WINDOW_COUNTS if window_counts else 0) | (DF11_ENCODE_ALIGNED_UNITS if aligned_units else 0)
    return df11_encode_block_ex(mats, n_threads, flags)


def df11_encode_block_ex(mats, n_threads: int = 0, flags: int = 0) -> Encoded:
    arrays = [_as_u16(m) for m in mats]
    views = (df11_bf16_view * max(1, len(arrays)))()
    for i, a in enumerate(arrays):
        views[i].data = a.ctypes.data if a.size else None
        views[i].numel = a.size
    h = _vp()
    if flags:
        _check(lib().df11_encode_block_ex(views, len(arrays), n_threads, flags, ctypes.byref(h)),
               "df11_encode_block_ex")
    else:
        _check(lib().df11_encode_block(views, len(arrays), n_threads, ctypes.byref(h)), "df11_encode_block")
    return Encoded(h.value)


def df11_encoded_sections(enc: Encoded) -> Sections:
    return enc.sections


def df11_encoded_free(enc: Encoded) -> None:
    enc.free()


def df11_validate(sections: Sections) -> int:
    """Host-side structural check; returns the status code."""
    return int(lib().df11_validate(ctypes.byref(sections.raw)))


def df11_tables_size(code_len) -> tuple:
    cl = np.ascontiguousarray(np.asarray(code_len, dtype=np.uint8).reshape(256))
    nb, nt = _u64(), _u32()
    _check(lib().df11_tables_size(cl.ctypes.data, ctypes.byref(nb), ctypes.byref(nt)), "df11_tables_size")
    return int(nb.value), int(nt.value)


def df11_build_tables(code_len) -> np.ndarray:
    cl = np.ascontiguousarray(np.asarray(code_len, dtype=np.uint8).reshape(256))
    nb, _ = df11_tables_size(cl)
    out = np.zeros(nb, dtype=np.uint8)
    _check(lib().df11_build_tables(cl.ctypes.data, out.ctypes.data, nb), "df11_build_tables")
    return out


def df11_device_block_from_blob(sections: Sections, device_ptr: int) -> df11_device_block:
    b = df11_device_block()
    _check(lib().df11_device_block_from_blob(ctypes.byref(sections.raw), device_ptr, ctypes.byref(b)),
           "df11_device_block_from_blob")
    return b


class DeviceBlock:
    """An encoded block resident in device memory (torch tensors) plus the
    df11_device_block that describes it."""

    def __init__(self, raw: df11_device_block, keep: list, n_total: int, mat_offset=None):
        self.raw = raw
        self._keep = keep
        self.n_total = int(n_total)
        self.mat_offset = None if mat_offset is None else np.asarray(mat_offset, dtype=np.int64)

    @classmethod
    def from_encoded(cls, enc: Encoded, device="cuda") -> "DeviceBlock":
        import torch
        s = enc.sections
        blob = torch.empty(int(s.raw.blob_bytes), dtype=torch.uint8, device=device)
        blob.copy_(torch.from_numpy(s.blob))
        raw = df11_device_block_from_blob(s, blob.data_ptr())
        return cls(raw, [blob], s.n_total, s.mat_offset.copy())

    @classmethod
    def from_parts(cls, *, code_len, stream, sign_mant, gaps, unit_pos, n_total, total_bits,
                   counts=None, unit_end=None, device="cuda") -> "DeviceBlock":
        """Device block from separately given host sections (for example the
        oracle's); the decode tables are built here from code_len.  counts:
        optional per-window code counts (padded here to 64 per unit);
        unit_end: the unit ends of the aligned-units layout."""
        import torch
        tables = df11_build_tables(code_len)
        _, n_tables = df11_tables_size(code_len)
        up = np.ascontiguousarray(unit_pos, dtype=np.uint64)
        parts = {}
        arrays = [("tables", tables), ("stream", stream), ("sign_mant", sign_mant),
                  ("gaps", gaps), ("unit_pos", up.view(np.uint8))]
        if counts is not None:
            nu = ((int(total_bits) + 63) // 64 + 63) // 64
            c = np.zeros(64 * nu, dtype=np.uint8)
            c[:len(counts)] = np.asarray(counts, dtype=np.uint8)[:64 * nu]
            arrays.append(("counts", c))
        if unit_end is not None:
            arrays.append(("unit_end", np.ascontiguousarray(unit_end, dtype=np.uint16)))
        for name, arr in arrays:
            a = np.ascontiguousarray(arr).view(np.uint8).reshape(-1)
            t = torch.empty(max(1, a.size), dtype=torch.uint8, device=device)
            if a.size:
                t[:a.size].copy_(torch.from_numpy(a))
            parts[name] = (t, a.size)
        b = df11_device_block()
        b.tables, b.tables_bytes = parts["tables"][0].data_ptr(), parts["tables"][1]
        b.stream, b.stream_bytes = parts["stream"][0].data_ptr(), parts["stream"][1]
        b.sign_mant, b.sign_mant_bytes = parts["sign_mant"][0].data_ptr(), parts["sign_mant"][1]
        b.gaps, b.gaps_bytes = parts["gaps"][0].data_ptr(), parts["gaps"][1]
        b.unit_pos = parts["unit_pos"][0].data_ptr()
        b.n_total = int(n_total)
        b.total_bits = int(total_bits)
        b.n_windows = (int(total_bits) + 63) // 64
        b.n_units = (b.n_windows + 63) // 64
        d = np.diff(up.astype(np.int64))
        b.max_unit_count = int(d.max()) if d.size else 0
        b.version = DF11_FORMAT_VERSION
        b.n_tables = n_tables
        b.counts = parts["counts"][0].data_ptr() if "counts" in parts else None
        b.unit_end = parts["unit_end"][0].data_ptr() if "unit_end" in parts else None
        return cls(b, [t for t, _ in parts.values()], n_total)

    def compressed_bytes(self) -> int:
        r = self.raw
        return int(r.stream_bytes + r.sign_mant_bytes + r.gaps_bytes + 8 * (r.n_units + 1) + r.tables_bytes)


def _device_tensor(t, name, min_bytes=0, sixteen_bit=False, dev=None):
    """Checks a tensor handed to the library: on a GPU (the given one, if any),
    contiguous, of at least min_bytes; raises before anything is launched."""
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, not {dev}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if sixteen_bit and t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must hold 16-bit values")
    if t.numel() * t.element_size() < min_bytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, {min_bytes} needed")


def _stream_handle(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def df11_decode_block(block: DeviceBlock, out=None, stream=None, launch=None):
    """Decode `block` into `out` (a flat torch.bfloat16 device tensor with at
    least n_total elements; allocated when None) on `stream` (torch stream,
    raw handle, or None for the current stream).  Returns out."""
    import torch
    if out is None:
        dev = torch.device("cuda", torch.cuda.current_device())
        out = torch.empty(max(1, block.n_total), dtype=torch.bfloat16, device=dev)
    if out.dtype not in (torch.bfloat16, torch.int16, torch.uint16) or not out.is_cuda:
        raise TypeError("out must be a 16-bit device tensor")
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    h = _stream_handle(stream, out.device)
    with torch.cuda.device(out.device):  # the launch goes to the output's GPU
        if launch is None:
            st = lib().df11_decode_block(ctypes.byref(block.raw), out.data_ptr(), out.numel(), h)
        else:
            L = launch if isinstance(launch, df11_launch) else df11_launch(*launch)
            st = lib().df11_decode_block_ex(ctypes.byref(block.raw), out.data_ptr(), out.numel(), h,
                                            ctypes.byref(L))
    _check(st, "df11_decode_block")
    return out


def df11_decode_block_ex(block: DeviceBlock, out=None, stream=None, waves_per_group=0, max_groups=0,
                         variant=0, oversubscribe=0):
    return df11_decode_block(block, out, stream, launch=(waves_per_group, max_groups, variant, oversubscribe))


def df11_bandwidth_reference(block: DeviceBlock, out, kind: int, stream=None, launch=None):
    """A bandwidth reference for the decode of `block`: DF11_REFERENCE_SKELETON
    or DF11_REFERENCE_STREAM move the decode's HBM bytes and write into `out`
    (a 16-bit device tensor) each weight with its exponent field zero;
    DF11_REFERENCE_WRITES writes zeros only, DF11_REFERENCE_READS reads the
    sections only.  Returns out."""
    import torch
    if out.dtype not in (torch.bfloat16, torch.int16, torch.uint16) or not out.is_cuda:
        raise TypeError("out must be a 16-bit device tensor")
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    L = None if launch is None else (launch if isinstance(launch, df11_launch) else df11_launch(*launch))
    with torch.cuda.device(out.device):
        st = lib().df11_bandwidth_reference(ctypes.byref(block.raw), out.data_ptr(), out.numel(), int(kind),
                                            _stream_handle(stream, out.device),
                                            None if L is None else ctypes.byref(L))
    _check(st, "df11_bandwidth_reference")
    return out


def df11_gpu_chunk_hist_bytes(n: int) -> int:
    """Bytes of the per-chunk exponent counts of n weights (256 uint16 per 4,096 weights)."""
    return int(lib().df11_gpu_chunk_hist_bytes(int(n)))


def df11_gpu_histogram(x, hist, chunk_hist=None, stream=None) -> None:
    """hist (device, 256 int64) := exponent histogram of x (16-bit device
    tensor); chunk_hist (device, df11_gpu_chunk_hist_bytes(x.numel()) bytes, or
    None) := the 256 counts of every chunk of 4,096 weights, as uint16."""
    import torch
    _device_tensor(x, "x", sixteen_bit=True)
    _device_tensor(hist, "hist", 256 * 8, dev=x.device)
    if hist.element_size() != 8:
        raise TypeError("hist must hold 64-bit counts")
    if chunk_hist is not None:
        _device_tensor(chunk_hist, "chunk_hist", df11_gpu_chunk_hist_bytes(x.numel()), dev=x.device)
    ptr = None if chunk_hist is None else chunk_hist.data_ptr()
    with torch.cuda.device(x.device):
        st = lib().df11_gpu_histogram(x.data_ptr(), x.numel(), hist.data_ptr(), ptr, _stream_handle(stream, x.device))
    _check(st, "df11_gpu_histogram")


def df11_gpu_plan_build(hist, flags: int = 0) -> df11_gpu_plan:
    """The GPU encoder's plan for a host histogram (256 counts)."""
    h = np.ascontiguousarray(hist, dtype=np.uint64)
    if h.size != 256:
        raise ValueError("a histogram has 256 counts")
    plan = df11_gpu_plan()
    _check(lib().df11_gpu_plan_build(h.ctypes.data, flags, ctypes.byref(plan)), "df11_gpu_plan_build")
    return plan


def df11_gpu_encode(plan: df11_gpu_plan, x, chunk_hist, stream_buf, sign_mant, gaps, unit_pos, counts, workspace,
                    stream=None) -> None:
    """Packs the sections of x (device) into the given device tensors (sizes
    from the plan); chunk_hist holds the per-chunk counts df11_gpu_histogram
    took from the same x."""
    import torch
    _device_tensor(x, "x", 2 * int(plan.n_total), sixteen_bit=True)
    need = {"stream_buf": (stream_buf, plan.stream_bytes), "sign_mant": (sign_mant, plan.sign_mant_bytes),
            "gaps": (gaps, plan.gaps_bytes), "unit_pos": (unit_pos, plan.unit_pos_bytes),
            "counts": (counts, plan.counts_bytes), "workspace": (workspace, plan.workspace_bytes),
            "chunk_hist": (chunk_hist, df11_gpu_chunk_hist_bytes(int(plan.n_total)))}
    for name, (t, nbytes) in need.items():
        if t is not None:  # a missing section is the library's to refuse
            _device_tensor(t, name, int(nbytes), dev=x.device)
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    with torch.cuda.device(x.device):
        st = lib().df11_gpu_encode(ctypes.byref(plan), ptr(x), ptr(chunk_hist), ptr(stream_buf), ptr(sign_mant),
                                   ptr(gaps), ptr(unit_pos), ptr(counts), ptr(workspace),
                                   _stream_handle(stream, x.device))
    _check(st, "df11_gpu_encode")


DF11_NOALLOC_WORKSPACE_BYTES = 48 << 20  # the workspace array of df11_gpu_encode_noalloc


def df11_gpu_encode_noalloc(plan: df11_gpu_plan, x, chunk_hist, stream_buf, sign_mant, gaps, unit_pos, counts,
                            stream=None) -> None:
    """df11_gpu_encode without a workspace argument: the library's own device
    array serves (no device memory is allocated)."""
    import torch
    _device_tensor(x, "x", 2 * int(plan.n_total), sixteen_bit=True)
    need = {"stream_buf": (stream_buf, plan.stream_bytes), "sign_mant": (sign_mant, plan.sign_mant_bytes),
            "gaps": (gaps, plan.gaps_bytes), "unit_pos": (unit_pos, plan.unit_pos_bytes),
            "counts": (counts, plan.counts_bytes),
            "chunk_hist": (chunk_hist, df11_gpu_chunk_hist_bytes(int(plan.n_total)))}
    for name, (t, nbytes) in need.items():
        if t is not None:
            _device_tensor(t, name, int(nbytes), dev=x.device)
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    with torch.cuda.device(x.device):
        st = lib().df11_gpu_encode_noalloc(ctypes.byref(plan), ptr(x), ptr(chunk_hist), ptr(stream_buf),
                                           ptr(sign_mant), ptr(gaps), ptr(unit_pos), ptr(counts),
                                           _stream_handle(stream, x.device))
    _check(st, "df11_gpu_encode_noalloc")


class GpuEncoded:
    """A block encoded on the device: its plan, the section tensors and a
    DeviceBlock ready for df11_decode_block."""

    def __init__(self, plan, tensors: dict, block: "DeviceBlock"):
        self.plan = plan
        self.tensors = tensors
        self.block = block

    def section(self, name) -> np.ndarray:
        """Host copy of a section as bytes (stream, sign_mant, gaps, unit_pos, counts)."""
        t = self.tensors[name]
        return t.cpu().numpy().view(np.uint8).reshape(-1)


def gpu_encode(x, window_counts: bool = False, stream=None, mat_offset=None) -> GpuEncoded:
    """Encode a block whose BF16 weights are in device memory (a contiguous
    16-bit tensor, matrices concatenated).  The histogram's 256 counts come
    back to the host for the code lengths (this synchronizes `stream`); every
    other step runs on the device."""
    import torch
    if x.dtype not in (torch.bfloat16, torch.int16, torch.uint16) or not x.is_cuda or not x.is_contiguous():
        raise TypeError("x must be a contiguous 16-bit device tensor")
    dev = x.device
    flat = x.reshape(-1)
    hist = torch.empty(256, dtype=torch.int64, device=dev)
    chunk_hist = torch.empty(max(8, df11_gpu_chunk_hist_bytes(flat.numel()) // 2), dtype=torch.int16, device=dev)
    df11_gpu_histogram(flat, hist, chunk_hist, stream)
    torch.cuda.synchronize(dev)  # the counts go to the host
    plan = df11_gpu_plan_build(hist.cpu().numpy().astype(np.uint64), DF11_ENCODE_WINDOW_COUNTS if window_counts else 0)
    t = {
        "stream": torch.empty(max(16, plan.stream_bytes), dtype=torch.uint8, device=dev),
        "sign_mant": torch.empty(max(16, plan.sign_mant_bytes), dtype=torch.uint8, device=dev),
        "gaps": torch.empty(max(16, plan.gaps_bytes), dtype=torch.uint8, device=dev),
        "unit_pos": torch.empty(plan.n_units + 1, dtype=torch.int64, device=dev),
        "counts": torch.empty(plan.counts_bytes, dtype=torch.uint8, device=dev) if window_counts else None,
        "workspace": torch.empty(max(16, plan.workspace_bytes), dtype=torch.uint8, device=dev),
        "chunk_hist": chunk_hist,
    }
    code_len = np.frombuffer(bytes(plan.code_len), dtype=np.uint8).copy()
    tables = df11_build_tables(code_len)
    t["tables"] = torch.from_numpy(tables.view(np.uint8).reshape(-1).copy()).to(dev)
    df11_gpu_encode(plan, flat, chunk_hist, t["stream"], t["sign_mant"], t["gaps"], t["unit_pos"], t["counts"],
                    t["workspace"], stream)
    b = df11_device_block()
    b.tables, b.tables_bytes = t["tables"].data_ptr(), plan.tables_bytes
    b.stream, b.stream_bytes = t["stream"].data_ptr(), plan.stream_bytes
    b.sign_mant, b.sign_mant_bytes = t["sign_mant"].data_ptr(), plan.sign_mant_bytes
    b.gaps, b.gaps_bytes = t["gaps"].data_ptr(), plan.gaps_bytes
    b.unit_pos = t["unit_pos"].data_ptr()
    b.n_total, b.total_bits, b.n_windows, b.n_units = plan.n_total, plan.total_bits, plan.n_windows, plan.n_units
    b.version = DF11_FORMAT_VERSION
    b.n_tables = plan.n_tables
    b.counts = t["counts"].data_ptr() if window_counts else None
    # the largest unit is only known from unit_pos: read it back (small)
    torch.cuda.synchronize(dev)
    up = t["unit_pos"].cpu().numpy().astype(np.int64)
    b.max_unit_count = int(np.diff(up).max()) if up.size > 1 else 0
    blk = DeviceBlock(b, [v for v in t.values() if v is not None], int(plan.n_total),
                      None if mat_offset is None else np.asarray(mat_offset, dtype=np.int64))
    return GpuEncoded(plan, t, blk)


def matrix_views(out, block_or_offsets, shapes=None):
    """Per-matrix views of a decoded block output."""
    off = block_or_offsets.mat_offset if hasattr(block_or_offsets, "mat_offset") else block_or_offsets
    off = [int(v) for v in off]
    views = []
    for i in range(len(off) - 1):
        v = out[off[i]:off[i + 1]]
        if shapes is not None:
            v = v.view(*shapes[i])
        views.append(v)
    return views


__all__ = [
    "df11_encode_block", "df11_encode_block_ex", "df11_encoded_sections", "df11_encoded_free", "df11_validate",
    "df11_tables_size", "df11_build_tables", "df11_device_block_from_blob", "df11_decode_block",
    "df11_decode_block_ex", "df11_status_str", "df11_last_hip_error", "df11_hip_error_name",
    "df11_gpu_chunk_hist_bytes", "df11_gpu_histogram", "df11_gpu_plan_build", "df11_gpu_encode", "gpu_encode",
    "GpuEncoded", "df11_bandwidth_reference", "df11_gpu_encode_noalloc", "DF11_NOALLOC_WORKSPACE_BYTES", "DF11_REFERENCE_SKELETON", "DF11_REFERENCE_STREAM", "DF11_REFERENCE_WRITES", "DF11_REFERENCE_READS",
    "Encoded", "Sections",
    "DeviceBlock", "DF11Error", "matrix_views", "lib", "library_stamp",
]
