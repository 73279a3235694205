"""Python binding of libshannonic.so: the C ABI of include/shannonic.h, same names.

Argument marshalling only -- every step of the codec runs in the library (HIP kernels
on the GPU, the table build on the host in C++).  PyTorch provides device memory and
streams.  There is no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import numpy as np

from . import build as _build

SH_OK = 0
SH_ERR_INVALID_ARG = -1
SH_ERR_UNSUPPORTED = -2
SH_ERR_SYMBOL_NOT_IN_TABLE = -3
SH_ERR_CORRUPT_STREAM = -4
SH_ERR_BUFFER_TOO_SMALL = -5
SH_ERR_HIP = -6


class sh_params(C.Structure):
    _fields_ = [("K", C.c_uint32), ("log2_L", C.c_uint32), ("chunk_symbols", C.c_uint32),
                ("streams", C.c_uint32)]


class sh_table(C.Structure):
    _fields_ = [("K", C.c_uint32), ("log2_L", C.c_uint32), ("lo", C.c_uint16 * 257),
                ("freq", C.c_uint16 * 256), ("hist", C.c_uint64 * 256), ("n", C.c_uint64)]

    @property
    def lo_array(self) -> np.ndarray:
        return np.array(self.lo[: self.K + 1], dtype=np.uint16)

    @property
    def freq_array(self) -> np.ndarray:
        return np.array(self.freq[: self.K], dtype=np.uint16)

    @property
    def hist_array(self) -> np.ndarray:
        return np.array(self.hist[:], dtype=np.uint64)


STAT_FIELDS = ["H", "H_P", "D_KL", "sum_Pw", "cl_thm1", "H_p_given_P", "dkl_tans_ref",
               "cl_tans_ref", "payload_bps", "container_bps", "csr", "pct_payload_over_H",
               "pct_container_over_H", "pct_thm1_over_H"]


class sh_stats_t(C.Structure):
    _fields_ = [(f, C.c_double) for f in STAT_FIELDS]


class sh_encode_info(C.Structure):
    _fields_ = [("container_bytes", C.c_uint64), ("payload_bits", C.c_uint64)]


class ShannonicError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


_lib = None
_EXPORTS = {
    "sh_version": (C.c_uint32, []),
    "sh_status_string": (C.c_char_p, [C.c_int32]),
    "sh_histogram": (C.c_int32, [C.c_void_p, C.c_uint64, C.c_void_p, C.c_void_p]),
    "sh_table_from_histogram": (C.c_int32, [C.c_void_p, C.POINTER(sh_params), C.POINTER(sh_table)]),
    "sh_build_tables_workspace": (C.c_uint64, []),
    "sh_build_tables": (C.c_int32, [C.c_void_p, C.c_uint64, C.c_int, C.POINTER(sh_params),
                                    C.c_void_p, C.c_uint64, C.c_void_p, C.POINTER(sh_table)]),
    "sh_encode_bound": (C.c_uint64, [C.c_uint64, C.POINTER(sh_params)]),
    "sh_encode_workspace": (C.c_uint64, [C.c_uint64, C.POINTER(sh_params)]),
    "sh_encode": (C.c_int32, [C.POINTER(sh_table), C.POINTER(sh_params), C.c_void_p, C.c_uint64,
                              C.c_void_p, C.c_uint64, C.c_void_p, C.c_uint64, C.c_void_p,
                              C.c_void_p, C.c_void_p]),
    "sh_encode_noalloc_scratch_bytes": (C.c_uint64, []),
    "sh_encode_noalloc": (C.c_int32, [C.POINTER(sh_table), C.POINTER(sh_params), C.c_void_p,
                                      C.c_uint64, C.c_void_p, C.c_uint64, C.c_void_p, C.c_void_p,
                                      C.c_void_p]),
    "sh_decode": (C.c_int32, [C.POINTER(sh_table), C.POINTER(sh_params), C.c_void_p, C.c_uint64,
                              C.c_void_p, C.c_uint64, C.c_void_p, C.c_void_p]),
    "sh_stats": (C.c_int32, [C.POINTER(sh_table), C.c_uint64, C.c_uint64, C.c_uint64,
                             C.POINTER(sh_stats_t)]),
    "sh_stats_batch": (C.c_int32, [C.c_void_p, C.c_uint32, C.c_void_p, C.c_void_p, C.c_void_p,
                                   C.c_void_p]),
    "sh_device_table_bytes": (C.c_uint64, []),
    "sh_table_to_device": (C.c_int32, [C.POINTER(sh_table), C.POINTER(sh_params), C.c_void_p,
                                       C.c_void_p]),
    "sh_tables_from_device": (C.c_int32, [C.c_void_p, C.c_uint32, C.c_void_p, C.c_void_p,
                                          C.c_void_p]),
    "sh_tables_from_bytes": (C.c_int32, [C.c_void_p, C.c_uint32, C.c_void_p, C.c_void_p]),
    "sh_build_tables_batch_workspace": (C.c_uint64, [C.c_uint32]),
    "sh_build_tables_batch": (C.c_int32, [C.c_void_p, C.c_void_p, C.c_uint32,
                                          C.POINTER(sh_params), C.c_void_p, C.c_void_p,
                                          C.c_uint64, C.c_void_p]),
    "sh_encode_batch_workspace": (C.c_uint64, [C.c_void_p, C.c_uint32, C.POINTER(sh_params)]),
    "sh_encode_batch": (C.c_int32, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_uint32,
                                    C.POINTER(sh_params), C.c_void_p, C.c_void_p, C.c_void_p,
                                    C.c_uint64, C.c_void_p, C.c_void_p, C.c_void_p,
                                    C.c_void_p]),
    "sh_decode_batch": (C.c_int32, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                    C.c_uint32, C.POINTER(sh_params), C.c_void_p, C.c_void_p]),
    "sh_decode_matvec_batch": (C.c_int32, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                           C.c_void_p, C.c_void_p, C.c_uint32, C.c_uint32,
                                           C.POINTER(sh_params), C.c_void_p, C.c_void_p]),
    "sh_decode_stream_staging": (C.c_uint64, [C.c_void_p, C.c_uint32, C.c_uint32]),
    "sh_decode_stream": (C.c_int32, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                     C.c_uint32, C.POINTER(sh_params), C.c_void_p, C.c_uint64,
                                     C.c_uint32, C.c_void_p, C.c_void_p, C.c_void_p]),
}


def library_path() -> str:
    return _build.LIB


def lib():
    """The loaded library; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"libshannonic.so is not built ({path}); run "
                               "`python -m entropy_coding_quantized_amd.build`")
        L = C.CDLL(path)
        for name, (res, args) in _EXPORTS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(st: int) -> str:
    return lib().sh_status_string(st).decode()


def _check(st: int, what: str):
    if st != SH_OK:
        raise ShannonicError(st, what)


@dataclass(frozen=True)
class Params:
    K: int = 16
    log2_L: int = 7
    chunk_symbols: int = 4096
    streams: int = 32

    def c(self) -> sh_params:
        """The C struct (one per Params, built on first use: the calls only read it)."""
        c = self.__dict__.get("_c")
        if c is None:
            c = sh_params(self.K, self.log2_L, self.chunk_symbols, self.streams)
            object.__setattr__(self, "_c", c)
        return c


def _ptr(t) -> int:
    """Device (or host) address of a torch tensor, a numpy array or an int."""
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _opt_stream(stream):
    """A stream argument that may be NULL: None stays None."""
    return None if stream is None else _stream(stream)


# ---- the C ABI, one to one -----------------------------------------------------------

def sh_version() -> int:
    return int(lib().sh_version())


def sh_histogram(d_x, n: int, d_hist, stream=None) -> None:
    _check(lib().sh_histogram(_ptr(d_x), n, _ptr(d_hist), _stream(stream)), "sh_histogram")


def sh_table_from_histogram(hist: np.ndarray, params: Params) -> sh_table:
    h = np.ascontiguousarray(hist, dtype=np.uint64)
    assert h.size == 256
    t = sh_table()
    p = params.c()
    _check(lib().sh_table_from_histogram(h.ctypes.data, C.byref(p), C.byref(t)),
           "sh_table_from_histogram")
    return t


def sh_build_tables_workspace() -> int:
    return int(lib().sh_build_tables_workspace())


def sh_build_tables(x, n: int, x_on_device: bool, params: Params, d_ws=None, ws_bytes: int = 0,
                    stream=None) -> sh_table:
    t = sh_table()
    p = params.c()
    st = lib().sh_build_tables(_ptr(x), n, int(bool(x_on_device)), C.byref(p), _ptr(d_ws),
                               ws_bytes, _stream(stream) if x_on_device else 0, C.byref(t))
    _check(st, "sh_build_tables")
    return t


def sh_encode_bound(n: int, params: Params) -> int:
    p = params.c()
    return int(lib().sh_encode_bound(n, C.byref(p)))


def sh_encode_workspace(n: int, params: Params) -> int:
    p = params.c()
    return int(lib().sh_encode_workspace(n, C.byref(p)))


def sh_encode(table: sh_table, params: Params, d_x, n: int, d_out, out_cap: int, d_ws,
              ws_bytes: int, d_info=None, d_status=None, stream=None) -> None:
    p = params.c()
    st = lib().sh_encode(C.byref(table), C.byref(p), _ptr(d_x), n, _ptr(d_out), out_cap,
                         _ptr(d_ws), ws_bytes, _ptr(d_info), _ptr(d_status), _stream(stream))
    _check(st, "sh_encode")


def sh_encode_noalloc_scratch_bytes() -> int:
    return lib().sh_encode_noalloc_scratch_bytes()


def sh_encode_noalloc(table: sh_table, params: Params, d_x, n: int, d_out, out_cap: int,
                      d_info=None, d_status=None, stream=None) -> None:
    p = params.c()
    st = lib().sh_encode_noalloc(C.byref(table), C.byref(p), _ptr(d_x), n, _ptr(d_out), out_cap,
                                 _ptr(d_info), _ptr(d_status), _stream(stream))
    _check(st, "sh_encode_noalloc")


def sh_decode(table: sh_table, params: Params, d_in, in_nbytes: int, d_y, n: int,
              d_status=None, stream=None) -> None:
    p = params.c()
    st = lib().sh_decode(C.byref(table), C.byref(p), _ptr(d_in), in_nbytes, _ptr(d_y), n,
                         _ptr(d_status), _stream(stream))
    _check(st, "sh_decode")


def sh_stats(table: sh_table, n: int = 0, payload_bits: int = 0, container_bytes: int = 0) -> dict:
    out = sh_stats_t()
    _check(lib().sh_stats(C.byref(table), n, payload_bits, container_bytes, C.byref(out)),
           "sh_stats")
    return {f: getattr(out, f) for f in STAT_FIELDS}


def sh_stats_batch(tables, n=None, payload_bits=None, container_bytes=None, out=None):
    """sh_stats of every table in one call; tables: a list of sh_table or a ctypes array of
    them.  Returns one dict per table, or, given out (a ctypes array of at least as many
    sh_stats_t), fills out and returns it."""
    if not isinstance(tables, C.Array):
        tables = (sh_table * max(len(tables), 1))(*tables)
    k = len(tables)
    raw = out is not None
    if raw and len(out) < k:
        raise ValueError("sh_stats_batch: out holds fewer records than tables")
    if not raw:
        out = (sh_stats_t * max(k, 1))()
    arrs = [None if a is None else _u64s(a) for a in (n, payload_bits, container_bytes)]
    _check(lib().sh_stats_batch(C.addressof(tables), k, *[None if a is None else C.addressof(a)
                                                          for a in arrs], C.addressof(out)),
           "sh_stats_batch")
    return out if raw else stats_dicts(out, k)


def stats_dicts(records, count: int) -> list:
    """sh_stats_t records as one dict per record."""
    return [{f: getattr(records[i], f) for f in STAT_FIELDS} for i in range(count)]


def _ptrs(items) -> C.Array:
    if isinstance(items, C.Array):
        return items
    return (C.c_void_p * max(len(items), 1))(*[_ptr(t) for t in items])


def _u64s(values) -> C.Array:
    if isinstance(values, C.Array):
        return values
    return (C.c_uint64 * max(len(values), 1))(*[int(v) for v in values])


def sh_device_table_bytes() -> int:
    return int(lib().sh_device_table_bytes())


def sh_table_to_device(table: sh_table, params: Params, d_table, stream=None) -> None:
    p = params.c()
    _check(lib().sh_table_to_device(C.byref(table), C.byref(p), _ptr(d_table), _stream(stream)),
           "sh_table_to_device")


def sh_tables_from_device(d_tables, count: int, stream=None):
    """([sh_table] * count, [build status] * count) of device tables."""
    out = (sh_table * max(count, 1))()
    st = (C.c_int32 * max(count, 1))()
    _check(lib().sh_tables_from_device(_ptr(d_tables), count, out, st, _stream(stream)),
           "sh_tables_from_device")
    return [out[i] for i in range(count)], [int(st[i]) for i in range(count)]


def sh_tables_from_bytes(tables, count: int, as_array: bool = False, out=None, status=None):
    """sh_tables_from_device for device-table images already in host memory.  With
    as_array, the tables come back as one ctypes array (for sh_stats_batch); out and status
    (ctypes arrays of at least count sh_table and int32) are filled instead of new ones."""
    if out is None:
        out = (sh_table * max(count, 1))()
    if status is None:
        status = (C.c_int32 * max(count, 1))()
    if len(out) < count or len(status) < count:
        raise ValueError("sh_tables_from_bytes: out or status holds fewer than count entries")
    _check(lib().sh_tables_from_bytes(_ptr(tables), count, out, status), "sh_tables_from_bytes")
    return ((out if as_array else [out[i] for i in range(count)]),
            [int(status[i]) for i in range(count)])


def table_from_device(d_table, stream=None) -> sh_table:
    """One device table; raises with the status its build recorded, if any."""
    (t,), (st,) = sh_tables_from_device(d_table, 1, stream)
    _check(st, "device table")
    return t


def sh_build_tables_batch_workspace(nseg: int) -> int:
    return int(lib().sh_build_tables_batch_workspace(nseg))


def sh_build_tables_batch(d_x: list, n: list, params: Params, d_tables, d_ws, ws_bytes: int,
                          stream=None) -> None:
    p = params.c()
    st = lib().sh_build_tables_batch(_ptrs(d_x), _u64s(n), len(n), C.byref(p), _ptr(d_tables),
                                     _ptr(d_ws), ws_bytes, _stream(stream))
    _check(st, "sh_build_tables_batch")


def sh_encode_batch_workspace(n: list, params: Params) -> int:
    p = params.c()
    return int(lib().sh_encode_batch_workspace(_u64s(n), len(n), C.byref(p)))


def sh_encode_batch(d_tables, d_x: list, n: list, params: Params, d_out: list, out_cap: list,
                    d_ws, ws_bytes: int, d_info=None, d_status=None, stream=None,
                    place_stream=None) -> None:
    p = params.c()
    st = lib().sh_encode_batch(_ptr(d_tables), _ptrs(d_x), _u64s(n), len(n), C.byref(p),
                               _ptrs(d_out), _u64s(out_cap), _ptr(d_ws), ws_bytes, _ptr(d_info),
                               _ptr(d_status), _stream(stream), _opt_stream(place_stream))
    _check(st, "sh_encode_batch")


def sh_decode_batch(d_tables, d_in: list, in_nbytes: list, d_y: list, n: list, params: Params,
                    d_status=None, stream=None) -> None:
    p = params.c()
    st = lib().sh_decode_batch(_ptr(d_tables), _ptrs(d_in), _u64s(in_nbytes), _ptrs(d_y),
                               _u64s(n), len(n), C.byref(p), _ptr(d_status), _stream(stream))
    _check(st, "sh_decode_batch")


def sh_decode_matvec_batch(d_tables, d_in: list, in_nbytes: list, d_a: list, d_y: list,
                           n: list, cols: int, params: Params, d_status=None,
                           stream=None) -> None:
    """y[i] += W_i a[i] for the int8 matrices W_i (rows of cols values) held by the
    containers, without writing W_i; d_a[i]: int8 vectors, d_y[i]: int32 outputs."""
    p = params.c()
    st = lib().sh_decode_matvec_batch(_ptr(d_tables), _ptrs(d_in), _u64s(in_nbytes), _ptrs(d_a),
                                      _ptrs(d_y), _u64s(n), cols, len(n), C.byref(p),
                                      _ptr(d_status), _stream(stream))
    _check(st, "sh_decode_matvec_batch")


def sh_decode_stream_staging(in_nbytes: list, depth: int) -> int:
    return int(lib().sh_decode_stream_staging(_u64s(in_nbytes), len(in_nbytes), depth))


def sh_decode_stream(d_tables, h_in: list, in_nbytes: list, d_y: list, n: list, params: Params,
                     d_staging, staging_bytes: int, depth: int, d_status=None, copy_stream=None,
                     stream=None) -> None:
    p = params.c()
    st = lib().sh_decode_stream(_ptr(d_tables), _ptrs(h_in), _u64s(in_nbytes), _ptrs(d_y),
                                _u64s(n), len(n), C.byref(p), _ptr(d_staging), staging_bytes,
                                depth, _ptr(d_status), _stream(copy_stream), _stream(stream))
    _check(st, "sh_decode_stream")


def raw_status(fn_name: str, *args) -> int:
    """Call a C entry point and return its status without raising (for tests)."""
    return int(getattr(lib(), fn_name)(*args))


# ---- torch conveniences: allocate the buffers, then call the C ABI ---------------------

def encode_tensor(x, table: sh_table, params: Params, stream=None):
    """Encode a device int8 tensor.  Returns (container uint8 tensor, info, status) where
    info and status are still on the device; call ``finish_encode`` to trim and check."""
    import torch
    x = x.contiguous().view(-1)
    n = x.numel()
    cap = sh_encode_bound(n, params)
    wsb = sh_encode_workspace(n, params)
    out = torch.empty(max(cap, 4), dtype=torch.uint8, device=x.device)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=x.device)
    info = torch.zeros(2, dtype=torch.int64, device=x.device)
    status = torch.zeros(1, dtype=torch.int32, device=x.device)
    sh_encode(table, params, x, n, out, cap, ws, wsb, info, status, stream)
    return out, info, status


def finish_encode(out, info, status):
    """Wait for an encode, raise on a device-side error, return (container, payload_bits)."""
    st = int(status.item())
    if st != SH_OK:
        raise ShannonicError(st, "sh_encode (device)")
    nbytes, bits = (int(v) for v in info.tolist())
    return out[:nbytes], bits


def decode_tensor(container, n: int, table: sh_table, params: Params, stream=None):
    """Decode a device container into a new int8 tensor; returns (y, status on device)."""
    import torch
    y = torch.empty(max(n, 1), dtype=torch.int8, device=container.device)
    status = torch.zeros(1, dtype=torch.int32, device=container.device)
    sh_decode(table, params, container, container.numel(), y, n, status, stream)
    return y[:n], status


# ---- batches of tensors with device tables --------------------------------------------

def _round_up(v: int, a: int) -> int:
    return (v + a - 1) // a * a


def build_tables_tensors(xs: list, params: Params, stream=None):
    """Device tables (one uint8 tensor, table i at i * sh_device_table_bytes()) for a list
    of device int8 tensors, built on the GPU."""
    import torch
    dev = xs[0].device
    xs = [x.contiguous().view(-1) for x in xs]
    tables = torch.empty(len(xs) * sh_device_table_bytes(), dtype=torch.uint8, device=dev)
    wsb = sh_build_tables_batch_workspace(len(xs))
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    sh_build_tables_batch(xs, [x.numel() for x in xs], params, tables, ws, wsb, stream)
    return tables, ws


def tables_to_device(tables: list, params: Params, device, stream=None):
    """Upload host tables back to back into one device tensor."""
    import torch
    tb = sh_device_table_bytes()
    d = torch.empty(len(tables) * tb, dtype=torch.uint8, device=device)
    for i, t in enumerate(tables):
        sh_table_to_device(t, params, d[i * tb:], stream)
    return d


def encode_tensors(d_tables, xs: list, params: Params, stream=None, place_stream=None):
    """Encode a list of device int8 tensors with their device tables (place_stream: see
    sh_encode_batch).  Returns (buffer, offsets, caps, info (nseg x 2 int64, device), status
    (device)); container i starts at buffer[offsets[i]]."""
    import torch
    dev = xs[0].device
    xs = [x.contiguous().view(-1) for x in xs]
    ns = [x.numel() for x in xs]
    caps = [max(sh_encode_bound(n, params), 4) for n in ns]
    offs, at = [], 0
    for c in caps:
        offs.append(at)
        at += _round_up(c, 256)
    buf = torch.empty(max(at, 256), dtype=torch.uint8, device=dev)
    wsb = sh_encode_batch_workspace(ns, params)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    info = torch.zeros((len(xs), 2), dtype=torch.int64, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    base = buf.data_ptr()
    sh_encode_batch(d_tables, xs, ns, params, [base + o for o in offs], caps, ws, wsb, info,
                    status, stream, place_stream)
    return buf, offs, caps, info, status


def decode_tensors(d_tables, buf, offs: list, in_nbytes: list, ns: list, params: Params,
                   stream=None):
    """Decode containers buf[offs[i]:] (in_nbytes[i] readable bytes) into one int8 tensor
    holding every output back to back (16-byte aligned starts).  Returns (y, starts,
    status on device)."""
    import torch
    starts, at = [], 0
    for n in ns:
        starts.append(at)
        at += _round_up(n, 256)
    y = torch.empty(max(at, 256), dtype=torch.int8, device=buf.device)
    status = torch.zeros(1, dtype=torch.int32, device=buf.device)
    base, ybase = buf.data_ptr(), y.data_ptr()
    sh_decode_batch(d_tables, [base + o for o in offs], in_nbytes, [ybase + s for s in starts],
                    ns, params, status, stream)
    return y, starts, status
