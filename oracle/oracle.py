"""ctypes wrapper of the C oracle -- test infrastructure only.

Every function here calls the plain single-threaded C oracle in
``shannonic_oracle.c``; nothing is computed in Python.  Only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import this module.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

STATUS = {0: "OK", -1: "INVALID", -2: "UNSUPPORTED", -3: "SYMBOL_NOT_IN_TABLE",
          -4: "CORRUPT_STREAM", -5: "BUFFER_TOO_SMALL"}
STAT_NAMES = ["H", "H_P", "D_KL", "sum_Pw", "cl_thm1", "H_p_given_P", "dkl_tans_ref",
              "cl_tans_ref", "payload_bps", "container_bps", "csr", "pct_payload_over_H",
              "pct_container_over_H", "pct_thm1_over_H"]
LG_FRAC = 24

_lib = None


class OracleError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: oracle status {status} ({STATUS.get(status, '?')})")
        self.status = status


def lib():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path):
            _build.build()
        L = C.CDLL(path)
        u8p, u16p, u64p = C.POINTER(C.c_uint8), C.POINTER(C.c_uint16), C.POINTER(C.c_uint64)
        i8p = C.POINTER(C.c_int8)
        L.orc_lg.restype = C.c_uint64
        L.orc_lg.argtypes = [C.c_uint64]
        L.orc_histogram.restype = None
        L.orc_histogram.argtypes = [i8p, C.c_uint64, u64p]
        L.orc_dp.argtypes = [u64p, C.c_int, C.c_int, u16p, u64p]
        L.orc_normalize.argtypes = [u64p, C.c_int, C.c_int, u16p]
        L.orc_build_table.argtypes = [u64p, C.c_int, C.c_int, u16p, u16p]
        L.orc_spread.argtypes = [u16p, C.c_int, C.c_int, u16p]
        L.orc_slot_tables.argtypes = [u16p, C.c_int, C.c_int, u16p, u8p, u16p, u16p]
        L.orc_container_bound.restype = C.c_uint64
        L.orc_container_bound.argtypes = [C.c_uint64, C.c_int, C.c_int, C.c_uint32, C.c_uint32]
        L.orc_encode.argtypes = [i8p, C.c_uint64, C.c_int, C.c_int, u16p, u16p, C.c_uint32,
                                 C.c_uint32, u8p, C.c_uint64, u64p, u64p]
        L.orc_decode.argtypes = [u8p, C.c_uint64, i8p, C.c_uint64]
        L.orc_stats.argtypes = [u64p, C.c_int, C.c_int, u16p, u16p, C.c_uint64, C.c_uint64,
                                C.c_uint64, C.POINTER(C.c_double)]
        L.orc_matvec_i8.argtypes = [i8p, C.c_uint64, C.c_uint32, i8p, C.POINTER(C.c_int32)]
        _lib = L
    return _lib


def _p(a: np.ndarray, t):
    return a.ctypes.data_as(C.POINTER(t))


def _check(st: int, what: str):
    if st != 0:
        raise OracleError(st, what)


def lg(x: int) -> int:
    """Fixed-point log2 with 24 fractional bits (the DP's logarithm)."""
    return int(lib().orc_lg(int(x)))


def histogram(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.int8).reshape(-1)
    h = np.zeros(256, dtype=np.uint64)
    lib().orc_histogram(_p(x, C.c_int8), x.size, _p(h, C.c_uint64))
    return h


def dp(h: np.ndarray, K: int):
    """Optimal split of the alphabet [0, len(h)) into K ranges: (lo[K+1], cost)."""
    h = np.ascontiguousarray(h, dtype=np.uint64)
    lo = np.zeros(K + 1, dtype=np.uint16)
    cost = C.c_uint64(0)
    _check(lib().orc_dp(_p(h, C.c_uint64), h.size, K, _p(lo, C.c_uint16), C.byref(cost)), "dp")
    return lo, int(cost.value)


def normalize(count: np.ndarray, log2_L: int) -> np.ndarray:
    count = np.ascontiguousarray(count, dtype=np.uint64)
    f = np.zeros(count.size, dtype=np.uint16)
    _check(lib().orc_normalize(_p(count, C.c_uint64), count.size, log2_L, _p(f, C.c_uint16)),
           "normalize")
    return f


def build_table(h: np.ndarray, K: int, log2_L: int):
    """Offline step from a 256-bin histogram: (lo[K+1], freq[K])."""
    h = np.ascontiguousarray(h, dtype=np.uint64)
    lo = np.zeros(K + 1, dtype=np.uint16)
    f = np.zeros(K, dtype=np.uint16)
    _check(lib().orc_build_table(_p(h, C.c_uint64), K, log2_L, _p(lo, C.c_uint16),
                                 _p(f, C.c_uint16)), "build_table")
    return lo, f


def spread(freq: np.ndarray, log2_L: int) -> np.ndarray:
    freq = np.ascontiguousarray(freq, dtype=np.uint16)
    out = np.zeros(1 << log2_L, dtype=np.uint16)
    _check(lib().orc_spread(_p(freq, C.c_uint16), freq.size, log2_L, _p(out, C.c_uint16)),
           "spread")
    return out


def slot_tables(freq: np.ndarray, log2_L: int):
    """(slot_range, slot_nb, slot_next, enc_slot), each of length L."""
    freq = np.ascontiguousarray(freq, dtype=np.uint16)
    L = 1 << log2_L
    rng = np.zeros(L, dtype=np.uint16)
    nb = np.zeros(L, dtype=np.uint8)
    nxt = np.zeros(L, dtype=np.uint16)
    enc = np.zeros(L, dtype=np.uint16)
    _check(lib().orc_slot_tables(_p(freq, C.c_uint16), freq.size, log2_L, _p(rng, C.c_uint16),
                                 _p(nb, C.c_uint8), _p(nxt, C.c_uint16), _p(enc, C.c_uint16)),
           "slot_tables")
    return rng, nb, nxt, enc


def container_bound(n: int, K: int, log2_L: int, chunk: int, streams: int) -> int:
    return int(lib().orc_container_bound(n, K, log2_L, chunk, streams))


def encode_status(x: np.ndarray, lo: np.ndarray, freq: np.ndarray, log2_L: int, chunk: int,
                  streams: int):
    """(status, container bytes or None, summed field bits)."""
    x = np.ascontiguousarray(x, dtype=np.int8).reshape(-1)
    lo = np.ascontiguousarray(lo, dtype=np.uint16)
    freq = np.ascontiguousarray(freq, dtype=np.uint16)
    K = freq.size
    cap = container_bound(x.size, K, log2_L, chunk, streams)
    out = np.zeros(max(cap, 1), dtype=np.uint8)
    nbytes = C.c_uint64(0)
    bits = C.c_uint64(0)
    st = lib().orc_encode(_p(x, C.c_int8), x.size, K, log2_L, _p(lo, C.c_uint16),
                          _p(freq, C.c_uint16), chunk, streams, _p(out, C.c_uint8), cap,
                          C.byref(nbytes), C.byref(bits))
    if st != 0:
        return st, None, 0
    return 0, out[: nbytes.value].copy(), int(bits.value)


def encode(x: np.ndarray, lo: np.ndarray, freq: np.ndarray, log2_L: int, chunk: int,
           streams: int):
    """Container bytes (numpy uint8) and the summed field bits."""
    st, out, bits = encode_status(x, lo, freq, log2_L, chunk, streams)
    _check(st, "encode")
    return out, bits


def decode(buf: np.ndarray, n: int, raise_on_error: bool = True):
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    y = np.zeros(max(n, 1), dtype=np.int8)
    st = lib().orc_decode(_p(buf, C.c_uint8), buf.size, _p(y, C.c_int8), n)
    if raise_on_error:
        _check(st, "decode")
        return y[:n]
    return st, y[:n]


def matvec_i8(w: np.ndarray, cols: int, a: np.ndarray, y=None) -> np.ndarray:
    """y + W a for the int8 matrix w (rows of cols values, row-major) and int8 vector a,
    int32 wrapping; y defaults to zeros."""
    w = np.ascontiguousarray(w, dtype=np.int8).reshape(-1)
    a = np.ascontiguousarray(a, dtype=np.int8).reshape(-1)
    rows = w.size // cols if cols else 0
    y = np.zeros(max(rows, 1), dtype=np.int32) if y is None else np.array(y, dtype=np.int32)
    _check(lib().orc_matvec_i8(_p(w, C.c_int8), w.size, cols, _p(a, C.c_int8),
                               _p(y, C.c_int32)), "matvec_i8")
    return y[:rows]


def decode_matvec(buf: np.ndarray, n: int, cols: int, a: np.ndarray, y=None) -> np.ndarray:
    """The fused decode's result: y + W a for the matrix W that the container holds."""
    return matvec_i8(decode(buf, n), cols, a, y)


def stats(h: np.ndarray, lo: np.ndarray, freq: np.ndarray, log2_L: int, payload_bits: int,
          container_bytes: int, n: int) -> dict:
    h = np.ascontiguousarray(h, dtype=np.uint64)
    lo = np.ascontiguousarray(lo, dtype=np.uint16)
    freq = np.ascontiguousarray(freq, dtype=np.uint16)
    out = np.zeros(len(STAT_NAMES), dtype=np.float64)
    _check(lib().orc_stats(_p(h, C.c_uint64), freq.size, log2_L, _p(lo, C.c_uint16),
                           _p(freq, C.c_uint16), payload_bits, container_bytes, n,
                           _p(out, C.c_double)), "stats")
    return dict(zip(STAT_NAMES, out.tolist()))


def roundtrip(x: np.ndarray, K: int, log2_L: int, chunk: int, streams: int) -> dict:
    """Build the table from x itself, encode, decode; everything the tests look at."""
    x = np.ascontiguousarray(x, dtype=np.int8).reshape(-1)
    h = histogram(x)
    lo, f = build_table(h, K, log2_L)
    buf, bits = encode(x, lo, f, log2_L, chunk, streams)
    y = decode(buf, x.size)
    st = stats(h, lo, f, log2_L, bits, buf.size, x.size)
    return dict(h=h, lo=lo, freq=f, buf=buf, payload_bits=bits, y=y, stats=st)
