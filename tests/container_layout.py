"""Parse the container layout (version 3) in tests: where each chunk's bytes lie.

Written from the format description in include/shannonic.h: a header of
4 * ceil((32 + 3K - 1) / 4) bytes; the index (u32 goff[G + 1] with G = ceil(n_chunks / 64),
then u16 size[n_chunks], zero-padded to 4 bytes); the payload, chunk after chunk, sizes
counted in units of 2^u bytes (u the smallest that lets the largest possible chunk's size
fit 16 bits); then zero bytes to a multiple of 4.
"""
from __future__ import annotations

import numpy as np


def header_bytes(K: int) -> int:
    return (32 + 3 * K - 1 + 3) // 4 * 4


def unit_bytes(C: int, log2_L: int, S: int) -> int:
    bound_bits = min(S, C) * log2_L + C * (8 + log2_L)
    B = (bound_bits + 7) // 8
    u = 0
    while -(-B // (1 << u)) > 65535:
        u += 1
    return 1 << u


def index_bytes(nch: int) -> int:
    groups = (nch + 63) // 64
    return 4 * (groups + 1) + (2 * nch + 3) // 4 * 4


def payload_at(n: int, K: int, C: int) -> int:
    return header_bytes(K) + index_bytes((n + C - 1) // C)


def chunk_spans(buf: np.ndarray, n: int, K: int, C: int, log2_L: int, S: int = 32):
    """[(start, end)] byte offsets of every chunk, from the payload start, and the payload
    start itself."""
    nch = (n + C - 1) // C
    hb = header_bytes(K)
    groups = (nch + 63) // 64
    raw = np.asarray(buf[hb: hb + index_bytes(nch)], dtype=np.uint8).tobytes()
    goff = np.frombuffer(raw[:4 * (groups + 1)], dtype="<u4")
    sizes = np.frombuffer(raw[4 * (groups + 1): 4 * (groups + 1) + 2 * nch], dtype="<u2")
    unit = unit_bytes(C, log2_L, S)
    spans = []
    at = 0
    for c in range(nch):
        if c % 64 == 0:
            at = int(goff[c // 64])
        size = unit * int(sizes[c])
        spans.append((at, at + size))
        at += size
    return spans, hb + index_bytes(nch)


def chunk_bytes(buf, n: int, K: int, C: int, log2_L: int, c: int, S: int = 32):
    """The bytes of chunk c (its size units, padding included)."""
    spans, pay0 = chunk_spans(buf, n, K, C, log2_L, S)
    a, b = spans[c]
    return np.asarray(buf[pay0 + a: pay0 + b])
