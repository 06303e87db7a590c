"""Bit-packing of quantized codes (oracle, test infrastructure only).

The pages give the storage cost (b bits per weight plus 32 bits of scale and
zero-point per group: 4 + 32/G bits per weight, "LLM quantization principles"
§4.2) but not a bit layout.  The layout here is this project's choice and the
device packer follows it: row r is one little-endian bitstream of uint32
words; column c occupies bits [c*b, c*b + b) of that stream, so 3-bit codes
straddle word boundaries; the last word of a row is zero-padded.

Written bit by bit with Python integers so that the layout is checkable by eye.
"""
from __future__ import annotations

import numpy as np


def words_per_row(n: int, bits: int) -> int:
    return (n * bits + 31) // 32


def pack_ref(codes: np.ndarray, bits: int) -> np.ndarray:
    codes = np.asarray(codes).astype(np.int64)
    m, n = codes.shape
    if codes.size and (codes.min() < 0 or codes.max() >= (1 << bits)):
        raise ValueError("code out of range")
    nw = words_per_row(n, bits)
    out = np.zeros((m, nw), dtype=np.uint32)
    for r in range(m):
        stream = 0
        for c in range(n):
            stream |= int(codes[r, c]) << (c * bits)
        for w in range(nw):
            out[r, w] = (stream >> (32 * w)) & 0xFFFFFFFF
    return out


def unpack_ref(packed: np.ndarray, n: int, bits: int) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint32)
    m, nw = packed.shape
    out = np.zeros((m, n), dtype=np.int64)
    mask = (1 << bits) - 1
    for r in range(m):
        stream = 0
        for w in range(nw):
            stream |= int(packed[r, w]) << (32 * w)
        for c in range(n):
            out[r, c] = (stream >> (c * bits)) & mask
    return out
