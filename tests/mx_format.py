"""Test-side writer and reader of the MXFP4 containers, written from the
layout stated in include/svdq.h (svdq_mx_prepare_residual): codes of `rows`
rows in blocks of 128 (n_b rows in the last), block b at byte 128 b K/2,
group g (64 k) of the block at + g n_b 32, half h (k-block 2g + h) at
+ h n_b 16, row r of the block at + 16 r; 32 E2M1 codes per 16 bytes, code i
in bits [4i, 4i + 4) (byte i / 2, low nibble for even i). Scales: E8M0 bytes
[K/32][ld], ld = rows rounded up to a multiple of 16."""

import numpy as np


def scale_ld(rows):
    return (rows + 15) // 16 * 16


def _offsets(rows, K):
    """Byte offset of (row, k-block) 16-byte pieces: [rows, K/32]."""
    off = np.zeros((rows, K // 32), dtype=np.int64)
    for r in range(rows):
        b0 = r // 128 * 128
        nb = min(128, rows - b0)
        for kb in range(K // 32):
            off[r, kb] = b0 * (K // 2) + (kb // 2) * nb * 32 + (kb % 2) * nb * 16 + (r - b0) * 16
    return off


def pack_mx_codes(codes):
    """codes [rows, K] (uint8, 0..15) -> container bytes [rows, K/2]."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, K = codes.shape
    out = np.zeros(rows * K // 2, dtype=np.uint8)
    off = _offsets(rows, K)
    for r in range(rows):
        for kb in range(K // 32):
            c = codes[r, 32 * kb:32 * kb + 32]
            out[off[r, kb]:off[r, kb] + 16] = c[0::2] | (c[1::2] << 4)
    return out.reshape(rows, K // 2)


def unpack_mx_codes(buf, K):
    buf = np.asarray(buf, dtype=np.uint8).reshape(-1)
    rows = buf.size // (K // 2)
    codes = np.zeros((rows, K), dtype=np.uint8)
    off = _offsets(rows, K)
    for r in range(rows):
        for kb in range(K // 32):
            piece = buf[off[r, kb]:off[r, kb] + 16]
            codes[r, 32 * kb:32 * kb + 32:2] = piece & 0xF
            codes[r, 32 * kb + 1:32 * kb + 32:2] = piece >> 4
    return codes


def pack_mx_scales(e):
    """exponents [rows, K/32] -> E8M0 bytes [K/32, ld] (padding 0)."""
    e = np.asarray(e, dtype=np.int64)
    rows, nb = e.shape
    out = np.zeros((nb, scale_ld(rows)), dtype=np.uint8)
    out[:, :rows] = (e + 127).T
    return out


def unpack_mx_scales(u, rows):
    return np.asarray(u, dtype=np.int64)[:, :rows].T - 127
