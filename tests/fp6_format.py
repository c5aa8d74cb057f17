"""Test-side writer/reader of the FP6 container of INT4 codes, written from
the layout documented in include/svdq.h (svdq_qformat): each code c is the
FP6 E2M3 number c/8 (bit 5 the sign, bits 0-2 the magnitude |c|, exponent
field zero: a subnormal of OCP FP6 E2M3); the codes of half h of a 64-code
group are packed least-significant-bit first into 24 bytes H_h (code k at
bits [6(k - 32h), +6)); the group's 48 bytes are
H_0[0:16] | H_1[0:16] | H_0[16:24] | H_1[16:24]. Rows go in blocks of 128
(the last one holds what is left), and inside a block the groups follow one
another, each as [rows of the block][48 bytes].
Independent of the library's own packers."""

import numpy as np

# byte j of H_h -> byte position within the group's 48 bytes
_POS = np.array([[16 * h + j if j < 16 else 32 + 8 * h + (j - 16) for j in range(24)] for h in range(2)])


def fp6_value(bits):
    """Value of one FP6 E2M3 number (exponent bias 1, 2 exponent bits, 3
    mantissa bits, no infinities or NaNs)."""
    s = -1.0 if bits & 0x20 else 1.0
    e = (bits >> 3) & 3
    m = bits & 7
    if e == 0:
        return s * (m / 8.0)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 1)


def _pack_halves(v):
    """v [..., 32] 6-bit values -> [..., 24] bytes, LSB-first."""
    words = np.zeros(v.shape[:-1] + (3,), dtype=np.uint64)
    for i in range(32):
        w, sh = divmod(6 * i, 64)
        words[..., w] |= v[..., i] << np.uint64(sh)
        if sh > 58:
            words[..., w + 1] |= v[..., i] >> np.uint64(64 - sh)
    return words.astype("<u8").view(np.uint8).reshape(v.shape[:-1] + (24,))


def _blocks(rows):
    """(first row, row count) of each 128-row block."""
    return [(b, min(128, rows - b)) for b in range(0, rows, 128)]


def pack_fp6(codes):
    """codes [rows, K] in [-7, 7] -> bytes [rows, 3K/4] (a flat buffer in the
    blocked order, shaped rows x row bytes)."""
    c = np.asarray(codes, dtype=np.int64)
    rows, K = c.shape
    G = K // 64
    v = (np.where(c < 0, 0x20, 0) | np.abs(c)).astype(np.uint64).reshape(rows, G, 2, 32)
    halves = _pack_halves(v)  # [rows, G, 2, 24]
    rowgrp = np.zeros((rows, G, 48), dtype=np.uint8)
    for h in range(2):
        rowgrp[:, :, _POS[h]] = halves[:, :, h, :]
    out = np.zeros(rows * G * 48, dtype=np.uint8)
    for b0, nb in _blocks(rows):
        blk = rowgrp[b0:b0 + nb].transpose(1, 0, 2)  # [G, nb, 48]
        out[b0 * G * 48:(b0 + nb) * G * 48] = blk.reshape(-1)
    return out.reshape(rows, G * 48)


def unpack_fp6(packed, K):
    """bytes [rows, 3K/4] in the blocked order -> codes [rows, K] (values
    decoded as FP6 E2M3 x 8)."""
    p = np.ascontiguousarray(packed, dtype=np.uint8).reshape(-1)
    G = K // 64
    rows = p.size // (G * 48)
    grp = np.zeros((rows, G, 48), dtype=np.uint8)
    for b0, nb in _blocks(rows):
        grp[b0:b0 + nb] = p[b0 * G * 48:(b0 + nb) * G * 48].reshape(G, nb, 48).transpose(1, 0, 2)
    table = np.array([fp6_value(b) * 8.0 for b in range(64)])
    out = np.zeros((rows, G, 64), dtype=np.float64)
    for h in range(2):
        half = np.ascontiguousarray(grp[:, :, _POS[h]])  # [rows, G, 24]
        words = half.view("<u8").reshape(rows, G, 3)
        for i in range(32):
            w, sh = divmod(6 * i, 64)
            f = words[:, :, w] >> np.uint64(sh)
            if sh > 58:
                f = f | (words[:, :, w + 1] << np.uint64(64 - sh))
            out[:, :, 32 * h + i] = table[(f & np.uint64(0x3F)).astype(np.int64)]
    assert np.all(out == np.rint(out)) and np.abs(out).max(initial=0) <= 7
    return out.reshape(rows, K).astype(np.int8)
