"""Test-side writer/reader of the FP6 container of INT4 codes, written from
the layout documented in include/svdq.h (svdq_qformat): per group of 64
codes, 48 bytes; code k of the group in bits [6k, 6k+6), least significant
bit first; each code c as FP6 E2M3 of the value c/8 -- bit 5 the sign, bits
0-2 the magnitude |c|, exponent field zero (a subnormal of OCP FP6 E2M3).
Independent of the library's own packers."""

import numpy as np


def fp6_value(bits):
    """Value of one FP6 E2M3 number (exponent bias 1, 2 exponent bits, 3
    mantissa bits, no infinities or NaNs)."""
    s = -1.0 if bits & 0x20 else 1.0
    e = (bits >> 3) & 3
    m = bits & 7
    if e == 0:
        return s * (m / 8.0)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 1)


def pack_fp6(codes):
    """codes [rows, K] in [-7, 7] -> bytes [rows, 3K/4]."""
    c = np.asarray(codes, dtype=np.int64)
    rows, K = c.shape
    G = K // 64
    v = (np.where(c < 0, 0x20, 0) | np.abs(c)).astype(np.uint64).reshape(rows, G, 64)
    words = np.zeros((rows, G, 6), dtype=np.uint64)
    for k in range(64):
        bit = 6 * k
        w, sh = divmod(bit, 64)
        words[:, :, w] |= v[:, :, k] << np.uint64(sh)
        if sh > 58:
            words[:, :, w + 1] |= v[:, :, k] >> np.uint64(64 - sh)
    return words.astype("<u8").view(np.uint8).reshape(rows, G * 48)


def unpack_fp6(packed, K):
    """bytes [rows, 3K/4] -> codes [rows, K] (values decoded as FP6 E2M3 x 8)."""
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    rows = p.shape[0]
    G = K // 64
    words = p.reshape(rows, G, 48).copy().view("<u8").reshape(rows, G, 6)
    table = np.array([fp6_value(b) * 8.0 for b in range(64)])
    out = np.zeros((rows, G, 64), dtype=np.float64)
    for k in range(64):
        bit = 6 * k
        w, sh = divmod(bit, 64)
        f = words[:, :, w] >> np.uint64(sh)
        if sh > 58:
            f = f | (words[:, :, w + 1] << np.uint64(64 - sh))
        out[:, :, k] = table[(f & np.uint64(0x3F)).astype(np.int64)]
    assert np.all(out == np.rint(out)) and np.abs(out).max(initial=0) <= 7
    return out.reshape(rows, K).astype(np.int8)
