"""Test-side writer and reader of the W4A16 weight container, written from
the layout stated in include/svdq.h (w4a16_prepare_weights): units of 32
columns (two 16-column tiles) by a pair of K-groups, 2 x 1024 bytes of code
slots followed by 64 fp32 scales; nibble u = q + 8. Independent of the
library's writer, so the two can be compared byte for byte."""

import numpy as np

UNIT = 2304


def _dims(K, N):
    G = K // 64
    return G, (G + 1) // 2, (N + 31) // 32


def _shift(i):
    return 16 + 4 * (i // 2) if i % 2 else 4 * (i // 2)


def pack_w4a16(qw, sw):
    """qw [K, N] codes in -7..7, sw [K/64, N] fp32 -> container bytes."""
    qw = np.asarray(qw, dtype=np.int64)
    sw = np.asarray(sw, dtype=np.float32)
    K, N = qw.shape
    G, P, C = _dims(K, N)
    u = np.full((C * 32, P * 128), 8, dtype=np.uint32)  # [column][k], padded
    u[:N, :K] = (qw + 8).T
    s = np.zeros((C * 32, P * 2), dtype=np.float32)
    s[:N, :G] = sw.T
    out = np.zeros(C * P * UNIT, dtype=np.uint8)
    l = np.arange(64)
    for b in range(C):
        for p in range(P):
            unit = out[(b * P + p) * UNIT:(b * P + p + 1) * UNIT]
            for j in range(2):
                cols = 32 * b + 16 * j + l % 16
                words = np.zeros((64, 4), dtype=np.uint32)
                for d in range(4):
                    kb = 64 * (2 * p + d // 2) + 32 * (d % 2) + 8 * (l // 16)
                    for i in range(8):
                        words[:, d] |= u[cols, kb + i] << np.uint32(_shift(i))
                unit[1024 * j:1024 * (j + 1)] = words.reshape(-1).view(np.uint8)
            sc = np.zeros((16, 2, 2), dtype=np.float32)  # [c, j, e] -> byte 16c + 8j + 4e
            for j in range(2):
                sc[:, j, :] = s[32 * b + 16 * j:32 * b + 16 * j + 16, 2 * p:2 * p + 2]
            unit[2048:] = sc.reshape(-1).view(np.uint8)
    return out


def unpack_w4a16(buf, K, N):
    """Container bytes -> (qw [K, N] int8, sw [K/64, N] fp32)."""
    buf = np.asarray(buf, dtype=np.uint8)
    G, P, C = _dims(K, N)
    q = np.zeros((C * 32, P * 128), dtype=np.int64)
    s = np.zeros((C * 32, P * 2), dtype=np.float32)
    l = np.arange(64)
    for b in range(C):
        for p in range(P):
            unit = buf[(b * P + p) * UNIT:(b * P + p + 1) * UNIT]
            for j in range(2):
                cols = 32 * b + 16 * j + l % 16
                words = unit[1024 * j:1024 * (j + 1)].view(np.uint32).reshape(64, 4)
                for d in range(4):
                    kb = 64 * (2 * p + d // 2) + 32 * (d % 2) + 8 * (l // 16)
                    for i in range(8):
                        q[cols, kb + i] = ((words[:, d] >> np.uint32(_shift(i))) & 0xF).astype(np.int64) - 8
            sc = unit[2048:].view(np.float32).reshape(16, 2, 2)
            for j in range(2):
                s[32 * b + 16 * j:32 * b + 16 * j + 16, 2 * p:2 * p + 2] = sc[:, j, :]
    return q[:N, :K].T.astype(np.int8), np.ascontiguousarray(s[:N, :G].T)
