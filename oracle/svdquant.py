"""Oracle for the SVDQuant W4A4 linear with its 16-bit low-rank branch.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``): only tests, the smoke check
and the bench's CPU-baseline leg may import this module.

What is computed, and where the pages say so
--------------------------------------------
[HF-SVDQ] method paragraph: the main layers run with 4-bit weights and 4-bit
activations; activation outliers are moved into the weights (per-channel
smoothing); the hardest part of each weight matrix is kept in a separate
16-bit low-rank branch; the rest of the weight is quantized to 4 bits.
[KREA-SVDQ] "Решение: INT8 и W4A4": the low-rank branches compensate the
quantization error and need no calibration dataset. [DC-README] "Compiler"
bullet: the weights are stored in a grouped INT4 physical format.

Together:  y = dequant(Q4(X / s) . Q4(R)) + (X / s) . L1 . L2 + bias,
with R = diag(s) W - L1 L2 evaluated on the stored 16-bit factors.

Readings taken where the pages are silent:
  R1  smoothing s_k = a_k^alpha / w_k^(1-alpha), a_k = max_m |X[m,k]|,
      w_k = max_n |W[k,n]|, alpha = 0.5; s_k = 1 when a_k or w_k is 0.
  R2  activation statistics come from the activations being quantized
      (self-calibration); no dataset is involved.
  R3  Sigma is split evenly: L1 = U_r Sigma_r^1/2, L2 = Sigma_r^1/2 V_r^T.
  R4  1/s is folded into the stored down factor: L1s = diag(1/s) U_r Sigma^1/2,
      so the branch reads raw X: (X/s) L1 = X L1s.
  R5  the residual uses the stored bf16 factors: R = diag(s) (W - L1s L2).
  R6  INT4 is symmetric on [-7, 7] with scale = absmax / 7; code -8 unused.
  R7  codes are round-half-to-even of the fp32 quotient value / scale.
  R8  "value / scale" is one IEEE fp32 division (round to nearest even).
  R9  an all-zero group gets scale 0 and codes 0 (no division).
  R10 scales are fp32, one per (group of 64 along K, row) for activations and
      per (group, output column) for weights; stored group-major.
  R11 nibble packing: two's complement, byte j holds k = 2j in its low nibble
      and k = 2j + 1 in its high nibble.
  R12 the low-rank intermediate T = X L1s is rounded to bf16 once, after an
      exact (here fp64) sum; the output sums main + low-rank + bias in fp64
      and is rounded once to fp32 or bf16.

Numerics. Everything is float64 except the points where the method rounds to
fp32 (RN32: IEEE binary32 round-to-nearest-even, numpy's float64->float32
cast) or to bf16 (bf16_round, round-to-nearest-even on 8 significant bits).
Dividing two fp32 numbers in float64 and rounding to fp32 gives the correctly
rounded fp32 quotient (53 >= 2*24 + 2 bits), so RN32(a / b) below is IEEE fp32
division.

Parity status: every public function here is pinned by tests/test_oracle_*.py
(brute force on tiny inputs, the dequantize-then-matmul closed form, the
full-rank identity, on-grid exactness, idempotence, scaling and sign
invariants, Eckart-Young, hand-derived golden files). The accuracy of the
method against the unquantized X W has no printed value on the pages and is
reported, not gated ("parity unpinned" for that comparison only).
"""

from __future__ import annotations

import numpy as np

GROUP = 64
QMAX = 7  # symmetric INT4 grid [-7, 7]  (reading R6)
ALPHA = 0.5

F64 = np.float64


# ----------------------------------------------------------------------------
# rounding points
# ----------------------------------------------------------------------------

def rn32(x):
    """Round float64 values to IEEE binary32, nearest-even (returns float32)."""
    return np.asarray(x, dtype=F64).astype(np.float32)


def bf16_round(x):
    """Round float64 values to bfloat16 (8 significant bits), nearest-even.

    Returned as float64 holding bf16-representable values. A value x = m 2^e
    (0.5 <= |m| < 1) has quantum 2^(e-8) while normal; below bf16's smallest
    normal 2^-126 the quantum is fixed at 2^-133. x / quantum is exact in
    float64, so one np.rint performs the single rounding.
    """
    x = np.asarray(x, dtype=F64)
    out = x.copy()
    nz = np.isfinite(x) & (x != 0.0)
    _, e = np.frexp(x[nz])
    quantum = np.ldexp(1.0, np.maximum(e - 8, -133))
    y = np.rint(x[nz] / quantum) * quantum
    bf16_max = (2.0 - 2.0 ** -7) * 2.0 ** 127
    y = np.where(np.abs(y) > bf16_max, np.copysign(np.inf, y), y)
    out[nz] = y
    return out


def bf16_bits(x):
    """uint16 bit patterns of bf16-representable float values."""
    f = np.asarray(x, dtype=F64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def bf16_from_bits(bits):
    """float64 values of uint16 bf16 bit patterns."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(F64)


# ----------------------------------------------------------------------------
# step 1: smoothing (outliers moved into the weights)   [HF-SVDQ] method
# ----------------------------------------------------------------------------

def channel_absmax(X):
    """a_k = max_m |X[m, k]| -- the activation statistic of reading R2."""
    X = np.asarray(X, dtype=F64)
    if X.shape[0] == 0:
        return np.zeros(X.shape[1], dtype=np.float32)
    return rn32(np.max(np.abs(X), axis=0))


def smoothing_factors(act_absmax, W, alpha=ALPHA):
    """s_k = RN32(a_k^alpha / w_k^(1-alpha)), w_k = max_n |W[k, n]| (R1).

    Dividing X by s and multiplying the weight rows by s leaves X W unchanged
    in exact arithmetic while flattening the activation outlier channels.
    """
    a = np.asarray(act_absmax, dtype=F64)
    w = np.max(np.abs(np.asarray(W, dtype=F64)), axis=1)
    s = np.ones_like(a)
    ok = (a > 0) & (w > 0)
    s[ok] = np.power(a[ok], alpha) / np.power(w[ok], 1.0 - alpha)
    return rn32(s)


# ----------------------------------------------------------------------------
# step 2: 16-bit low-rank branch from the SVD of the smoothed weight
# ----------------------------------------------------------------------------

def smoothed_svd(W, s):
    """Thin SVD of W_hat = diag(s) W in float64 (LAPACK through numpy)."""
    What = np.asarray(s, dtype=F64)[:, None] * np.asarray(W, dtype=F64)
    U, S, Vt = np.linalg.svd(What, full_matrices=False)
    return U, S, Vt


def lowrank_factors(W, s, rank, round_to_bf16=True):
    """L1s = diag(1/s) U_r Sigma_r^1/2  [K, r],  L2 = Sigma_r^1/2 V_r^T  [r, N].

    [HF-SVDQ] method: the hardest part of each weight is a separate 16-bit
    low-rank branch; readings R3 (even split of Sigma) and R4 (1/s folded
    into L1s). With round_to_bf16 the factors are rounded to bf16 once each
    (the "16-bit" of the branch); without it they stay float64, which the
    full-rank identity test uses.
    Returns (L1s, L2, singular_values).
    """
    K, N = np.asarray(W).shape
    if rank < 0 or rank > min(K, N):
        raise ValueError("rank out of range")
    U, S, Vt = smoothed_svd(W, s)
    root = np.sqrt(S[:rank])
    L1s = (U[:, :rank] * root[None, :]) / np.asarray(s, dtype=F64)[:, None]
    L2 = root[:, None] * Vt[:rank, :]
    if round_to_bf16:
        L1s = bf16_round(L1s)
        L2 = bf16_round(L2)
    return L1s, L2, S


# ----------------------------------------------------------------------------
# step 3: the 4-bit residual   (reading R5)
# ----------------------------------------------------------------------------

def lowrank_product(L1s, L2):
    """D = L1s L2, summed over j = 0 .. r-1 in that order, in float64."""
    L1s = np.asarray(L1s, dtype=F64)
    L2 = np.asarray(L2, dtype=F64)
    D = np.zeros((L1s.shape[0], L2.shape[1]), dtype=F64)
    for j in range(L1s.shape[1]):
        D += L1s[:, j:j + 1] * L2[j:j + 1, :]
    return D


def residual(W, s, L1s, L2):
    """R32[k, n] = RN32(s_k * (W[k, n] - D[k, n])): the part of the smoothed
    weight left after the low-rank branch, on the stored factors."""
    D = lowrank_product(L1s, L2)
    W = np.asarray(W, dtype=F64)
    return rn32(np.asarray(s, dtype=F64)[:, None] * (W - D))


# ----------------------------------------------------------------------------
# INT4 group quantization  (readings R6-R11)
# ----------------------------------------------------------------------------

def quantize_int4_rows(V, group=GROUP):
    """Quantize each row of V [rows, K] in groups of `group` along K.

    scale = RN32(absmax / 7); code = clamp(RNE(RN32(v / scale)), -7, 7);
    all-zero group -> scale 0, codes 0. Returns (codes int8 [rows, K],
    scales float32 [rows, K / group]).
    """
    V = np.asarray(V, dtype=np.float32)
    rows, K = V.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    Vg = V.reshape(rows, K // group, group).astype(F64)
    amax = np.max(np.abs(Vg), axis=2) if rows else np.zeros((0, K // group))
    scale = rn32(amax / QMAX)
    scale64 = scale.astype(F64)
    safe = np.where(scale64 > 0, scale64, 1.0)
    quot = rn32(Vg / safe[:, :, None]).astype(F64)
    codes = np.clip(np.rint(quot), -QMAX, QMAX)
    codes = np.where(scale64[:, :, None] > 0, codes, 0.0)
    return codes.reshape(rows, K).astype(np.int8), scale


def quantize_weights(R32, group=GROUP):
    """Weight side: R32 [K, N] quantized per output column n and K-group g.

    Returns codes qw [K, N] int8 and scales sw [K/G, N] float32.
    """
    codes_t, scale_t = quantize_int4_rows(np.asarray(R32, dtype=np.float32).T, group)
    return codes_t.T.copy(), scale_t.T.copy()


def smooth_activations(X, s):
    """X_hat = RN32(X / s_k) per channel (X is bf16, hence exact in fp32)."""
    return rn32(np.asarray(X, dtype=F64) / np.asarray(s, dtype=F64)[None, :])


def quantize_activations(X, s, group=GROUP):
    """Activation side: per (row m, K-group g) INT4 codes of X_hat = X / s.

    Returns codes qx [M, K] int8 and scales sx [K/G, M] float32 (group-major).
    """
    codes, scale = quantize_int4_rows(smooth_activations(X, s), group)
    return codes, scale.T.copy()


def dequantize(codes, scales_gm, group=GROUP):
    """codes [rows, K] and group-major scales [K/G, rows] -> float64 values."""
    c = np.asarray(codes, dtype=F64)
    sc = np.repeat(np.asarray(scales_gm, dtype=F64).T, group, axis=1)
    return c * sc


# ----------------------------------------------------------------------------
# the linear
# ----------------------------------------------------------------------------

def lowrank_down(X, L1s):
    """T = bf16(X L1s): the branch's down-projection on raw X (reading R4),
    one rounding to bf16 after a float64 sum (reading R12)."""
    return bf16_round(np.asarray(X, dtype=F64) @ np.asarray(L1s, dtype=F64))


def group_partials(qx, qw, group=GROUP):
    """P[g, m, n] = sum_{k in g} qx[m, k] qw[k, n], exact.

    The codes are small integers, so the float64 matmul of one group is exact
    (every partial sum is an integer below 2^53); the result is returned as
    int64.
    """
    qx = np.asarray(qx, dtype=F64)
    qw = np.asarray(qw, dtype=F64)
    M, K = qx.shape
    N = qw.shape[1]
    G = K // group
    P = np.empty((G, M, N), dtype=np.int64)
    for g in range(G):
        sl = slice(g * group, (g + 1) * group)
        P[g] = (qx[:, sl] @ qw[sl, :]).astype(np.int64)
    return P


def main_product(qx, sx, qw, sw, group=GROUP):
    """y_main[m, n] = sum_g sx[g, m] sw[g, n] P[g, m, n] in float64."""
    qx = np.asarray(qx, dtype=F64)
    qw = np.asarray(qw, dtype=F64)
    sx = np.asarray(sx, dtype=F64)
    sw = np.asarray(sw, dtype=F64)
    M, K = qx.shape
    N = qw.shape[1]
    y = np.zeros((M, N), dtype=F64)
    for g in range(K // group):
        sl = slice(g * group, (g + 1) * group)
        Pg = qx[:, sl] @ qw[sl, :]
        y += (sx[g][:, None] * sw[g][None, :]) * Pg
    return y


def main_product_dense(qx, sx, qw, sw, group=GROUP):
    """y_main = dequant(qx) @ dequant(qw): the dequantize-then-matmul closed
    form of main_product, one float64 matmul over all of K. Every product
    sx qx sw qw is exact to 2^-53 and the K-term sum carries float64 rounding
    only, so it agrees with main_product to far below fp32 resolution; it is
    what full-size comparisons use (one multithreaded matmul instead of a
    loop of G matmuls and elementwise passes)."""
    Xd = dequantize(qx, sx, group)
    Wd = dequantize(np.asarray(qw).T, sw, group)
    return Xd @ Wd.T


def linear_from_parts(qx, sx, T, qw, sw, L2, bias=None, group=GROUP):
    """y = sum_g sx sw P + T L2 + bias, float64 (before the output rounding)."""
    y = main_product(qx, sx, qw, sw, group)
    if T is not None and np.asarray(T).size and np.asarray(L2).size:
        y += np.asarray(T, dtype=F64) @ np.asarray(L2, dtype=F64)
    if bias is not None:
        y += np.asarray(bias, dtype=F64)[None, :]
    return y


def round_output(y, dtype):
    """Single rounding of the float64 output to 'f32' or 'bf16'."""
    if dtype == "f32":
        return rn32(y).astype(F64)
    if dtype == "bf16":
        return bf16_round(y)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# whole pipeline
# ----------------------------------------------------------------------------

def prepare_from_factors(W, s, L1s, L2, group=GROUP):
    """Residual + weight quantization given smoothing factors and factors."""
    R32 = residual(W, s, L1s, L2)
    qw, sw = quantize_weights(R32, group)
    return {"s": rn32(s), "L1s": np.asarray(L1s, dtype=F64),
            "L2": np.asarray(L2, dtype=F64), "R32": R32, "qw": qw, "sw": sw}


def prepare_weights(W, act_absmax, rank, alpha=ALPHA, group=GROUP):
    """Offline weight preparation: smoothing, low-rank branch, 4-bit residual."""
    s = smoothing_factors(act_absmax, W, alpha)
    L1s, L2, S = lowrank_factors(W, s, rank)
    out = prepare_from_factors(W, s, L1s, L2, group)
    out["sigma"] = S
    return out


def forward(X, prep, bias=None, out_dtype="bf16", group=GROUP):
    """The W4A4 linear on prepared weights. Returns a dict of every stage."""
    qx, sx = quantize_activations(X, prep["s"], group)
    T = lowrank_down(X, prep["L1s"])
    y64 = linear_from_parts(qx, sx, T, prep["qw"], prep["sw"], prep["L2"], bias, group)
    return {"qx": qx, "sx": sx, "T": T, "y64": y64, "y": round_output(y64, out_dtype)}


def forward_dense(X, prep, bias=None, out_dtype="bf16", group=GROUP):
    """forward with the main product in its closed form (main_product_dense);
    the same stages otherwise."""
    qx, sx = quantize_activations(X, prep["s"], group)
    T = lowrank_down(X, prep["L1s"])
    y64 = main_product_dense(qx, sx, prep["qw"], prep["sw"], group)
    if T.size and np.asarray(prep["L2"]).size:
        y64 += T @ np.asarray(prep["L2"], dtype=F64)
    if bias is not None:
        y64 += np.asarray(bias, dtype=F64)[None, :]
    return {"qx": qx, "sx": sx, "T": T, "y64": y64, "y": round_output(y64, out_dtype)}


# ----------------------------------------------------------------------------
# byte layouts of the library boundary (reading R10, R11)
# ----------------------------------------------------------------------------

def pack_int4(codes):
    """codes [rows, K] in [-8, 7] -> bytes [rows, K/2]; low nibble = even k."""
    c = np.asarray(codes, dtype=np.int16)
    if c.shape[1] % 2:
        raise ValueError("K must be even")
    lo = c[:, 0::2] & 0xF
    hi = c[:, 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_int4(packed):
    """bytes [rows, K/2] -> codes [rows, K] int8 (two's complement nibbles)."""
    p = np.asarray(packed, dtype=np.uint8).astype(np.int16)
    lo = p & 0xF
    hi = (p >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.int8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def to_abi(prep):
    """Prepared weights in the library's byte layouts.

    qw  : uint8  [N, K/2]  packed codes, one row per output column
    sw  : fp32   [K/G, N]
    s   : fp32   [K]
    l1t : uint16 [r, K]    bf16 bits of L1s^T (one row per rank component)
    l2t : uint16 [N, r]    bf16 bits of L2^T  (one row per output column)
    """
    return {
        "qw": pack_int4(np.asarray(prep["qw"]).T),
        "sw": np.ascontiguousarray(prep["sw"], dtype=np.float32),
        "s": np.ascontiguousarray(prep["s"], dtype=np.float32),
        "l1t": np.ascontiguousarray(bf16_bits(np.asarray(prep["L1s"]).T)),
        "l2t": np.ascontiguousarray(bf16_bits(np.asarray(prep["L2"]).T)),
    }
