"""Seeded synthetic inputs shaped like diffusion-transformer linears.

This module only draws inputs; it holds none of the quantized linear's
arithmetic, so both the HIP library's callers and the CPU oracle's callers can
use it without sharing any of the method's code.

The pages measure on real checkpoints (Krea 2 Turbo at 1024x1024, FLUX, a
480p video model) that are not available here; these generators stand in for
their activations and weights:

* activations ~ N(0, 1) with a few seeded outlier channels scaled up -- the
  per-channel outliers that smoothing moves into the weights;
* weights ~ N(0, 0.02), optionally with a few seeded heavy output columns;
* bias ~ N(0, 0.01) (zero for the tiny case).

Every array is drawn in float32 from numpy's PCG64 with a fixed seed, scaled,
then rounded to bfloat16 (nearest-even on the fp32 bit pattern) and returned
both as uint16 bit patterns and as the float32 values those bits hold.
Seeds: X = 1000c, W = 1000c+1, outlier picks = 1000c+2, heavy columns =
1000c+3, bias = 1000c+4 (c = 1..6, the case number below); the MLP pair's
second weight uses 1000c+5 (values), 1000c+7 (heavy columns) and 1000c+8
(bias).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Case:
    name: str
    number: int
    M: int
    K: int
    N: int
    outlier_channels: int
    outlier_gain: float
    heavy_columns: int
    heavy_gain: float
    bias: bool
    rank: int
    kind: str  # "w4a4", "w8a8", "w4a16"


CASES = {
    # tiny W4A4 case: 2 outlier channels x20, rank 16, bias 0
    "tiny": Case("tiny", 1, 64, 256, 256, 2, 20.0, 0, 1.0, False, 16, "w4a4"),
    # INT8 tensorwise: 1% of 3072 channels (31) x10, bias N(0, 0.01)
    "w8a8_attn": Case("w8a8_attn", 2, 4608, 3072, 3072, 31, 10.0, 0, 1.0, True, 0, "w8a8"),
    # attention projection: 4096 image + 512 text tokens, 0.5% channels (15) x20,
    # 8 heavy weight columns x8, rank 32
    "attn_proj": Case("attn_proj", 3, 4608, 3072, 3072, 15, 20.0, 8, 8.0, True, 32, "w4a4"),
    # MLP up-projection 3072 -> 12288 (the headline shape)
    "mlp_up": Case("mlp_up", 4, 4608, 3072, 12288, 15, 20.0, 8, 8.0, True, 32, "w4a4"),
    # video-scale: 32760 tokens (21 latent frames x 30 x 52 patches), 0.5% (26) x20
    "video": Case("video", 5, 32760, 5120, 5120, 26, 20.0, 0, 1.0, True, 32, "w4a4"),
    "video_w8a8": Case("video_w8a8", 5, 32760, 5120, 5120, 26, 20.0, 0, 1.0, True, 0, "w8a8"),
    # adaLN modulation of a 3072-wide DiT block (6 x 3072 shift/scale/gate
    # outputs) on the conditioning vectors of a batch of 2: the W4A16 layer
    "modulation": Case("modulation", 6, 2, 3072, 18432, 0, 1.0, 0, 1.0, True, 0, "w4a16"),
}

# the MLP down-projection 12288 -> 3072 takes GELU of the up-projection's
# output as its input; its weight is drawn here, its input by the caller
MLP_DOWN = Case("mlp_down", 4, 4608, 12288, 3072, 0, 1.0, 8, 8.0, True, 32, "w4a4")


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Nearest-even bfloat16 bit patterns of finite float32 values."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u.astype(np.uint64) + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal(seed: int, shape, std: float) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    out = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def _picks(seed: int, n: int, count: int) -> np.ndarray:
    if count == 0:
        return np.zeros(0, dtype=np.int64)
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.sort(rng.choice(n, size=count, replace=False))


def activations(case: Case, M: int | None = None) -> dict:
    """X [M, K] bf16 with the case's outlier channels (M may be cut short)."""
    M = case.M if M is None else M
    c = case.number
    X = _normal(1000 * c, (case.M, case.K), 1.0)[:M]
    ch = _picks(1000 * c + 2, case.K, case.outlier_channels)
    if ch.size:
        X[:, ch] *= np.float32(case.outlier_gain)
    bits = bf16_bits_from_f32(X)
    return {"bits": bits, "values": f32_from_bf16_bits(bits), "outlier_channels": ch}


def weight(case: Case, seed_offset: int = 1) -> dict:
    """W [K, N] bf16 ~ N(0, 0.02) with the case's heavy output columns."""
    c = case.number
    W = _normal(1000 * c + seed_offset, (case.K, case.N), 0.02)
    cols = _picks(1000 * c + seed_offset + 2, case.N, case.heavy_columns)
    if cols.size:
        W[:, cols] *= np.float32(case.heavy_gain)
    bits = bf16_bits_from_f32(W)
    return {"bits": bits, "values": f32_from_bf16_bits(bits), "heavy_columns": cols}


def bias(case: Case, seed_offset: int = 4) -> dict:
    """bias [N] bf16 ~ N(0, 0.01), or zeros when the case has none."""
    if not case.bias:
        b = np.zeros(case.N, dtype=np.float32)
    else:
        b = _normal(1000 * case.number + seed_offset, (case.N,), 0.01)
    bits = bf16_bits_from_f32(b)
    return {"bits": bits, "values": f32_from_bf16_bits(bits)}


def mlp_down_weight() -> dict:
    return weight(MLP_DOWN, seed_offset=5)


def mlp_down_bias() -> dict:
    return bias(MLP_DOWN, seed_offset=8)


def random_bf16(seed: int, shape, std: float = 1.0) -> dict:
    """Plain N(0, std) bf16 array for edge-case tests."""
    x = _normal(seed, shape, std)
    bits = bf16_bits_from_f32(x)
    return {"bits": bits, "values": f32_from_bf16_bits(bits)}
