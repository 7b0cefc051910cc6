"""Q8_0 weight quantisation (oracle side).

Kipp Model Support, "Quantization (Q8_0)": each run of 32 consecutive weights
along the input dimension becomes one block of an fp16 scale plus 32 int8
quants (34 bytes, 8.5 bits per weight). The pages do not spell out the scale
rule; this follows the plain reading: d = max|w| / 127 as an FP32 division,
scale = fp16(d) rounded to nearest even, q = clamp(round_half_away(w / d),
-127, 127) with the FP32 d, and q = 0 for an all-zero block. Dequantised
weight = fp32(scale) * q, which is exact in FP32 (11 x 8 significant bits).
"""
import numpy as np

QK = 32


def quantize_q8_0(w: np.ndarray):
    """w: float32 [rows, cols] with cols % 32 == 0 -> (scale fp16 [rows, cols/32], q int8 [rows, cols])."""
    w = np.asarray(w, dtype=np.float32)
    rows, cols = w.shape
    if cols % QK:
        raise ValueError("row length must be a multiple of 32")
    b = w.reshape(rows, cols // QK, QK)
    amax = np.abs(b).max(axis=2)
    d = (amax / np.float32(127.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = b / d[..., None]                       # FP32 IEEE division
    r = np.where(d[..., None] == 0, np.float32(0), r)
    r64 = r.astype(np.float64)
    q = np.trunc(r64 + np.copysign(0.5, r64))      # round half away from zero, exact in float64
    q = np.clip(q, -127, 127).astype(np.int8)
    return d.astype(np.float16), q.reshape(rows, cols)


def dequantize_q8_0(scale: np.ndarray, q: np.ndarray) -> np.ndarray:
    rows, cols = q.shape
    s = scale.astype(np.float32)[..., None]
    return (s * q.reshape(rows, cols // QK, QK).astype(np.float32)).reshape(rows, cols)
