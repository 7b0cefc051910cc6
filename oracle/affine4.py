"""AFFINE4_GS32 weight quantisation (oracle side).

Kipp Model Support, "Quantization (AFFINE4_GS32)": a private 4-bit affine format with groups
of 32 weights, each group 16 bytes of packed 4-bit codes plus an fp16 scale and an fp16 bias
(5.0 bits per weight), a lossy Q4-class format checked against a per-vector tolerance. The
pages fix the group size, the field widths and the affine form w = scale * q + bias; the
rounding rules are not printed, so this takes the plain reading of an asymmetric min/max
quantiser, per run of 32 consecutive weights along the input dimension:

    v      = the group's weights (BF16 values, exact in FP32)
    d      = (max v - min v) / 15                    FP32 subtraction and division
    scale  = fp16(d), bias = fp16(min v)             round to nearest even
    q      = clamp(round_half_away((v - fp32(bias)) / fp32(scale)), 0, 15)
                                                     FP32 subtraction and division; q = 0 when
                                                     scale == 0
    w      = scale * q + bias                        exact (float64)

The nibble packing is the library's storage detail; codes are compared one per weight.
"""
import numpy as np

GS = 32


def quantize_affine4(w: np.ndarray):
    """w: float32 [rows, cols], cols % 32 == 0 -> (scale fp16 [rows, cols/32],
    bias fp16 [rows, cols/32], q uint8 [rows, cols] in 0..15)."""
    w = np.asarray(w, dtype=np.float32)
    rows, cols = w.shape
    if cols % GS:
        raise ValueError("row length must be a multiple of 32")
    g = w.reshape(rows, cols // GS, GS)
    mn = g.min(axis=2)
    mx = g.max(axis=2)
    d = ((mx - mn) / np.float32(15.0)).astype(np.float32)            # FP32 IEEE operations
    scale = d.astype(np.float16)
    bias = mn.astype(np.float16)
    s32 = scale.astype(np.float32)[..., None]
    b32 = bias.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = (g - b32) / s32                                           # FP32 subtraction, division
    r = np.where(s32 == 0, np.float32(0), r)
    r64 = r.astype(np.float64)
    q = np.trunc(r64 + np.copysign(0.5, r64))                        # round half away from zero
    q = np.clip(q, 0, 15).astype(np.uint8)
    return scale, bias, q.reshape(rows, cols)


def dequantize_affine4(scale: np.ndarray, bias: np.ndarray, q: np.ndarray) -> np.ndarray:
    """float64 [rows, cols]: scale * q + bias per group, exact."""
    rows, cols = q.shape
    s = scale.astype(np.float64)[..., None]
    b = bias.astype(np.float64)[..., None]
    return (s * q.reshape(rows, cols // GS, GS).astype(np.float64) + b).reshape(rows, cols)
