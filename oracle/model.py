"""Forward pass of the dense Qwen3-style GQA decoder, written out plainly (oracle).

Test infrastructure: see the package docstring for who may use it and for the
passages each step follows. Every array is FP32 unless stated; BF16 tensors are
widened exactly to FP32 before use.

Step order per layer (standard Qwen3 block; Kipp Model Support, "The
registry", names the family and its constants):

    a   = RMSNorm(x) * w_attn                      eps 1e-6
    q,k,v = a Wq^T, a Wk^T, a Wv^T                 (nq, 8, 8 heads of 128)
    q_h = RMSNorm_128(q_h) * w_qn ; k_h likewise    per-head q/k norm
    q,k = RoPE(q, p), RoPE(k, p)                   rotate-half pairs (i, i+64)
    K[p], V[p] = bf16(k), bf16(v)                  storage contract (Model Support,
                                                   "Validated results", qwen3-0.6b-base)
    o_h = softmax_j<=p(q_h . K_{h//g}[j] / sqrt(128)) V_{h//g}
    x  += o Wo^T
    b   = RMSNorm(x) * w_ffn
    x  += (silu(b Wg^T) * (b Wu^T)) Wd^T
logits = (RMSNorm(x) * w_final) W_lm^T,  W_lm = embedding when tied.
"""
from __future__ import annotations

import math

import numpy as np

import synth

from .q8_0 import dequantize_q8_0, quantize_q8_0

HEAD_DIM = 128
BLOCK = 32


def nmse(y, ref) -> float:
    """sum((y - ref)^2) / sum(ref^2) over one logit vector, in float64."""
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    return float(np.sum((y - r) ** 2) / np.sum(r ** 2))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round FP32 values to the nearest BF16 (ties to even) and widen back to FP32."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)) << np.uint32(16)
    return r.view(np.float32)


def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * w over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True, dtype=np.float32)
    return (x / np.sqrt(ms + np.float32(eps))) * w


def rope_tables(theta: float, positions: np.ndarray, dim: int = HEAD_DIM):
    """cos/sin of p * theta^(-2i/dim), i < dim/2, evaluated in float64 and rounded to FP32."""
    i = np.arange(dim // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / dim)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE: pairs (x_i, x_{i+64}) rotated by angle phi_i. x: [T, heads, 128]; cos/sin: [T, 64]."""
    half = x.shape[-1] // 2
    x1, x2 = x[..., :half], x[..., half:]
    c, s = cos[:, None, :], sin[:, None, :]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(z: np.ndarray) -> np.ndarray:
    """z / (1 + exp(-z))."""
    with np.errstate(over="ignore"):
        return z / (np.float32(1.0) + np.exp(-z))


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, q_pos: np.ndarray) -> np.ndarray:
    """Causal GQA attention.

    q: [T, nq, d] queries at absolute positions q_pos; K, V: [n, nkv, d] cached keys/values for
    positions 0..n-1. Query head h reads KV head h // (nq // nkv); key j is visible iff j <= q_pos.
    Returns o: [T, nq * d].
    """
    T, nq, d = q.shape
    n, nkv, _ = K.shape
    g = nq // nkv
    scale = np.float32(1.0 / math.sqrt(d))
    o = np.empty((T, nq, d), dtype=np.float32)
    visible = np.arange(n)[None, :] <= np.asarray(q_pos)[:, None]          # [T, n]
    for h in range(nq):
        kv = h // g
        s = (q[:, h, :] @ K[:, kv, :].T) * scale                          # [T, n]
        s = np.where(visible, s, np.float32(-np.inf))
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        l = e.sum(axis=1, keepdims=True, dtype=np.float32)
        o[:, h, :] = (e @ V[:, kv, :]) / l
    return o.reshape(T, nq * d)


class ContiguousKV:
    """K/V cache as one [positions, kv_heads, 128] array per layer (the contiguous layout)."""

    def __init__(self, n_layers: int, max_pos: int, n_kv: int = 8, d: int = HEAD_DIM):
        self.k = np.zeros((n_layers, max_pos, n_kv, d), dtype=np.float32)
        self.v = np.zeros_like(self.k)

    def write(self, layer, positions, k, v):
        self.k[layer, positions] = k
        self.v[layer, positions] = v

    def read(self, layer, n):
        return self.k[layer, :n], self.v[layer, :n]

    @classmethod
    def for_shape(cls, shape, max_pos):
        return cls(shape.n_layers, max_pos, shape.n_kv_heads, shape.head_dim)


class PagedKV:
    """K/V cache in a pool of 32-position blocks addressed through a block table.

    Kipp Roadmap, status v0.0.2: a per-session 32-position block table. Position p lives in
    physical block table[p // 32], slot p % 32. ``fault`` selects one of the four addressing
    defects of Kipp Reproducing, "Mutation gate" (1 read-block, 2 read-slot, 3 rollover,
    4 K/V swap); 0 is the correct cache.
    """

    def __init__(self, n_layers: int, pool_blocks: int, table, n_kv: int = 8, d: int = HEAD_DIM, fault: int = 0):
        self.table = np.asarray(table, dtype=np.int64)
        if len(set(self.table.tolist())) != len(self.table) or self.table.min() < 0 or self.table.max() >= pool_blocks:
            raise ValueError("block table must hold distinct physical block ids inside the pool")
        self.k = np.zeros((n_layers, pool_blocks, n_kv, BLOCK, d), dtype=np.float32)
        self.v = np.zeros_like(self.k)
        self.fault = fault

    def _addr(self, positions):
        p = np.asarray(positions, dtype=np.int64)
        return self.table[p // BLOCK], p % BLOCK

    def write(self, layer, positions, k, v):
        blk, slot = self._addr(positions)
        self.k[layer, blk, :, slot] = k
        self.v[layer, blk, :, slot] = v

    def read(self, layer, n):
        p = np.arange(n, dtype=np.int64)
        logical = p // BLOCK
        slot = p % BLOCK
        blk = self.table[logical]
        if self.fault == 1:            # read-block: physical block taken as the logical index
            blk = logical
        elif self.fault == 2:          # read-slot: neighbouring slot inside the block
            slot = slot ^ 1
        elif self.fault == 3:          # rollover: first slot of a block read from the previous block
            blk = np.where((slot == 0) & (logical > 0), self.table[np.maximum(logical - 1, 0)], blk)
        K = self.k[layer, blk, :, slot]
        V = self.v[layer, blk, :, slot]
        if self.fault == 4:            # K/V swap
            K, V = V, K
        return K, V

    @classmethod
    def for_shape(cls, shape, pool_blocks, table, fault=0):
        return cls(shape.n_layers, pool_blocks, table, shape.n_kv_heads, shape.head_dim, fault)


class OracleModel:
    """Weights of one seeded synthetic model, widened to FP32 (Q8_0 projections dequantised)."""

    PROJ = ("q", "k", "v", "o", "gate", "up", "down")

    def __init__(self, shape: synth.ModelShape, seed: int, scheme: str = "bf16", cache: bool = True):
        if scheme not in ("bf16", "q8_0", "affine4"):
            raise ValueError(scheme)
        self.shape, self.seed, self.scheme, self.cache = shape, seed, scheme, cache
        self._layers = {}
        self.embed = synth.bf16_bits_to_f32(synth.tensor_bits(shape, seed, "embed"))
        self.final_norm = synth.bf16_bits_to_f32(synth.tensor_bits(shape, seed, "final_norm"))
        self.lm_head = self.embed if shape.tied else synth.bf16_bits_to_f32(synth.tensor_bits(shape, seed, "lm_head"))

    def _make_layer(self, l):
        from .q8_0 import quantize_q8_0, dequantize_q8_0
        from .affine4 import quantize_affine4, dequantize_affine4
        out = {}
        for nm in synth.LAYER_TENSORS:
            w = synth.bf16_bits_to_f32(synth.tensor_bits(self.shape, self.seed, nm, l))
            if self.scheme == "q8_0" and nm in self.PROJ:
                w = dequantize_q8_0(*quantize_q8_0(w))
            elif self.scheme == "affine4" and nm in self.PROJ:
                w = dequantize_affine4(*quantize_affine4(w)).astype(np.float32)
            out[nm] = w
        return out

    def layer(self, l):
        if l in self._layers:
            return self._layers[l]
        w = self._make_layer(l)
        if self.cache:
            self._layers[l] = w
        return w


def final_logits(model: OracleModel, x: np.ndarray) -> np.ndarray:
    """logits = (RMSNorm(x) * w_final) W_lm^T for residual rows x [rows, hidden]; W_lm is the
    embedding when tied, the separate lm_head otherwise (Kipp Model Support, "Validated
    results", qwen3-8b-base)."""
    x = np.asarray(x, dtype=np.float32)
    return rmsnorm(x, model.final_norm, model.shape.rms_eps) @ model.lm_head.T


def kv_q8_0_roundtrip(x: np.ndarray) -> np.ndarray:
    """What attention reads back from a Q8_0 KV cache (Kipp Roadmap, status v0.0.4: the opt-in
    Q8_0 KV cache). Each head row of 128 FP32 values is stored as four Q8_0 blocks of 32 (the
    weight format of Model Support, "Quantization (Q8_0)", with its scale and rounding rule);
    reading gives fp32(scale) * q, exact in FP32, which enters attention rounded to BF16, the
    operand format of the BF16 cache (the pages fix no read precision; this is the reading)."""
    x = np.asarray(x, dtype=np.float32)
    scale, q = quantize_q8_0(x.reshape(-1, HEAD_DIM))
    return bf16_round(dequantize_q8_0(scale, q)).reshape(x.shape)


class OracleSession:
    """One sequence: a KV cache and a position counter. kv_quant "bf16" stores K/V as BF16;
    "q8_0" stores them as Q8_0 blocks (kv_q8_0_roundtrip)."""

    def __init__(self, model: OracleModel, kv, kv_round: bool = True, kv_quant: str = "bf16"):
        if kv_quant not in ("bf16", "q8_0"):
            raise ValueError("kv_quant must be bf16 or q8_0")
        self.m, self.kv, self.pos, self.kv_round, self.kv_quant = model, kv, 0, kv_round, kv_quant

    def forward(self, ids, all_logits: bool = False):
        """Append tokens ``ids`` at positions pos.. and return logits of the last (or every) new position."""
        x = self.residual(ids)
        xs = x if all_logits else x[-1:]
        logits = final_logits(self.m, xs)
        return logits if all_logits else logits[0]

    def residual(self, ids):
        """Append tokens ``ids`` at positions pos.. and return the residual stream x [T, hidden]
        of the new positions after the last layer (the input of the final norm)."""
        sh, m = self.m.shape, self.m
        ids = np.asarray(ids, dtype=np.int64)
        if ids.min() < 0 or ids.max() >= sh.vocab:
            raise ValueError("token id out of range")
        T = len(ids)
        positions = np.arange(self.pos, self.pos + T)
        cos, sin = rope_tables(sh.rope_theta, positions, sh.head_dim)
        eps = sh.rms_eps
        x = m.embed[ids]
        for l in range(sh.n_layers):
            w = m.layer(l)
            a = rmsnorm(x, w["attn_norm"], eps)
            q = (a @ w["q"].T).reshape(T, sh.n_q_heads, sh.head_dim)
            k = (a @ w["k"].T).reshape(T, sh.n_kv_heads, sh.head_dim)
            v = (a @ w["v"].T).reshape(T, sh.n_kv_heads, sh.head_dim)
            q = rope(rmsnorm(q, w["q_norm"], eps), cos, sin)
            k = rope(rmsnorm(k, w["k_norm"], eps), cos, sin)
            if self.kv_quant == "q8_0":
                k, v = kv_q8_0_roundtrip(k), kv_q8_0_roundtrip(v)
            elif self.kv_round:
                k, v = bf16_round(k), bf16_round(v)
            self.kv.write(l, positions, k, v)
            K, V = self.kv.read(l, self.pos + T)
            o = attention(q, K, V, positions)
            x = x + o @ w["o"].T
            b = rmsnorm(x, w["ffn_norm"], eps)
            x = x + (silu(b @ w["gate"].T) * (b @ w["up"].T)) @ w["down"].T
        self.pos += T
        return x

    def prefill(self, ids):
        return self.forward(ids)

    def truncate(self, pos: int):
        """Keep the first ``pos`` positions; later KV entries are rewritten when evaluated again
        (Kipp Model Support, "What the gates check": truncate/resume)."""
        if not 0 <= pos <= self.pos:
            raise ValueError("truncate position out of range")
        self.pos = pos

    def score(self, ids):
        """Append ``ids`` (n >= 2) and return the n-1 log-probabilities log p(ids[i+1] | ..ids[i])
        (Kipp Roadmap, status v0.0.3: multi-row scoring)."""
        if len(ids) < 2:
            raise ValueError("scoring needs at least two ids")
        logits = self.forward(ids, all_logits=True)
        return next_token_log_probs(logits[:-1], np.asarray(ids[1:], dtype=np.int64))

    def decode(self, token: int):
        return self.forward([token])


def next_token_log_probs(logits: np.ndarray, targets: np.ndarray) -> np.ndarray:
    """Row i: log softmax(logits[i])[targets[i]] = logits[i, t] - log sum_j exp(logits[i, j]),
    in float64, with the row maximum taken out before exponentiating."""
    z = np.asarray(logits, dtype=np.float64)
    mx = z.max(axis=1, keepdims=True)
    lse = mx[:, 0] + np.log(np.exp(z - mx).sum(axis=1))
    return z[np.arange(len(z)), targets] - lse


def argmax(logits: np.ndarray) -> int:
    """Index of the largest logit; ties go to the lowest index."""
    return int(np.argmax(logits))
