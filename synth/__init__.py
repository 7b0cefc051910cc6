"""Seeded synthetic workload generator shared by the tests, the bench and the oracle.

This module produces inputs only: model shapes, BF16 weight values, token ids,
block tables and context lengths. It holds none of the decoder's arithmetic.

Randomness is counter based. ``h(key, i)`` is the (i+1)-th output of a
SplitMix64 stream seeded with ``key`` (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014; constants of Vigna's public
``splitmix64.c``): the state after i+1 steps is ``key + (i+1)*GAMMA`` and the
output is the finaliser of that state. The HIP library implements the same
definition on the device for its weight generator; the two implementations
share no code.

Weight values ("BF16 weights ~N(0, 0.02)"): for element i (row-major index of the
logical ``[out][in]`` matrix) of tensor t, u = h(key_t, i) with
key_t = h(seed, t); S = sum of the four 16-bit fields of u (Irwin-Hall of order
4, exact integer); z = S - 131070; w = bf16_rne(fp32(z) * WEIGHT_SCALE), where
WEIGHT_SCALE = fp32(0.02 / std(S)). The FP32 product is one correctly rounded
IEEE multiply, so every implementation that follows this definition produces
identical bytes. Norm weights are exactly 1.0.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

M64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB

#: std of the sum of four independent uniform 16-bit integers: sqrt(4 * (65536^2 - 1) / 12)
IH4_STD = math.sqrt(4.0 * (65536.0 ** 2 - 1.0) / 12.0)
IH4_CENTER = 2 * 65535
WEIGHT_STD = 0.02
WEIGHT_SCALE = np.float32(WEIGHT_STD / IH4_STD)

VOCAB = 151936
KV_HEADS = 8
HEAD_DIM = 128
BLOCK = 32  # positions per KV block

# tensor kinds within a layer, in generator id order
LAYER_TENSORS = ("attn_norm", "q", "k", "v", "q_norm", "k_norm", "o", "ffn_norm", "gate", "up", "down")
NORM_TENSORS = ("attn_norm", "q_norm", "k_norm", "ffn_norm")


def fmix64(z: int) -> int:
    """SplitMix64 output finaliser on a Python int (mod 2^64)."""
    z &= M64
    z = ((z ^ (z >> 30)) * MIX1) & M64
    z = ((z ^ (z >> 27)) * MIX2) & M64
    return z ^ (z >> 31)


def h(key: int, i: int) -> int:
    """(i+1)-th output of a SplitMix64 stream seeded with ``key``."""
    return fmix64((key + (i + 1) * GAMMA) & M64)


def h_array(key: int, start: int, n: int) -> np.ndarray:
    """h(key, start .. start+n-1) as a uint64 array."""
    with np.errstate(over="ignore"):
        c = np.arange(start + 1, start + n + 1, dtype=np.uint64)
        z = c * np.uint64(GAMMA) + np.uint64(key & M64)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(MIX1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(MIX2)
        z ^= z >> np.uint64(31)
    return z


def _fp32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    b = x.view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _weight_chunk(key: int, start: int, n: int) -> np.ndarray:
    u = h_array(key, start, n)
    m = np.uint64(0xFFFF)
    s = (u & m) + ((u >> np.uint64(16)) & m) + ((u >> np.uint64(32)) & m) + (u >> np.uint64(48))
    z = (s.astype(np.int64) - IH4_CENTER).astype(np.float32)
    return _fp32_to_bf16_bits(z * WEIGHT_SCALE)


_POOL = None


def _pool() -> ThreadPoolExecutor:
    global _POOL
    if _POOL is None:
        n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
        _POOL = ThreadPoolExecutor(max_workers=max(1, min(n, 16)))
    return _POOL


def weight_bits(key: int, shape) -> np.ndarray:
    """BF16 bit patterns (uint16) of a generated tensor with the given logical shape."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    chunk = 1 << 22
    starts = list(range(0, n, chunk))

    def work(s):
        e = min(n, s + chunk)
        out[s:e] = _weight_chunk(key, s, e - s)

    list(_pool().map(work, starts))
    return out.reshape(shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass(frozen=True)
class ModelShape:
    """Shape of a dense Qwen3-style GQA decoder."""
    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    ffn: int
    tied: bool = True
    vocab: int = VOCAB
    n_kv_heads: int = KV_HEADS
    head_dim: int = HEAD_DIM
    rope_theta: float = 1.0e6
    rms_eps: float = 1.0e-6

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def layer_tensor_shapes(self):
        H, Q, KV, F, D = self.hidden, self.q_dim, self.kv_dim, self.ffn, self.head_dim
        return {
            "attn_norm": (H,), "q": (Q, H), "k": (KV, H), "v": (KV, H), "q_norm": (D,), "k_norm": (D,),
            "o": (H, Q), "ffn_norm": (H,), "gate": (F, H), "up": (F, H), "down": (H, F),
        }

    def tensor_ids(self):
        """(name, layer, generator tensor id) in generator order."""
        out = [("embed", -1, 0)]
        for l in range(self.n_layers):
            for j, nm in enumerate(LAYER_TENSORS):
                out.append((nm, l, 1 + l * len(LAYER_TENSORS) + j))
        base = 1 + self.n_layers * len(LAYER_TENSORS)
        out.append(("final_norm", -1, base))
        if not self.tied:
            out.append(("lm_head", -1, base + 1))
        return out

    def tensor_id(self, name: str, layer: int = -1) -> int:
        if name == "embed":
            return 0
        base = 1 + self.n_layers * len(LAYER_TENSORS)
        if name == "final_norm":
            return base
        if name == "lm_head":
            if self.tied:
                raise ValueError("tied model has no separate lm_head")
            return base + 1
        return 1 + layer * len(LAYER_TENSORS) + LAYER_TENSORS.index(name)


# The five workloads: a tiny 2-layer decoder and the Qwen3 0.6B, 4B and 8B shapes.
TINY = ModelShape("tiny-2l-1024", 2, 1024, 16, 3072)
Q06B = ModelShape("qwen3-0.6b-shape", 28, 1024, 16, 3072)
Q4B = ModelShape("qwen3-4b-shape", 36, 2560, 32, 9728)
Q8B = ModelShape("qwen3-8b-shape", 36, 4096, 32, 12288, tied=False)
SHAPES = {s.name: s for s in (TINY, Q06B, Q4B, Q8B)}


def weight_key(seed: int, tensor_id: int) -> int:
    return h(seed, tensor_id)


def tensor_bits(shape: ModelShape, seed: int, name: str, layer: int = -1) -> np.ndarray:
    """BF16 bits of one logical tensor. Norm weights are exactly 1.0 (0x3F80)."""
    if name in NORM_TENSORS or name == "final_norm":
        n = shape.hidden if name in ("attn_norm", "ffn_norm", "final_norm") else shape.head_dim
        return np.full(n, 0x3F80, dtype=np.uint16)
    if name in ("embed", "lm_head"):
        dims = (shape.vocab, shape.hidden)
    else:
        dims = shape.layer_tensor_shapes()[name]
    return weight_bits(weight_key(seed, shape.tensor_id(name, layer)), dims)


def token_ids(seed: int, n: int, vocab: int = VOCAB, offset: int = 0) -> np.ndarray:
    """n uniform token ids in [0, vocab): floor(hi32(h) * vocab / 2^32)."""
    u = h_array(seed, offset, n)
    return ((u >> np.uint64(32)) * np.uint64(vocab) >> np.uint64(32)).astype(np.int32)


def uniform_int(seed: int, i: int, lo: int, hi: int) -> int:
    """Uniform integer in [lo, hi] from h(seed, i)."""
    return lo + (((h(seed, i) >> 32) * (hi - lo + 1)) >> 32)


def shuffled_blocks(seed: int, pool_blocks: int) -> np.ndarray:
    """A Fisher-Yates permutation of range(pool_blocks) driven by h(seed, .)."""
    p = list(range(pool_blocks))
    for i in range(pool_blocks - 1, 0, -1):
        j = ((h(seed, i) >> 32) * (i + 1)) >> 32
        p[i], p[j] = p[j], p[i]
    return np.asarray(p, dtype=np.int32)


def context_lengths(seed: int, n: int, lo: int = 512, hi: int = 8192) -> np.ndarray:
    return np.asarray([uniform_int(seed, i, lo, hi) for i in range(n)], dtype=np.int32)


def blocks_for(positions: int) -> int:
    return (positions + BLOCK - 1) // BLOCK


@dataclass(frozen=True)
class Workload:
    """One of the five measured workloads (seeds: weights 1000+k, ids 2000+k, shuffle 3000+k)."""
    key: str
    shape: ModelShape
    scheme: str            # "bf16" or "q8_0"
    prompt: int            # prompt tokens (per sequence)
    decode: int            # decode steps (per sequence)
    paged: str             # "identity" or "shuffled"
    n_seqs: int = 1
    k: int = 1
    kv_quant: str = "bf16"  # KV cache format: "bf16" or "q8_0"

    @property
    def weight_seed(self) -> int:
        return 1000 + self.k

    @property
    def ids_seed(self) -> int:
        return 2000 + self.k

    @property
    def shuffle_seed(self) -> int:
        return 3000 + self.k


WORKLOADS = {
    "tiny": Workload("tiny", TINY, "bf16", 16, 16, "identity", k=1),
    "0.6b": Workload("0.6b", Q06B, "bf16", 348, 64, "shuffled", k=2),
    "4b": Workload("4b", Q4B, "bf16", 2048, 64, "shuffled", k=3),
    "4b-q8": Workload("4b-q8", Q4B, "q8_0", 12800, 32, "shuffled", k=4),
    "4b-a4": Workload("4b-a4", Q4B, "affine4", 2048, 64, "shuffled", k=6),
    "4b-kvq8": Workload("4b-kvq8", Q4B, "bf16", 2048, 64, "shuffled", k=7, kv_quant="q8_0"),
    "8b-batch": Workload("8b-batch", Q8B, "bf16", 0, 128, "shuffled", n_seqs=32, k=5),
}

CONTEXT_SEED_8B = 4005


def reduced(shape: ModelShape, **kw) -> ModelShape:
    return replace(shape, **kw)
