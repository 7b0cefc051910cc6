"""Plain CPU oracle of the dense Qwen3-style GQA decoder forward pass.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The HIP library
never calls it, and it shares no code with the library: the only module both
sides use is ``synth`` (seeded inputs, no decoder arithmetic).

It is the definition of the forward pass written out in NumPy FP32 (RoPE angles
in float64 then rounded to FP32), with a NumPy matmul as the only library step.
Sources, cited by page title and section:

* Kipp Model Support, "The registry": dense Qwen3 decoders, BF16 weights, 8 KV
  heads of width 128, vocabulary 151,936, RMS epsilon 1e-6, per-checkpoint
  RoPE theta and embedding tying.
* Kipp Model Support, "Validated results" (qwen3-0.6b-base): K and V are
  stored rounded to BF16 (the storage contract) and that rounding is the only
  intended source of deviation from an FP32 reference.
* Kipp Model Support, "Validated results" (qwen3-8b-base): an untied checkpoint
  binds a separate lm_head.
* Kipp Roadmap, status v0.0.2: paged KV is a per-session 32-position block table
  that must be bitwise equal to the contiguous layout.
* Kipp Model Support, "Quantization (Q8_0)": seven per-layer projections in
  32-weight blocks of an fp16 scale and int8 quants; embedding, lm_head and
  norms stay BF16.
* Kipp Model Support, "Quantization (AFFINE4_GS32)": 32-weight groups of 4-bit
  codes with an fp16 scale and an fp16 bias (5.0 bits per weight), w = scale*q + bias.
* Kipp Reproducing, "Mutation gate": four KV addressing faults (read-block,
  read-slot, rollover, K/V swap), used here as oracle fault modes.
* Kipp Roadmap, status v0.0.2 and v0.0.3: logits of several positions from one
  call, and scoring of several rows (the log-probability of each next id).
* Kipp Model Support, "What the gates check": truncate/resume of a session.

The layer equations themselves (pre-norm blocks, per-head q/k RMSNorm before a
rotate-half RoPE, SwiGLU) are the standard Qwen3 block; the pages name the
family but print no equations. Pins: tests/test_oracle_*.py. Parity pinned
against a library routine (transformers' Qwen3 model) with the BF16 KV rounding
switched off, against brute force, closed forms and invariants; absolute
agreement with trained Qwen3 checkpoints is parity unpinned (no trained weights).
"""
from .model import OracleModel, OracleSession, ContiguousKV, PagedKV, kv_q8_0_roundtrip, nmse, next_token_log_probs, final_logits  # noqa: F401
from .q8_0 import quantize_q8_0, dequantize_q8_0  # noqa: F401
from .affine4 import quantize_affine4, dequantize_affine4  # noqa: F401
