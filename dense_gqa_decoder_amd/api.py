"""Thin object wrappers over the C ABI for torch callers (device buffers are torch tensors)."""
from __future__ import annotations

import atexit
import ctypes
import sys
import weakref

import numpy as np

from . import _lib as L

# Objects still alive at interpreter exit are released before the HIP runtime shuts down
# (sessions before their models); __del__ does nothing once the interpreter is finalising.
_live_sessions = weakref.WeakSet()
_live_models = weakref.WeakSet()


@atexit.register
def _release_all():
    for s in list(_live_sessions):
        s.close()
    for m in list(_live_models):
        m.close()


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


class Model:
    """A model on the current HIP device with seeded synthetic weights."""

    def __init__(self, *, n_layers, hidden, n_q_heads, ffn, vocab=151936, tied=True, rope_theta=1e6, rms_eps=1e-6,
                 scheme="bf16", kv_pool_blocks, max_positions, max_round_tokens=0, seed=0, prefill="split",
                 q8_prefill="copy", kv_quant="bf16"):
        self.desc = L.ModelDesc(n_layers, hidden, n_q_heads, 8, 128, ffn, vocab, 1 if tied else 0, rope_theta,
                                rms_eps, L.SCHEMES[scheme],
                                kv_pool_blocks, max_positions, max_round_tokens,
                                {"split": 0, "fp16": 1}[prefill], {"copy": 0, "direct": 1}[q8_prefill],
                                {"bf16": 0, "q8_0": 1}[kv_quant])
        self.vocab, self.hidden, self.n_layers = vocab, hidden, n_layers
        self.handle = None
        self.handle = L.gqa_model_create(self.desc, seed)
        _live_models.add(self)

    @classmethod
    def from_shape(cls, shape, *, seed, scheme="bf16", kv_pool_blocks, max_positions, max_round_tokens=0,
                   prefill="split", q8_prefill="copy", kv_quant="bf16"):
        return cls(n_layers=shape.n_layers, hidden=shape.hidden, n_q_heads=shape.n_q_heads, ffn=shape.ffn,
                   vocab=shape.vocab, tied=shape.tied, rope_theta=shape.rope_theta, rms_eps=shape.rms_eps,
                   scheme=scheme, kv_pool_blocks=kv_pool_blocks, max_positions=max_positions,
                   max_round_tokens=max_round_tokens, seed=seed, prefill=prefill, q8_prefill=q8_prefill,
                   kv_quant=kv_quant)

    def info(self):
        return L.gqa_model_get_info(self.handle)

    def close(self):
        if self.handle:
            for s in list(_live_sessions):
                if s.model is self:
                    s.close()
            L.gqa_model_destroy(self.handle)
            self.handle = None

    def read_weight(self, kind, layer, row0, rows, cols):
        out = np.empty((rows, cols), dtype=np.uint16)
        L.gqa_debug_read_weight(self.handle, L.GQA_T[kind], layer, row0, rows, out.ctypes.data)
        return out

    def read_q8(self, kind, layer, row0, rows, cols):
        q = np.empty((rows, cols), dtype=np.int8)
        s = np.empty((rows, cols // 32), dtype=np.uint16)
        L.gqa_debug_read_q8(self.handle, L.GQA_T[kind], layer, row0, rows, q.ctypes.data, s.ctypes.data)
        return q, s

    def read_affine4(self, kind, layer, row0, rows, cols):
        q = np.empty((rows, cols), dtype=np.uint8)
        s = np.empty((rows, cols // 32), dtype=np.uint16)
        b = np.empty((rows, cols // 32), dtype=np.uint16)
        L.gqa_debug_read_affine4(self.handle, L.GQA_T[kind], layer, row0, rows, q.ctypes.data, s.ctypes.data,
                                 b.ctypes.data)
        return q, s, b

    SCRATCH = {"resid_a": (0, np.float32), "resid_b": (1, np.float32), "part_a": (2, np.float32),
               "part_b": (3, np.float32), "attn_hi": (4, np.float16), "attn_lo": (5, np.float16),
               "mlp_hi": (6, np.float16), "mlp_lo": (7, np.float16), "norm_hi": (8, np.float16),
               "norm_lo": (9, np.float16), "sumsq": (10, np.float32), "qrot": (11, np.float32),
               "qkv": (12, np.float32)}

    def read_scratch(self, name, offset, count):
        which, dt = self.SCRATCH[name]
        out = np.empty(count, dtype=dt)
        L.gqa_debug_read_scratch(self.handle, which, offset, count, out.ctypes.data)
        return out

    def read_rope(self, n):
        c = np.empty((n, 64), dtype=np.float32)
        s = np.empty((n, 64), dtype=np.float32)
        L.gqa_debug_read_rope(self.handle, n, c.ctypes.data, s.ctypes.data)
        return c, s

    def debug_chain_offset(self, offset: int):
        """Test hook: make the decode chain's waits unsatisfiable (offset > 0) or normal (0)."""
        L.gqa_model_debug_chain_offset(self.handle, offset)

    def profile(self, kernel_class: str):
        L.gqa_model_profile(self.handle, L.GQA_PROF[kernel_class])

    def profile_read(self):
        return L.gqa_model_profile_read(self.handle)

    def check_device_error(self, stream=None):
        L.gqa_model_check_device_error(self.handle, _stream(stream))

    def eval_batch(self, sessions, ids, logits, argmax=None, stream=None):
        """ids: host sequence of ints, or an int32 device tensor (ids_on_device)."""
        B = len(sessions)
        arr = (ctypes.c_void_p * B)(*[s.handle for s in sessions])
        if hasattr(ids, "data_ptr"):
            L.gqa_session_eval_batch(ctypes.addressof(arr), B, ids.data_ptr(), 1, _ptr(logits), _ptr(argmax),
                                     _stream(stream))
        else:
            h = np.ascontiguousarray(ids, dtype=np.int32)
            L.gqa_session_eval_batch(ctypes.addressof(arr), B, h.ctypes.data, 0, _ptr(logits), _ptr(argmax),
                                     _stream(stream))

    def __del__(self):
        if sys.is_finalizing():
            return
        try:
            self.close()
        except Exception:
            pass


class Session:
    def __init__(self, model: Model, max_positions: int, block_ids=None, pooled=False):
        """pooled=True: blocks mapped on demand from the model's pool, with prefix sharing
        (gqa_session_create_pooled); block_ids must then be None."""
        self.model = model
        self._ids = None
        ptr = None
        if block_ids is not None:
            if pooled:
                raise ValueError("a pooled session takes no block ids")
            self._ids = np.ascontiguousarray(block_ids, dtype=np.int32)
            ptr = self._ids.ctypes.data
        self.handle = None
        if pooled:
            self.handle = L.gqa_session_create_pooled(model.handle, max_positions)
        else:
            self.handle = L.gqa_session_create(model.handle, max_positions, ptr)
        _live_sessions.add(self)

    @property
    def reused(self):
        """Positions the last prefill took from the prefix cache."""
        return L.gqa_session_reused(self.handle)

    def publish(self):
        L.gqa_session_publish(self.handle)

    @property
    def position(self):
        return L.gqa_session_position(self.handle)

    def reset(self):
        L.gqa_session_reset(self.handle)

    def prefill(self, ids, logits, argmax=None, stream=None):
        """ids: host ints (checked on the host), or an int32 device tensor (checked on the device)."""
        if hasattr(ids, "data_ptr"):
            L.gqa_session_eval_prefill_device(self.handle, ids.data_ptr(), ids.numel(), _ptr(logits), _ptr(argmax),
                                              _stream(stream))
        else:
            h = np.ascontiguousarray(ids, dtype=np.int32)
            L.gqa_session_eval_prefill(self.handle, h.ctypes.data, len(h), _ptr(logits), _ptr(argmax), _stream(stream))

    def eval_n(self, ids, logits, argmax=None, stream=None):
        """Append host ids and write logits [n][vocab] (and argmax [n]) for every new position."""
        h = np.ascontiguousarray(ids, dtype=np.int32)
        L.gqa_session_eval_n(self.handle, h.ctypes.data, len(h), _ptr(logits), _ptr(argmax), _stream(stream))

    def eval_scored(self, ids, scores, stream=None):
        """Append host ids and write scores [n-1]: log p(ids[i+1] | ids[..i], earlier context)."""
        h = np.ascontiguousarray(ids, dtype=np.int32)
        L.gqa_session_eval_scored(self.handle, h.ctypes.data, len(h), _ptr(scores), _stream(stream))

    def truncate(self, pos):
        L.gqa_session_truncate(self.handle, pos)

    def decode(self, token, logits, argmax=None, stream=None):
        """token: a host int, or an int32 device tensor holding the id."""
        if hasattr(token, "data_ptr"):
            L.gqa_session_eval_decode(self.handle, token.data_ptr(), 1, _ptr(logits), _ptr(argmax), _stream(stream))
        else:
            h = np.asarray([token], dtype=np.int32)
            L.gqa_session_eval_decode(self.handle, h.ctypes.data, 0, _ptr(logits), _ptr(argmax), _stream(stream))

    def decode_static(self, token, logits, argmax=None, stream=None):
        """decode() through gqa_session_eval_decode_static: the call's scratch is the library's
        static device array, nothing is allocated."""
        if hasattr(token, "data_ptr"):
            L.gqa_session_eval_decode_static(self.handle, token.data_ptr(), 1, _ptr(logits), _ptr(argmax),
                                             _stream(stream))
        else:
            h = np.asarray([token], dtype=np.int32)
            L.gqa_session_eval_decode_static(self.handle, h.ctypes.data, 0, _ptr(logits), _ptr(argmax),
                                             _stream(stream))

    def read_kv(self, layer, pos0, n):
        k = np.empty((n, 8, 128), dtype=np.uint16)
        v = np.empty((n, 8, 128), dtype=np.uint16)
        L.gqa_debug_read_kv(self.handle, layer, pos0, n, k.ctypes.data, v.ctypes.data)
        return k, v

    def read_kv_q8(self, layer, pos0, n):
        """Q8_0 KV cache: (K codes, K scale bits, V codes, V scale bits), [n, 8, 128] int8 and [n, 8, 4] uint16."""
        kc = np.empty((n, 8, 128), dtype=np.int8)
        vc = np.empty((n, 8, 128), dtype=np.int8)
        ks = np.empty((n, 8, 4), dtype=np.uint16)
        vs = np.empty((n, 8, 4), dtype=np.uint16)
        L.gqa_debug_read_kv_q8(self.handle, layer, pos0, n, kc.ctypes.data, ks.ctypes.data, vc.ctypes.data,
                               vs.ctypes.data)
        return kc, ks, vc, vs

    def close(self):
        if self.handle:
            L.gqa_session_destroy(self.handle)
            self.handle = None

    def __del__(self):
        if sys.is_finalizing():
            return
        try:
            self.close()
        except Exception:
            pass
