"""ctypes declarations of include/gqa.h; each wrapper raises GqaError on a negative status."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(HERE, "libgqa355.so")

GQA_OK = 0
GQA_E_INVALID = -1
GQA_E_OOM = -2
GQA_E_DEVICE = -3
GQA_E_HIP = -4
GQA_E_RANGE = -5
GQA_SCHEME_BF16 = 0
GQA_SCHEME_Q8_0 = 1
GQA_SCHEME_AFFINE4 = 2
SCHEMES = {"bf16": GQA_SCHEME_BF16, "q8_0": GQA_SCHEME_Q8_0, "affine4": GQA_SCHEME_AFFINE4}
GQA_MAX_BATCH = 32
GQA_BLOCK_POSITIONS = 32
GQA_T = {"embed": 0, "attn_norm": 1, "q": 2, "k": 3, "v": 4, "q_norm": 5, "k_norm": 6, "o": 7, "ffn_norm": 8,
         "gate": 9, "up": 10, "down": 11, "final_norm": 12, "lm_head": 13}


class GqaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"gqa error {code}: {msg}")
        self.code = code


class ModelDesc(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("tied", ctypes.c_int32), ("rope_theta", ctypes.c_float),
                ("rms_eps", ctypes.c_float), ("scheme", ctypes.c_int32), ("kv_pool_blocks", ctypes.c_int32),
                ("max_positions", ctypes.c_int32), ("max_round_tokens", ctypes.c_int32),
                ("prefill_operands", ctypes.c_int32), ("prefill_q8_direct", ctypes.c_int32),
                ("kv_quant", ctypes.c_int32)]


class ModelInfo(ctypes.Structure):
    _fields_ = [("round_tokens", ctypes.c_int32), ("cu_count", ctypes.c_int32), ("weight_bytes", ctypes.c_int64),
                ("kv_pool_bytes", ctypes.c_int64), ("scratch_bytes", ctypes.c_int64),
                ("prefill_copy_bytes", ctypes.c_int64), ("free_blocks", ctypes.c_int32),
                ("cached_blocks", ctypes.c_int32), ("prefix_lookups", ctypes.c_int64),
                ("prefix_hits", ctypes.c_int64), ("prefix_evictions", ctypes.c_int64)]


class DeviceDesc(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 256), ("arch", ctypes.c_char * 64), ("cu_count", ctypes.c_int32),
                ("clock_khz", ctypes.c_int32), ("memory_clock_khz", ctypes.c_int32),
                ("memory_bus_bits", ctypes.c_int32), ("total_memory", ctypes.c_int64),
                ("l2_bytes", ctypes.c_int64), ("lds_per_cu", ctypes.c_int64), ("runtime_version", ctypes.c_int32),
                ("driver_version", ctypes.c_int32)]


_lib = None
P = ctypes.c_void_p
I32 = ctypes.c_int32

_SIGS = {
    "gqa_model_create": (I32, [ctypes.POINTER(ModelDesc), ctypes.c_uint64, ctypes.POINTER(P)]),
    "gqa_model_destroy": (None, [P]),
    "gqa_model_get_info": (I32, [P, ctypes.POINTER(ModelInfo)]),
    "gqa_session_create": (I32, [P, I32, P, ctypes.POINTER(P)]),
    "gqa_session_destroy": (None, [P]),
    "gqa_session_reset": (I32, [P]),
    "gqa_session_create_pooled": (I32, [P, I32, ctypes.POINTER(P)]),
    "gqa_session_publish": (I32, [P]),
    "gqa_session_reused": (I32, [P]),
    "gqa_session_position": (I32, [P]),
    "gqa_session_eval_prefill": (I32, [P, P, I32, P, P, P]),
    "gqa_session_eval_prefill_device": (I32, [P, P, I32, P, P, P]),
    "gqa_session_eval_n": (I32, [P, P, I32, P, P, P]),
    "gqa_session_eval_scored": (I32, [P, P, I32, P, P]),
    "gqa_session_truncate": (I32, [P, I32]),
    "gqa_session_eval_decode": (I32, [P, P, I32, P, P, P]),
    "gqa_session_eval_batch": (I32, [P, I32, P, I32, P, P, P]),
    "gqa_session_eval_decode_static": (I32, [P, P, I32, P, P, P]),
    "gqa_model_check_device_error": (I32, [P, P]),
    "gqa_model_profile": (I32, [P, I32]),
    "gqa_model_debug_chain_offset": (I32, [P, I32]),
    "gqa_model_profile_read": (I32, [P, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_int64)]),
    "gqa_last_error": (ctypes.c_char_p, []),
    "gqa_build_info": (ctypes.c_char_p, []),
    "gqa_device_describe": (I32, [I32, ctypes.POINTER(DeviceDesc)]),
    "gqa_debug_read_weight": (I32, [P, I32, I32, I32, I32, P]),
    "gqa_debug_read_q8": (I32, [P, I32, I32, I32, I32, P, P]),
    "gqa_debug_read_affine4": (I32, [P, I32, I32, I32, I32, P, P, P]),
    "gqa_debug_read_kv": (I32, [P, I32, I32, I32, P, P]),
    "gqa_debug_read_kv_q8": (I32, [P, I32, I32, I32, P, P, P, P]),
    "gqa_debug_read_rope": (I32, [P, I32, P, P]),
    "gqa_debug_read_scratch": (I32, [P, I32, ctypes.c_int64, ctypes.c_int64, P]),
}
EXPORTS = tuple(_SIGS)


def load(path: str | None = None):
    """Load the built library (no build here: run __graft_entry__.build() or build.py first)."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or lib_path
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: build it with `python dense_gqa_decoder_amd/build.py`")
    h = ctypes.CDLL(p)
    for name, (res, args) in _SIGS.items():
        f = getattr(h, name)
        f.restype = res
        f.argtypes = args
    _lib = h
    return h


def lib():
    return load()


def _check(rc: int):
    if rc < 0:
        raise GqaError(rc, lib().gqa_last_error().decode(errors="replace"))
    return rc


def gqa_last_error() -> str:
    return lib().gqa_last_error().decode(errors="replace")


def gqa_build_info() -> dict:
    import json
    return json.loads(lib().gqa_build_info().decode())


def gqa_device_describe(device: int = 0) -> dict:
    d = DeviceDesc()
    _check(lib().gqa_device_describe(device, ctypes.byref(d)))
    out = {k: getattr(d, k) for k, _ in DeviceDesc._fields_}
    out["name"], out["arch"] = d.name.decode(errors="replace"), d.arch.decode(errors="replace")
    return out


def gqa_model_create(desc: ModelDesc, seed: int) -> int:
    out = P()
    _check(lib().gqa_model_create(ctypes.byref(desc), seed, ctypes.byref(out)))
    return out.value


def gqa_model_destroy(model: int) -> None:
    lib().gqa_model_destroy(model)


def gqa_model_get_info(model: int) -> ModelInfo:
    info = ModelInfo()
    _check(lib().gqa_model_get_info(model, ctypes.byref(info)))
    return info


def gqa_session_create(model: int, max_positions: int, block_ids_ptr: int | None) -> int:
    out = P()
    _check(lib().gqa_session_create(model, max_positions, block_ids_ptr, ctypes.byref(out)))
    return out.value


def gqa_session_destroy(session: int) -> None:
    lib().gqa_session_destroy(session)


def gqa_session_create_pooled(model, max_positions):
    out = P()
    _check(lib().gqa_session_create_pooled(model, max_positions, ctypes.byref(out)))
    return out.value


def gqa_session_publish(session) -> None:
    _check(lib().gqa_session_publish(session))


def gqa_session_reused(session) -> int:
    return lib().gqa_session_reused(session)


def gqa_session_reset(session: int) -> None:
    _check(lib().gqa_session_reset(session))


def gqa_session_position(session: int) -> int:
    return lib().gqa_session_position(session)


def gqa_session_eval_prefill(session, ids_ptr, n, logits_ptr, argmax_ptr, stream) -> None:
    _check(lib().gqa_session_eval_prefill(session, ids_ptr, n, logits_ptr, argmax_ptr, stream))


def gqa_session_eval_prefill_device(session, ids_dev_ptr, n, logits_ptr, argmax_ptr, stream) -> None:
    _check(lib().gqa_session_eval_prefill_device(session, ids_dev_ptr, n, logits_ptr, argmax_ptr, stream))


def gqa_session_eval_n(session, ids_ptr, n, logits_ptr, argmax_ptr, stream) -> None:
    _check(lib().gqa_session_eval_n(session, ids_ptr, n, logits_ptr, argmax_ptr, stream))


def gqa_session_eval_scored(session, ids_ptr, n, scores_ptr, stream) -> None:
    _check(lib().gqa_session_eval_scored(session, ids_ptr, n, scores_ptr, stream))


def gqa_session_truncate(session, pos) -> None:
    _check(lib().gqa_session_truncate(session, pos))


def gqa_session_eval_decode(session, id_ptr, id_on_device, logits_ptr, argmax_ptr, stream) -> None:
    _check(lib().gqa_session_eval_decode(session, id_ptr, id_on_device, logits_ptr, argmax_ptr, stream))


def gqa_session_eval_decode_static(session, id_ptr, id_on_device, logits_ptr, argmax_ptr, stream) -> None:
    _check(lib().gqa_session_eval_decode_static(session, id_ptr, id_on_device, logits_ptr, argmax_ptr, stream))


def gqa_session_eval_batch(sessions_ptr, B, ids_ptr, ids_on_device, logits_ptr, argmax_ptr, stream) -> None:
    _check(lib().gqa_session_eval_batch(sessions_ptr, B, ids_ptr, ids_on_device, logits_ptr, argmax_ptr, stream))


def gqa_model_check_device_error(model, stream) -> None:
    _check(lib().gqa_model_check_device_error(model, stream))


GQA_PROF = {"none": 0, "decode_gateup": 1, "prefill_gateup": 2, "prefill_attn": 3, "decode_lmhead": 4, "rows_lmhead": 5}


def gqa_model_debug_chain_offset(model, offset: int) -> None:
    _check(lib().gqa_model_debug_chain_offset(model, offset))


def gqa_model_profile(model, kernel_class: int) -> None:
    _check(lib().gqa_model_profile(model, kernel_class))


def gqa_model_profile_read(model):
    n = ctypes.c_int64()
    ms = ctypes.c_double()
    dropped = ctypes.c_int64()
    _check(lib().gqa_model_profile_read(model, ctypes.byref(n), ctypes.byref(ms), ctypes.byref(dropped)))
    return n.value, ms.value, dropped.value


def gqa_debug_read_weight(model, kind, layer, row0, rows, dst_ptr) -> None:
    _check(lib().gqa_debug_read_weight(model, kind, layer, row0, rows, dst_ptr))


def gqa_debug_read_affine4(model, kind, layer, row0, rows, q_ptr, s_ptr, b_ptr) -> None:
    _check(lib().gqa_debug_read_affine4(model, kind, layer, row0, rows, q_ptr, s_ptr, b_ptr))


def gqa_debug_read_q8(model, kind, layer, row0, rows, q_ptr, s_ptr) -> None:
    _check(lib().gqa_debug_read_q8(model, kind, layer, row0, rows, q_ptr, s_ptr))


def gqa_debug_read_kv(session, layer, pos0, n, k_ptr, v_ptr) -> None:
    _check(lib().gqa_debug_read_kv(session, layer, pos0, n, k_ptr, v_ptr))


def gqa_debug_read_kv_q8(session, layer, pos0, n, kc_ptr, ks_ptr, vc_ptr, vs_ptr) -> None:
    _check(lib().gqa_debug_read_kv_q8(session, layer, pos0, n, kc_ptr, ks_ptr, vc_ptr, vs_ptr))


def gqa_debug_read_rope(model, n, c_ptr, s_ptr) -> None:
    _check(lib().gqa_debug_read_rope(model, n, c_ptr, s_ptr))


def gqa_debug_read_scratch(model, which, offset, count, dst_ptr) -> None:
    _check(lib().gqa_debug_read_scratch(model, which, offset, count, dst_ptr))
