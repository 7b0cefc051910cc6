"""MI355X (gfx950) dense Qwen3-style GQA decoder: Python binding of libgqa355.so.

Argument marshalling only: every step of the forward pass runs in the library's HIP kernels.
The functions below carry the C ABI's names (include/gqa.h) and take plain integers for
pointers; ``Model``/``Session`` wrap them for torch callers, whose CUDA (HIP) tensors provide
device memory and whose current stream is passed through. Loading fails loudly if the built
library is missing; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

from ._lib import (  # noqa: F401
    GQA_OK, GQA_E_INVALID, GQA_E_OOM, GQA_E_DEVICE, GQA_E_HIP, GQA_E_RANGE,
    GQA_SCHEME_BF16, GQA_SCHEME_Q8_0, GQA_SCHEME_AFFINE4, GQA_BLOCK_POSITIONS, GQA_MAX_BATCH,
    GQA_T, GqaError, ModelDesc, ModelInfo, lib, lib_path, load,
    gqa_model_create, gqa_model_destroy, gqa_model_get_info, gqa_session_create, gqa_session_destroy,
    gqa_session_reset, gqa_session_position, gqa_session_eval_prefill, gqa_session_eval_decode,
    gqa_session_eval_decode_static,
    gqa_session_eval_batch, gqa_session_eval_n, gqa_session_eval_scored, gqa_session_truncate,
    gqa_session_create_pooled, gqa_session_publish, gqa_session_reused,
    gqa_model_check_device_error, gqa_model_profile, gqa_model_profile_read, GQA_PROF,
    gqa_last_error, gqa_build_info, gqa_device_describe, DeviceDesc, gqa_debug_read_weight,
    gqa_debug_read_q8, gqa_debug_read_affine4, gqa_debug_read_kv, gqa_debug_read_kv_q8, gqa_debug_read_rope,
)
from .api import Model, Session  # noqa: F401
