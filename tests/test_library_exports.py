"""CPU checks of the C ABI: the built library loads and exports every function include/gqa.h
declares, and a call without a GPU fails with an error code instead of falling back."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "gqa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gqa_[a-z0-9_]+)\s*\(", src)))


def test_header_and_binding_agree():
    from dense_gqa_decoder_amd import _lib
    assert sorted(_lib.EXPORTS) == _declared()


def test_library_exports_every_declared_symbol():
    import ctypes
    from dense_gqa_decoder_amd import _lib
    if not os.path.exists(_lib.lib_path):
        pytest.fail("libgqa355.so is not built (run __graft_entry__.build())")
    h = ctypes.CDLL(_lib.lib_path)
    for name in _declared():
        assert hasattr(h, name), name


def test_create_without_gpu_reports_an_error():
    import dense_gqa_decoder_amd as g
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present")
    except ImportError:
        pass
    d = g.ModelDesc(2, 1024, 16, 8, 128, 3072, 151936, 1, 1e6, 1e-6, 0, 8, 64, 0)
    with pytest.raises(g.GqaError) as ei:
        g.gqa_model_create(d, 1)
    assert ei.value.code in (g.GQA_E_HIP, g.GQA_E_DEVICE)
