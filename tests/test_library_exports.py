"""CPU checks of the C ABI: the built library loads and exports every function include/gqa.h
declares, the Python mirrors of its structs have the header's layout, and a call without a GPU
fails with an error code instead of falling back."""
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


def test_struct_layouts_match_the_header(tmp_path):
    """The ctypes mirrors of gqa_model_desc, gqa_model_info and gqa_device_desc have the header's field offsets and
    sizes (compiled from include/gqa.h with the host C compiler)."""
    import ctypes
    import shutil
    import subprocess
    from dense_gqa_decoder_amd import _lib
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    structs = {"gqa_model_desc": _lib.ModelDesc, "gqa_model_info": _lib.ModelInfo, "gqa_device_desc": _lib.DeviceDesc}
    body = ""
    for cname, py in structs.items():
        body += '  printf("%s size %%zu\\n", sizeof(%s));\n' % (cname, cname)
        for fname, _ in py._fields_:
            body += '  printf("%s %s %%zu\\n", offsetof(%s, %s));\n' % (cname, fname, cname, fname)
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include "%s"\nint main(void) {\n%s  return 0;\n}\n'
                   % (os.path.join(ROOT, "include", "gqa.h"), body))
    exe = tmp_path / "layout"
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    r = subprocess.run([cc, "-std=c11", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
                        str(src), "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    got = {}
    for line in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.splitlines():
        parts = line.split()
        got[tuple(parts[:-1])] = int(parts[-1])
    for cname, py in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for fname, _ in py._fields_:
            assert got[(cname, fname)] == getattr(py, fname).offset, (cname, fname)


def test_build_info_is_baked_into_the_library():
    """The build record (commit, dirty state, sources hash, compiler) is a JSON object compiled
    into the library, and its sources hash is that of the current sources (the library in the
    tree was built from them)."""
    import dense_gqa_decoder_amd as g
    from dense_gqa_decoder_amd import build
    info = g.gqa_build_info()
    assert set(info) >= {"commit", "dirty", "sources_sha256", "hipcc", "flags", "built_utc"}
    assert info["sources_sha256"] == build.sources_sha256()
