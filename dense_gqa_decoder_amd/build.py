"""Build libgqa355.so (all HIP kernels + the host runtime) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgqa355.so")
SOURCES = ["k_weights.hip", "k_elementwise.hip", "k_gemm.hip", "k_gemv.hip", "k_gemv_full.hip", "k_attn.hip",
           "runtime.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed FP32 instructions (v_pk_*_f32) anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no implicit multiply-add contraction: every kernel rounds the same expression the same way
    # (explicit fmaf() where a fused multiply-add is intended)
    "-ffp-contract=off",
    # leading scalar and pointer kernel arguments (up to 16) are preloaded into SGPRs by the
    # dispatcher, so a wave's first loads need no kernel-argument load
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
]


def sources_sha256() -> str:
    """Hash of every library source and the C header, in a fixed order (also computed by
    bench.py at run time to tell whether the loaded library was built from the current tree)."""
    import hashlib
    h = hashlib.sha256()
    names = sorted(n for n in os.listdir(CSRC) if n.endswith((".hip", ".h")))
    paths = [os.path.join(CSRC, n) for n in names] + [os.path.join(HERE, "..", "include", "gqa.h")]
    for p in paths:
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode() + b"\0" + f.read())
    return h.hexdigest()


def _git(*args):
    try:
        r = subprocess.run(["git", *args], cwd=HERE, capture_output=True, text=True, timeout=30)
    except (OSError, subprocess.SubprocessError):
        return None
    return r.stdout if r.returncode == 0 else None


def build_info() -> dict:
    """The build record baked into the library (gqa_build_info): commit and dirty state from
    git when it is available (None otherwise), the sources hash, the compiler and the flags."""
    import datetime
    rev = _git("rev-parse", "HEAD")
    st = _git("status", "--porcelain", "--untracked-files=no")
    try:
        v = subprocess.run([HIPCC, "--version"], capture_output=True, text=True, timeout=60).stdout
        hipcc = next((l.strip() for l in v.splitlines() if "version" in l.lower()), v.strip()[:200])
    except (OSError, subprocess.SubprocessError):
        hipcc = None
    return {"commit": rev.strip() if rev else None, "dirty": None if st is None else bool(st.strip()),
            "sources_sha256": sources_sha256(), "hipcc": hipcc, "flags": " ".join(FLAGS),
            "built_utc": datetime.datetime.now(datetime.timezone.utc).strftime("%Y-%m-%dT%H:%M:%SZ")}


def _write_build_info():
    import json
    text = json.dumps(build_info())
    esc = text.replace("\\", "\\\\").replace('"', '\\"')
    with open(os.path.join(CSRC, "_build", "build_info.h"), "w") as f:
        f.write("// written by build.py before every build; not a source file\n")
        f.write('#define GQA_BUILD_INFO "%s"\n' % esc)


def _obj(src: str) -> str:
    return os.path.join(CSRC, "_build", os.path.splitext(src)[0] + ".o")


def build(verbose: bool = False, jobs: int = 6) -> str:
    os.makedirs(os.path.join(CSRC, "_build"), exist_ok=True)
    _write_build_info()
    procs = []
    for src in SOURCES:
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", _obj(src)]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len([p for _, p in procs if p.poll() is None]) >= jobs:
            procs[-jobs][1].wait()
    for src, p in procs:
        out, _ = p.communicate()
        text = "\n".join(l for l in out.decode().splitlines() if "packed-fp32-ops' is not a recognized" not in l)
        if p.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{text}")
        if verbose and text.strip():
            print(text)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *[_obj(s) for s in SOURCES]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
