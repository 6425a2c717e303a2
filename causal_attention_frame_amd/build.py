"""Build librtr_attn.so (HIP kernels + C-ABI host layer) in-tree for gfx950.

Compiles every source under csrc/ with hipcc into one shared library next to
this file.  Always recompiles; writes to a temporary name and renames, so a
failed build never leaves a half-written library behind.
"""

import os
import subprocess
import sys
import shutil
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_NAME = "librtr_attn.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["rtr_api.hip", "attn_fwd.hip", "attn_bwd.hip", "kv_copy.hip"]
ARCH = "gfx950"


def hipcc():
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # Packed fp32 VALU ops are kept out of every kernel.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        "-I", os.path.join(ROOT, "include"),
        "-I", os.path.join(HERE, "csrc"),
    ]


# Extra flags per source.  attn_bwd.hip: builtin MFMAs in VGPR form (their
# results feed VALU code); its long-lived accumulators use AGPRs explicitly.
SOURCE_FLAGS = {"attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    if verbose and res.stderr.strip():
        print(res.stderr, file=sys.stderr)


def build(verbose=False, extra_flags=(), out_path=LIB_PATH):
    """Compile every source to an object (with its own extra flags), link them
    into one shared library, and move it into place."""
    tmpdir = tempfile.mkdtemp(prefix=".librtr_build.", dir=os.path.dirname(out_path))
    tmp = os.path.join(tmpdir, LIB_NAME)
    try:
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmpdir, src + ".o")
            _run([hipcc()] + flags() + list(SOURCE_FLAGS.get(src, [])) + list(extra_flags)
                 + ["-c", os.path.join(HERE, "csrc", src), "-o", obj], verbose)
            objs.append(obj)
        _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
        os.replace(tmp, out_path)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
