"""Build librtr_attn.so (HIP kernels + C-ABI host layer) in-tree for gfx950.

Compiles every source under csrc/ with hipcc into one shared library next to
this file.  Always recompiles; writes to a temporary name and renames, so a
failed build never leaves a half-written library behind.
"""

import os
import subprocess
import sys
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
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # Packed fp32 VALU ops are kept out of every kernel.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        "-I", os.path.join(ROOT, "include"),
        "-I", os.path.join(HERE, "csrc"),
    ]


def build(verbose=False, extra_flags=(), out_path=LIB_PATH):
    srcs = [os.path.join(HERE, "csrc", s) for s in SOURCES]
    fd, tmp = tempfile.mkstemp(prefix=".librtr_attn.", suffix=".so.tmp", dir=os.path.dirname(out_path))
    os.close(fd)
    cmd = [hipcc()] + flags() + list(extra_flags) + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    try:
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
        if verbose and res.stderr.strip():
            print(res.stderr, file=sys.stderr)
        os.replace(tmp, out_path)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
