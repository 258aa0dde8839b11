"""Build libar.so (the HIP all-reduce library) for gfx950 with hipcc.

The translation units compile in parallel; the result lands next to this
file so it travels with the source tree.
"""

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libar.so")
SOURCES = ("api.hip", "kernels.hip", "rmsnorm.hip", "noalloc.hip", "ceiling.hip")

# -packed-fp32-ops: keep hipcc from fusing float adds into packed-FP32
# instructions.  No fast-math, no denormal flushing: fp32 adds stay IEEE.
HIPFLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile every source and link the library (libar.so next to this file
    unless `out` says otherwise); `defines` are extra -D options."""
    hipcc = _hipcc()
    with tempfile.TemporaryDirectory(prefix="ar_build_") as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, src + ".o")
            cmd = [hipcc, *HIPFLAGS, *[f"-D{d}" for d in defines], "-c", os.path.join(CSRC, src), "-o", obj]
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
            if verbose:
                sys.stderr.write(res.stderr)
            return obj

        with ThreadPoolExecutor(len(SOURCES)) as pool:
            objs = list(pool.map(compile_one, SOURCES))
        tmp_lib = out + ".tmp"
        cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed:\n{res.stderr}")
        os.replace(tmp_lib, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
