"""Compile the HIP library ``liblct.so`` in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblct.so")
ARCH = "gfx950"

# Device code: no packed-fp32 instructions (v_pk_*_f32) anywhere.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def build(verbose: bool = False, save_temps: str | None = None) -> str:
    """Build every source and link liblct.so; returns its path."""
    if save_temps:
        save_temps = os.path.abspath(save_temps)
    with tempfile.TemporaryDirectory(prefix="lct_build_") as tmp:
        objs = []
        for src in ["kernels.hip", "api.cpp", "codebook.cpp"]:
            obj = os.path.join(tmp, src + ".o")
            cmd = [hipcc(), "--offload-arch=" + ARCH] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
            if src.endswith(".hip"):
                cmd += DEVICE_FLAGS
                if save_temps:
                    os.makedirs(save_temps, exist_ok=True)
                    cmd += ["-save-temps=obj"]
                    cmd[cmd.index("-o") + 1] = os.path.join(save_temps, src + ".o")
                    obj = cmd[cmd.index("-o") + 1]
            else:
                cmd = [hipcc()] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.check_call(cmd, cwd=save_temps or tmp)
            objs.append(obj)
        out = LIB + ".tmp%d" % os.getpid()
        cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", out] + objs
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        os.replace(out, LIB)
    return LIB


if __name__ == "__main__":
    import sys
    print(build(verbose=True, save_temps=sys.argv[1] if len(sys.argv) > 1 else None))
