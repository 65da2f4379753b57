"""Build the gfx950 library libphx_expert.so in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libphx_expert.so")
SOURCES = ["phx_kernels.hip", "phx_decide.hip", "phx_tokens.hip", "phx_engine.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-FP32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-result",
]
# per-source flags: the large-token kernels keep MFMA accumulators in ordinary
# VGPRs (their register budget fits), so the softmax and the rescales read
# them without accumulator-register copies
EXTRA = {"phx_tokens.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _clean(stderr: str) -> str:
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    return "\n".join(l for l in stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel) and link libphx_expert.so (always recompiles)."""
    tmpdir = tempfile.mkdtemp(prefix="phx_build_")
    try:
        procs = []
        for s in SOURCES:
            obj = os.path.join(tmpdir, s + ".o")
            cmd = [HIPCC, *FLAGS, *EXTRA.get(s, []), "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", "-o", obj,
                   os.path.join(CSRC, s)]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((s, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs = []
        failed = []
        for s, obj, p in procs:
            _, err = p.communicate()
            err = _clean(err)
            if p.returncode != 0:
                failed.append(f"{s} ({p.returncode}):\n{err}")
            elif verbose and err:
                print(err, file=sys.stderr)
            objs.append(obj)
        if failed:
            raise RuntimeError("hipcc failed: " + "\n".join(failed))
        tmp = LIB + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed ({res.returncode}):\n{_clean(res.stderr)}")
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
