"""Ahead-of-time build of librra.so for gfx950 with hipcc (in-tree)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["rra_api.hip", "varlen_fwd.hip", "varlen_bwd.hip", "paged_decode.hip", "pack_rows.hip"]
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # keep the compiler from forming packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in arch VGPRs where they fit (fewer AGPR<->VGPR moves next to
    # the softmax VALU work; measured on gfx950: head_dim 256 forward -10 %, the
    # head_dim 128 forward and the decode unchanged)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def build(out: str | None = None, verbose: bool = False) -> str:
    out = out or os.path.join(HERE, "librra.so")
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = ["hipcc", *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
        if verbose and msgs.strip():
            print(msgs)
        return obj

    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = out + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    # A kernel body the host pass cannot handle makes it drop the kernel's
    # launch stub without a diagnostic; the library would then fail to load.
    r = subprocess.run(["nm", "-u", tmp], capture_output=True, text=True)
    missing = [l.split()[-1] for l in r.stdout.splitlines() if "__device_stub__" in l]
    if missing:
        os.remove(tmp)
        raise RuntimeError("kernel launch stubs missing from the host objects: " + ", ".join(missing))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
