"""Build liblsh.so (all HIP sources, gfx950 only) in-tree with hipcc.

    python -m lsh_sparse_attention_amd.build
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "liblsh.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    f"--offload-arch={ARCH}",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
    "-Wall", "-Wno-unused-function",
]


# per-source extra flags: the hash keeps its matrix-core accumulators in
# ordinary VGPRs (the argmax reads every accumulator element)
EXTRA_FLAGS = {"hash.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def compile_commands(objdir: str) -> list[list[str]]:
    flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    return [[_hipcc(), *flags, *EXTRA_FLAGS.get(os.path.basename(src), []), f"-I{INCLUDE}", f"-I{CSRC}", "-c", src,
             "-o", os.path.join(objdir, os.path.basename(src) + ".o")] for src in sources()]


def _run(cmd: list[str]) -> tuple[int, str]:
    res = subprocess.run(cmd, capture_output=True, text=True)
    return res.returncode, res.stdout + res.stderr


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every HIP source (in parallel) and link liblsh.so; always recompiles."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    cmds = compile_commands(objdir)
    jobs = jobs or min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    for cmd, (rc, out) in zip(cmds, results):
        if verbose:
            print(" ".join(cmd), flush=True)
        noise = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if rc != 0 or (verbose and noise):
            sys.stderr.write("\n".join(noise) + "\n")
        if rc != 0:
            raise RuntimeError("hipcc failed on " + cmd[-3])
    tmp = LIB + ".tmp%d" % os.getpid()
    link = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
            *[c[-1] for c in cmds]]
    rc, out = _run(link)
    if rc != 0:
        sys.stderr.write(out)
        raise RuntimeError("hipcc link of liblsh.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
