"""Compile libw4a16.so for gfx950 in-tree with hipcc (runs on a machine without a GPU)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = [os.path.join(CSRC, "gemm.hip"), os.path.join(CSRC, "repack.hip"),
           os.path.join(CSRC, "moe.hip"), os.path.join(CSRC, "probe.hip"),
           os.path.join(CSRC, "pack.cpp")]
LIB = os.path.join(PKG, "libw4a16.so")
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            # code object v5 loads in the HIP runtime PyTorch bundles as well as the system one
            "-mcode-object-version=5",
            "-Wall", "-Wno-unused-function",
            # packed fp32 arithmetic stays off (plain fp32 only in this library)
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA results in ordinary VGPRs: the fp32 epilogue math reads them directly
            # instead of copying each accumulator out of the AGPR file first
            "-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form",
            "-I", os.path.join(ROOT, "include")]


def command(out: str = LIB, extra=()) -> list:
    """One hipcc line that compiles every source and links the library."""
    return [hipcc(), *flags(), "-shared", *SOURCES, "-o", out, *extra]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (res.stdout + res.stderr).splitlines()
            if "packed-fp32-ops' is not a recognized feature" not in l]
    return res.returncode, msgs


ABLATIONS = ("cached_weights", "shallow", "no_swizzle")


def ablation_lib(name: str) -> str:
    """Path of a measurement-only build (see the W4A16_ABLATE_* switches in gemm.hip)."""
    return os.path.join(PKG, f"libw4a16_ablate_{name}.so")


def build(verbose: bool = False, ablation: str | None = None) -> str:
    """Compile each source to an object in parallel, then link libw4a16.so (the same flags as
    command(), one compiler process per source).  ablation: one of ABLATIONS, for a
    measurement-only library beside it (libw4a16_ablate_<name>.so)."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(PKG, "_build" if ablation is None else f"_build_{ablation}")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(src) + ".o") for src in SOURCES]
    extra = [] if ablation is None else [f"-DW4A16_ABLATE_{ablation.upper()}"]
    if ablation is not None and ablation not in ABLATIONS:
        raise ValueError(f"unknown ablation {ablation!r}; one of {ABLATIONS}")
    cmds = [[hipcc(), *flags(), *extra, "-c", src, "-o", obj] for src, obj in zip(SOURCES, objs)]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        results = list(ex.map(_run, cmds))
    for (rc, msgs), c in zip(results, cmds):
        if rc != 0:
            sys.stderr.write("\n".join(msgs) + "\n")
            raise RuntimeError(f"hipcc failed with exit code {rc}: {c[-3]}")
        if verbose and msgs:
            print("\n".join(msgs))
    out = LIB if ablation is None else ablation_lib(ablation)
    tmp = out + ".tmp"
    link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    rc, msgs = _run(link)
    if rc != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError(f"hipcc link failed with exit code {rc}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("--ablation", choices=ABLATIONS + ("all",),
                    help="build a measurement-only library instead (all: each of them)")
    a = ap.parse_args()
    if a.ablation == "all":
        for name in ABLATIONS:
            print(build(verbose=True, ablation=name))
    else:
        print(build(verbose=True, ablation=a.ablation))
