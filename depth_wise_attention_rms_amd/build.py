"""Build the gfx950 shared libraries in-tree with hipcc.

  libattnres.so         the product: the C ABI of include/attnres.h and its kernels
  libattnres_inputs.so  the seeded synthetic-input generator and sublayer callbacks
                        used by tests and the benchmark (no AttnRes arithmetic)

Usage: python -m depth_wise_attention_rms_amd.build [--verbose]
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function", "-I", INCLUDE,
    # fuse a*b+c only inside one expression: a score stored and then offset by
    # the running max stays separately rounded, so the max source gets exactly
    # exp(0) = 1 and a one-source aggregate returns its source bit for bit
    "-ffp-contract=on",
    # keep hipcc from forming packed-fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

LIBS = {
    "libattnres.so": ["csrc/kernels.hip", "csrc/api.hip"],
    "libattnres_inputs.so": ["inputs/gen.hip"],
}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature: harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False, extra_flags=(), out_dir: str = PKG) -> dict:
    """Compile every library into ``out_dir`` (the package directory by default)."""
    out = {}
    objdir = os.path.join(out_dir, "_build")
    os.makedirs(objdir, exist_ok=True)
    jobs = []
    for lib, srcs in LIBS.items():
        objs = []
        for s in srcs:
            src = os.path.join(PKG, s)
            obj = os.path.join(objdir, s.replace("/", "_") + ".o")
            objs.append(obj)
            jobs.append([HIPCC, *COMMON, *extra_flags, "-c", src, "-o", obj])
        out[lib] = objs
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    paths = {}
    for lib, objs in out.items():
        path = os.path.join(out_dir, lib)
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", path + ".tmp"], verbose)
        os.replace(path + ".tmp", path)
        paths[lib] = path
    return paths


if __name__ == "__main__":
    for k, v in build(verbose="--verbose" in sys.argv).items():
        print(k, "->", v)
