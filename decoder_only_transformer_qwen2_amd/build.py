"""Build libqw.so in-tree with hipcc for gfx950.

    python -m decoder_only_transformer_qwen2_amd.build

Every .hip file under csrc/ is compiled to an object in _build/ and linked
into decoder_only_transformer_qwen2_amd/libqw.so.  Packed-fp32 instructions
are turned off for device code (a correctness precaution on this target).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqw.so")
ARCH = os.environ.get("QW_OFFLOAD_ARCH", "gfx950")

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-munsafe-fp-atomics", "-I", os.path.join(ROOT, "include"),
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Per-source device-code options.  The prefill attention keeps its output
# accumulators in ordinary VGPRs (the VGPR form of the MFMA instructions):
# with the accumulation registers the compiler copied every accumulator out
# and back in once per key block.
EXTRA = {
    "k_attn_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    # the MFMA-only peak loop: with accumulation registers the compiler
    # rotated every accumulator through VGPRs once per iteration
    "k_peak.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str, build_dir: str = BUILD, defines=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *CFLAGS, *[f"-D{d}" for d in defines], *EXTRA.get(os.path.basename(src), []), "-c", src,
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = True, defines=(), out: str = LIB, build_dir: str = BUILD) -> str:
    """Compile every source and link `out` (the in-tree libqw.so by default).
    `defines` adds -D macros, e.g. for a tuning build placed elsewhere."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, build_dir, defines), srcs))
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out} from {len(srcs)} sources")
    return out


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("-D", dest="defines", action="append", default=[], help="extra preprocessor macro")
    ap.add_argument("--out", default=LIB)
    ap.add_argument("--build-dir", default=BUILD)
    args = ap.parse_args()
    build(defines=args.defines, out=args.out, build_dir=args.build_dir)
