"""Builds liblcattn.so in-tree from csrc/*.hip with hipcc for gfx950.

    python -m long_context_attention_causal_amd.build [--jobs N] [--save-temps]

Every source is compiled with packed-fp32 VALU ops disabled (-Xclang -target-feature -Xclang -packed-fp32-ops);
hipcc's host pass warns that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblcattn.so")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")]

# Per-source extras. The prefill kernels' row maxima see no NaN unless the inputs hold one (the output is then NaN
# regardless), so they are built without NaN semantics: a max then needs no quieting of its inputs, which otherwise
# doubles the VALU work of every tile's row-max reduction. Infinities keep their meaning (masked scores are -inf).
EXTRA = {"prefill.hip": ["-fno-honor-nans"]}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, save_temps: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = ["hipcc", *COMMON, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if save_temps:
        cmd.append("--save-temps")
    r = subprocess.run(cmd, cwd=BUILD, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(jobs: int = 4, save_temps: bool = False, verbose: bool = True, out: str = LIB) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, save_temps), sources()))
    tmp = out + ".tmp"
    r = subprocess.run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--save-temps", action="store_true")
    ap.add_argument("--out", default=LIB, help="output path of the shared library")
    a = ap.parse_args()
    try:
        build(a.jobs, a.save_temps, out=os.path.abspath(a.out))
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
