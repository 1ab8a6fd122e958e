"""A host-sanitized build of the C ABI layer, for checking the argument validation on the CPU.

    python -m long_context_attention_causal_amd.sanitize

builds _build/sanitize/liblcattn.so: csrc/abi.hip with AddressSanitizer and UndefinedBehaviorSanitizer on its host
code (UB in trap mode, so a finding stops the process with an illegal instruction; no UBSan runtime is needed),
linked with the ordinary objects of the kernel sources (their device code is not instrumented). It prints the
environment under which a Python process uses it:

    LD_PRELOAD=<clang's ASan runtime> ASAN_OPTIONS=detect_leaks=0 LCATTN_LIB=_build/sanitize/liblcattn.so

The ASan runtime must come first in the process (Python itself is not instrumented), hence the preload. Nothing
here touches a GPU.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

from long_context_attention_causal_amd import build as B

OUT_DIR = os.path.join(B.ROOT, "_build", "sanitize")
LIB = os.path.join(OUT_DIR, "liblcattn.so")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fsanitize-trap=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def asan_runtime() -> str:
    r = subprocess.run(["hipcc", "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        path = hits[0] if hits else ""
    if not path:
        raise RuntimeError("clang's AddressSanitizer runtime was not found")
    return path


def build() -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    objs = []
    for src in B.sources():
        name = os.path.basename(src)
        obj = os.path.join(OUT_DIR, name + ".o")
        extra = HOST_SAN if name == "abi.hip" else B.EXTRA.get(name, [])
        r = subprocess.run(["hipcc", *B.COMMON, *extra, "-c", src, "-o", obj], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        objs.append(obj)
    r = subprocess.run(["hipcc", f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-o", LIB, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    return LIB


def environment() -> dict:
    env = dict(os.environ)
    env.update({"LD_PRELOAD": asan_runtime(), "ASAN_OPTIONS": "detect_leaks=0", "LCATTN_LIB": LIB})
    return env


if __name__ == "__main__":
    build()
    e = environment()
    print(f"built {LIB}\nLD_PRELOAD={e['LD_PRELOAD']} ASAN_OPTIONS={e['ASAN_OPTIONS']} LCATTN_LIB={e['LCATTN_LIB']}")
    sys.exit(0)
