"""Build libsss.so (HIP, gfx950) in-tree with hipcc.

``python -m sparse_self_speculative_sss_amd.build`` compiles every source in
``csrc/`` and links ``libsss.so`` next to this file.  Object files go to
``_build/`` at the repository root.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
OBJ_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG_DIR, "libsss.so")
SOURCES = ["api.hip", "attn_mfma.hip", "attn_simple.hip", "finalize.hip", "fused.hip",
           "kv_update.hip", "persist.hip", "probe.hip", "topk.hip", "verify_rows.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU instructions stay off: plain scalar fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-result",
]


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in res.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    return res.returncode, out


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        rc, out = _run(cmd)
        return src, obj, rc, out

    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(SOURCES)))) as ex:
        results = list(ex.map(compile_one, SOURCES))
    errors = [(s, out) for s, _, rc, out in results if rc != 0]
    for s, _, rc, out in results:
        if out.strip() and (verbose or rc != 0):
            print(f"--- {s}\n{out}", file=sys.stderr)
    if errors:
        raise RuntimeError("hipcc failed for: " + ", ".join(s for s, _ in errors))
    tmp = LIB + ".tmp"
    rc, out = _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
                    *[obj for _, obj, _, _ in results]])
    if rc != 0:
        print(out, file=sys.stderr)
        raise RuntimeError("link of libsss.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
