"""Build step: compile the HIP sources into ``libdsa.so`` (gfx950 only).

Run ``python -m sparse_attention_08_amd._build`` (or ``__graft_entry__.build()``).
The library is placed next to this file so that it travels with the source tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libdsa.so")
SOURCES = ["dsa_api.hip", "topk.hip", "indexer.hip", "indexer_topk.hip", "indexer_topk_rows.hip",
           "mla.hip", "prep.hip", "noalloc.hip"]
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", f"-I{INCLUDE}",
    # packed fp32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(args):
    cmd, src = args
    p = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature flag: harmless
    err = "\n".join(l for l in p.stderr.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return err


def build(verbose: bool = False, extra_flags=()) -> str:
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="dsa_build_") as tmp:
        jobs = []
        objs = []
        for s in SOURCES:
            obj = os.path.join(tmp, s.replace(".hip", ".o"))
            objs.append(obj)
            jobs.append(([cc, *COMMON, *extra_flags, "-c", os.path.join(CSRC, s), "-o", obj], s))
        with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 4)) as ex:
            for msg in ex.map(_compile, jobs):
                if verbose and msg.strip():
                    print(msg, file=sys.stderr)
        out_tmp = LIB + ".tmp"
        cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", out_tmp]
        p = subprocess.run(cmd, capture_output=True, text=True)
        if p.returncode != 0:
            raise RuntimeError("link failed:\n" + p.stderr)
        os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
