"""Build libtq.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python -m kv_cache_vector_rht_amd.build            # build
    python -m kv_cache_vector_rht_amd.build --check    # + print exported tq_* symbols

Every call recompiles. Objects go to kv_cache_vector_rht_amd/_build/, the
library to kv_cache_vector_rht_amd/libtq.so.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libtq.so")
BUILD = os.path.join(HERE, "_build")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

SOURCES = ["tq_decode_d128.hip", "tq_append_d128.hip", "tq_encode_d128.hip", "tq_decode_d64.hip",
           "tq_append_d64.hip", "tq_encode_d64.hip", "tq_msek_d128.hip", "tq_msek_append_d128.hip",
           "tq_msek_d64.hip", "tq_msek_append_d64.hip", "tq_prefill_d128.hip", "tq_prefill_d64.hip",
           "tq_fp8.hip", "tq_topk.hip", "tq_probe.hip", "tq_table.hip", "tq_api.hip", "tq_codebook.cpp"]

ARCH = os.environ.get("TQ_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 VALU forms anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=fast", "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libtq)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [hipcc(), "-O2", "-std=c++17", "-fPIC", "-x", "c++", "-c",
               os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


def exported_symbols(path: str = OUT) -> list[str]:
    r = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True)
    return sorted(ln.split()[-1] for ln in r.stdout.splitlines() if ln.split()[-1].startswith("tq_"))


if __name__ == "__main__":
    build()
    if "--check" in sys.argv:
        print("\n".join(exported_symbols()))
