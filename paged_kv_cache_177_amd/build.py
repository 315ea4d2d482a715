"""Build libpa.so (gfx950) in-tree with hipcc.

``python -m paged_kv_cache_177_amd.build`` compiles every source under ``csrc/`` into
``paged_kv_cache_177_amd/lib/libpa.so``, and the benchmark's read-ceiling probe under ``probe/``
into ``lib/libpa_probe.so``. It always recompiles.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIB_DIR, "libpa.so")
PROBE_DIR = os.path.join(PKG, "probe")
PROBE_LIB = os.path.join(LIB_DIR, "libpa_probe.so")
OBJ_DIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
# Packed fp32 instructions are switched off for all device code (the compiler would otherwise
# form v_pk_* ops from ordinary float code).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function"]
# Per-source flags. The multi-query kernel's scores and weights are finite or -inf, never NaN (NaN
# filler never reaches them: masked keys are replaced before use), so its maxima need not quiet
# NaN inputs first; without this the compiler puts a canonicalising v_max before every v_max.
SOURCE_FLAGS = {"pa_mq.hip": ["-fno-honor-nans"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, *SOURCE_FLAGS.get(os.path.basename(src), []), "-c",
           src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def probe_sources():
    return sorted(os.path.join(PROBE_DIR, f) for f in os.listdir(PROBE_DIR) if f.endswith(".hip"))


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    srcs = sources()
    psrcs = probe_sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(psrcs))) as ex:
        objs = list(ex.map(_compile, srcs + psrcs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
