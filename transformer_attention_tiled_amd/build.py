"""Build libattn.so in-tree with hipcc for gfx950 only.

Each source compiles to its own object (in parallel) under ``_build/`` at the
repository root, then one link produces ``transformer_attention_tiled_amd/libattn.so``.
Every HIP compile disables packed fp32 VALU instructions
(``-Xclang -target-feature -Xclang -packed-fp32-ops``).
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
OUT = os.path.join(PKG, "libattn.so")
ARCH = "gfx950"

SOURCES = ["attn_api.cpp", "prefill_bf16.hip", "prefill_f32.hip", "decode_paged.hip",
           "decode_noalloc.hip",
           "kv_append.hip", "add_rmsnorm.hip"]
# the benchmark's measurement probe: a library of its own, not part of libattn
PROBE_SOURCES = ["probe.hip"]
PROBE_OUT = os.path.join(PKG, "libattn_probe.so")

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def _compile(src, extra):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{errs}")
    return obj, errs


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose=False, extra_flags=()):
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(lambda s: _compile(s, list(extra_flags)), srcs))
    if verbose:
        for _, errs in results:
            if errs.strip():
                print(errs, file=sys.stderr)
    objs = [o for o, _ in results]
    _link(objs[:len(SOURCES)], OUT)
    _link(objs[len(SOURCES):], PROBE_OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
