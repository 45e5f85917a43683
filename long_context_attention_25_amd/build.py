"""Build libdsv4attn.so (all HIP kernels + the C ABI) for gfx950 with hipcc, its debug
build libdsv4attn_debug.so (-DDSV4_DEBUG: kernel-side checks, read with dsv4_debug_flags)
and the measurement probes libdsv4probe.so.

    python -m long_context_attention_25_amd.build

The libraries are built in-tree next to this file.  Every call recompiles.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdsv4attn.so")
# measurement helpers for bench.py (HBM streaming and MFMA throughput), a library of their own
PROBE_SRC = os.path.join(HERE, "probe", "ceilings.hip")
PROBE_LIB = os.path.join(HERE, "libdsv4probe.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-mcode-object-version=5",
    # packed fp32 forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# Per-source additions: the indexer keeps its MFMA results in ordinary VGPRs (with AGPR
# results every score took an extra copy into a VGPR before its epilogue, ~7 % of the
# decode index loop's VALU instructions).
EXTRA_FLAGS = {
    "index_topk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    raise RuntimeError("hipcc not found")


DEBUG_LIB = os.path.join(HERE, "libdsv4attn_debug.so")


def build(verbose: bool = False) -> str:
    """The release library, its debug build (kernel-side checks) and the probe library."""
    with concurrent.futures.ThreadPoolExecutor(2) as ex:   # the two builds' compiles run side by side
        for f in [ex.submit(_build, verbose, d) for d in (False, True)]:
            f.result()
    return LIB


def _build(verbose: bool, debug: bool) -> None:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "abi.cpp")]
    if not debug:
        srcs.append(PROBE_SRC)
    objs = []
    build_dir = os.path.join(HERE, "_build", "debug" if debug else "release")
    os.makedirs(build_dir, exist_ok=True)
    procs = []
    for s in srcs:
        o = os.path.join(build_dir, os.path.basename(s) + ".o")
        lang = ["-x", "hip"] if s.endswith(".cpp") else []
        cmd = [_hipcc(), *HIPCC_FLAGS, *EXTRA_FLAGS.get(os.path.basename(s), []),
               *(["-DDSV4_DEBUG"] if debug else []), *lang, "-I",
               os.path.join(HERE, "..", "include"), "-c", s, "-o", o]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((s, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(o)
    failed = []
    for s, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        if p.returncode != 0:
            failed.append((s, text))
        elif verbose and text.strip():
            print(text)
    if failed:
        for s, t in failed:
            sys.stderr.write(f"--- {s}\n{t}\n")
        raise RuntimeError(f"hipcc failed for {[os.path.basename(s) for s, _ in failed]}")
    if debug:
        targets = ((DEBUG_LIB, objs),)
    else:
        probe_obj = objs.pop()               # the last source is the probe library's
        targets = ((LIB, objs), (PROBE_LIB, [probe_obj]))
    for lib, parts in targets:
        tmp = lib + ".tmp"
        cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *parts]
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
