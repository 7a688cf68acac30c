"""Compile the HIP sources into ``libpaged_attention_attn.so`` (gfx950 only).

Run as ``python -m paged_attention_attn_amd.build`` or through
``__graft_entry__.build()``.  Every call recompiles.  No GPU is needed: hipcc
cross-compiles for gfx950.
"""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB_NAME = "libpaged_attention_attn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["abi.hip", "prefill_bf16.hip", "prefill_fp8.hip", "prefill_f32.hip", "paged_decode.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # host symbols are hidden unless the public header marks them (ATTN_API): the library exports
    # exactly the declared C entry points
    "-Xarch_host", "-fvisibility=hidden",
    "-Xarch_host", "-fvisibility-inlines-hidden",
    # packed fp32 VALU ops stay off: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(cmds), 4)) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    # the dynamic symbol table holds exactly the entry points the public header declares
    from ._binding import declared_functions
    version_script = os.path.join(BUILD, "exports.map")
    with open(version_script, "w") as f:
        f.write("{\n  global:\n" + "".join(f"    {n};\n" for n in declared_functions()) + "  local: *;\n};\n")
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, f"-Wl,--version-script={version_script}",
          "-o", tmp])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
