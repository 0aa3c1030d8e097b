"""Build libgdn.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc.

Also builds libgdn_hooks.so, the same library with chunk_mfma.hip compiled with GDN_TEST_HOOKS:
that build lets environment variables override the automatic route choice so that the tests
can run every kernel family on small shapes.  The release library reads no environment.  And
libgdn_debug.so: the hooks build with GDN_DEBUG too, whose prefill kernels check their indices
and report failed checks through gdn_debug_take_flags (include/gdn_debug.h)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgdn.so")
LIB_HOOKS = os.path.join(PKG, "libgdn_hooks.so")
LIB_DEBUG = os.path.join(PKG, "libgdn_debug.so")
SOURCES = ["api.cpp", "decode.hip", "chunk_simt.hip", "chunk_mfma.hip", "layer_ops.hip", "chunk_bwd.hip", "kda.hip",
           "noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed-fp32 instructions are kept out of the generated code (plain float code only).
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall",
         "-Wno-unused-command-line-argument"]


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = []   # (label, object, command)
    objs = []
    for src in SOURCES:
        obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        jobs.append((src, obj, [HIPCC] + FLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", obj]))
    hooks_obj = os.path.join(OBJDIR, "chunk_mfma_hooks.o")
    jobs.append(("chunk_mfma.hip (test hooks)", hooks_obj,
                 [HIPCC] + FLAGS + ["-DGDN_TEST_HOOKS", "-x", "hip", "-c", os.path.join(CSRC, "chunk_mfma.hip"), "-o", hooks_obj]))
    debug_obj = os.path.join(OBJDIR, "chunk_mfma_debug.o")
    jobs.append(("chunk_mfma.hip (index checks)", debug_obj,
                 [HIPCC] + FLAGS + ["-DGDN_TEST_HOOKS", "-DGDN_DEBUG", "-x", "hip", "-c", os.path.join(CSRC, "chunk_mfma.hip"),
                                    "-o", debug_obj]))
    procs = []
    for label, _, cmd in jobs:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((label, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for label, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature flag and says so; that is harmless.
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if p.returncode != 0:
            failed.append(label)
            sys.stderr.write(text)
        elif verbose and lines:
            sys.stderr.write("\n".join(lines) + "\n")
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    hooks_objs = [hooks_obj if o.endswith(os.sep + "chunk_mfma.o") else o for o in objs]
    debug_objs = [debug_obj if o.endswith(os.sep + "chunk_mfma.o") else o for o in objs]
    for out, parts in ((LIB, objs), (LIB_HOOKS, hooks_objs), (LIB_DEBUG, debug_objs)):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}"] + parts + ["-o", tmp], check=True)
        os.replace(tmp, out)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
