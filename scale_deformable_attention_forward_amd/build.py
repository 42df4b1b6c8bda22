"""Build libmsda.so (the gfx950 HIP library behind include/msda.h) and the
benchmark's probe library libmsda_probe.so in-tree.

Usage: python -m scale_deformable_attention_forward_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmsda.so")
SOURCES = ["msda_api.hip", "msda_forward.hip", "msda_backward.hip", "msda_producer.hip"]
PROBE_LIB = os.path.join(PKG, "libmsda_probe.so")
PROBE_SOURCES = ["msda_probe.hip"]
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
# -munsafe-fp-atomics: float atomicAdd lowers to global_atomic_add_f32 (device memory from hipMalloc).
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-munsafe-fp-atomics", f"-I{INCLUDE}"]


def _build(sources, lib_path, verbose):
    """Compile `sources` in parallel, link them into `lib_path`, replace it atomically."""
    with tempfile.TemporaryDirectory(prefix="msda_build_") as tmp:
        procs = []
        objs = []
        for src in sources:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
        failed = []
        for cmd, p in procs:
            out, _ = p.communicate()
            text = out.decode(errors="replace")
            # the host pass does not know the device-only feature flag: harmless
            text = "\n".join(ln for ln in text.splitlines() if "packed-fp32-ops" not in ln)
            if p.returncode != 0:
                failed.append((cmd, text))
            elif verbose and text.strip():
                print(text, flush=True)
        if failed:
            msg = "\n\n".join(" ".join(c) + "\n" + t for c, t in failed)
            raise RuntimeError(f"hipcc failed:\n{msg}")
        tmp_lib = os.path.join(tmp, os.path.basename(lib_path))
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib, *objs,
               "-Wl,-rpath,/opt/rocm/lib"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        shutil.copyfile(tmp_lib, lib_path + ".tmp")
        os.replace(lib_path + ".tmp", lib_path)
    return lib_path


def build_library(verbose: bool = False) -> str:
    """Build libmsda.so (the library behind include/msda.h) and
    libmsda_probe.so (cache-bandwidth probes the benchmark's roofline uses)."""
    _build(PROBE_SOURCES, PROBE_LIB, verbose)
    return _build(SOURCES, LIB, verbose)


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
