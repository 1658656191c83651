"""Build the HIP library libfa_mi355x.so for gfx950, in-tree.

    python -m io_aware_exact_forward_amd.build

compiles every translation unit under csrc/ with hipcc for gfx950 and links
them (plus rocBLAS, used by the materialised baseline's two products) into
io_aware_exact_forward_amd/lib/libfa_mi355x.so, and builds the measurement
helper csrc/probe/fa_mfma_probe.hip (the sustained matrix-core rate bench.py
reports beside the roofline) into lib/libfa_probe.so.  It always recompiles.
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
LIBDIR = os.path.join(PKG, "lib")
LIBNAME = "libfa_mi355x.so"
PROBE_LIBNAME = "libfa_probe.so"
PROBE_SOURCE = os.path.join(CSRC, "probe", "fa_mfma_probe.hip")
ARCH = "gfx950"

SOURCES = ["fa_api.cpp", "fa_fwd_bf16.hip", "fa_fwd_f32.hip", "fa_merge.hip", "fa_decode.hip",
           "fa_bwd_bf16.hip", "naive_softmax.hip", "naive_backward.hip"]

# Packed fp32 VALU forms are kept out of the generated code; the compiler
# would otherwise pair independent fp32 operations into them.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def lib_path() -> str:
    return os.path.join(LIBDIR, LIBNAME)


def probe_lib_path() -> str:
    return os.path.join(LIBDIR, PROBE_LIBNAME)


def build(verbose: bool = False) -> str:
    cc = hipcc()
    os.makedirs(LIBDIR, exist_ok=True)
    with tempfile.TemporaryDirectory(prefix="fa_build_") as tmp:
        procs = []
        objs = []
        probe_tmp = os.path.join(tmp, PROBE_LIBNAME)
        probe_cmd = [cc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
                     *DEVICE_FLAGS, PROBE_SOURCE, "-o", probe_tmp]
        if verbose:
            print(" ".join(probe_cmd), flush=True)
        probe_proc = subprocess.Popen(probe_cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".", "_") + ".o")
            cmd = [cc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-c",
                   "-I", INCLUDE, "-I", CSRC, *DEVICE_FLAGS, os.path.join(CSRC, src), "-o", obj]
            if src.endswith(".cpp"):
                cmd.insert(1, "-xhip")
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
        errors = []
        for src, p in procs:
            out, _ = p.communicate()
            text = out.decode(errors="replace")
            # hipcc's host pass does not know the device-only feature: drop that note
            text = "\n".join(ln for ln in text.splitlines() if "not a recognized feature" not in ln)
            if p.returncode != 0:
                errors.append(f"{src}:\n{text}")
            elif verbose and text.strip():
                print(text, flush=True)
        out, _ = probe_proc.communicate()
        if probe_proc.returncode != 0:
            text = "\n".join(ln for ln in out.decode(errors="replace").splitlines()
                             if "not a recognized feature" not in ln)
            errors.append(f"probe/fa_mfma_probe.hip:\n{text}")
        if errors:
            raise RuntimeError("HIP build failed:\n" + "\n".join(errors))
        tmp_lib = os.path.join(tmp, LIBNAME)
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib,
               "-L/opt/rocm/lib", "-lrocblas", "-Wl,-rpath,/opt/rocm/lib"]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        if r.returncode != 0:
            raise RuntimeError("HIP link failed:\n" + r.stdout.decode(errors="replace"))
        # replace atomically so a loaded copy is never half-written
        for src, dst in ((tmp_lib, lib_path()), (probe_tmp, probe_lib_path())):
            shutil.copyfile(src, dst + ".tmp")
            os.replace(dst + ".tmp", dst)
    return lib_path()


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
