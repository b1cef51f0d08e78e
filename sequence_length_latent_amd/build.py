"""Build the SFA shared library (gfx950) in-tree.

    python -m sequence_length_latent_amd.build

Compiles every source under ``csrc/`` with hipcc for gfx950 only and links
``sequence_length_latent_amd/_hd_sfa.so``.  Objects go to ``_build/`` at the
repository root.  Packed-fp32 instructions are disabled for all device code.
The compiler's resource report of every kernel (registers, scratch, LDS,
occupancy) is written next to the library as ``_hd_sfa.resources.json``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import json
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "_hd_sfa.so")
RESOURCES = os.path.join(PKG, "_hd_sfa.resources.json")
_REMARK = "-Rpass-analysis=kernel-resource-usage"
_FIELDS = {"vgpr": r"VGPRs: (\d+)", "agpr": r"AGPRs: (\d+)", "sgpr": r"SGPRs: (\d+)",
           "scratch_bytes_per_lane": r"ScratchSize \[bytes/lane\]: (\d+)",
           "vgpr_spill": r"VGPRs Spill: (\d+)", "sgpr_spill": r"SGPRs Spill: (\d+)",
           "lds_bytes": r"LDS Size \[bytes/block\]: (\d+)",
           "occupancy_waves_per_simd": r"Occupancy \[waves/SIMD\]: (\d+)"}

ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build the library)")
    return path


def _resources(report: str) -> dict:
    """Kernel name -> resource fields, from the compiler's resource remarks."""
    out = {}
    for chunk in report.split("Function Name: ")[1:]:
        name = chunk.split()[0]
        out[name] = {k: int(m.group(1)) for k, pat in _FIELDS.items() if (m := re.search(pat, chunk))}
    return out


def _compile(src: str):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    device = src.endswith(".hip")
    cmd = [hipcc(), *CFLAGS, *([_REMARK] if device else []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    lines = [l for l in (r.stderr or "").splitlines() if noise not in l]
    remarks = "\n".join(l for l in lines if "remark:" in l)
    # a remark is followed by its source line and a caret line ("  12 | ...", "     | ^")
    err = "\n".join(l for l in lines if "remark:" not in l and not re.match(r"^\s*\d*\s*\|", l))
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj, _resources(remarks)


# Host-side sanitizers for the checking build: AddressSanitizer and
# UndefinedBehaviorSanitizer on the host code only (argument validation, plans,
# launches); every flag is routed to the host pass, the device code is built
# exactly as in the product library.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
SANITIZED_BUILD = os.path.join(BUILD, "sanitized")
SANITIZED_LIB = os.path.join(SANITIZED_BUILD, "_hd_sfa_sanitized.so")


def build_sanitized(verbose: bool = True) -> str:
    """Compile the library with host-side ASan + UBSan into
    ``_build/sanitized/_hd_sfa_sanitized.so`` (for the CPU sanitizer test; it
    needs the sanitizer runtime preloaded to be loaded)."""
    os.makedirs(SANITIZED_BUILD, exist_ok=True)
    srcs = _sources()

    def one(src):
        obj = os.path.join(SANITIZED_BUILD, os.path.basename(src) + ".o")
        cmd = [hipcc(), *CFLAGS, *SANITIZE_FLAGS, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(one, srcs))
    tmp = SANITIZED_LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libsan",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, SANITIZED_LIB)
    if verbose:
        print(f"built {SANITIZED_LIB} (host ASan + UBSan)")
    return SANITIZED_LIB


def sanitizer_runtime() -> str:
    """Path of the ASan runtime shared library of the compiler hipcc uses."""
    clangxx = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang++")
    if not os.path.exists(clangxx):
        clangxx = "/opt/rocm/llvm/bin/clang++"
    r = subprocess.run([clangxx, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                       text=True)
    return r.stdout.strip()


def _sources():
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    if not srcs:
        raise RuntimeError("no sources under csrc/")
    return srcs


def build(verbose: bool = True) -> str:
    """Compile all sources and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = _sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        done = list(ex.map(_compile, srcs))
    objs = [o for o, _ in done]
    resources = {}
    for _, res in done:
        resources.update(res)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    with open(RESOURCES + ".tmp", "w") as f:
        json.dump(resources, f, indent=1, sort_keys=True)
    os.replace(RESOURCES + ".tmp", RESOURCES)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build()
