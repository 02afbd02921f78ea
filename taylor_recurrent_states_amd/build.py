"""Builds libtaylor_states.so in-tree with hipcc for gfx950.

    python -m taylor_recurrent_states_amd.build [-v] [--resource-usage]
    python -m taylor_recurrent_states_amd.build --sanitize

Every source is compiled on each call (this is the "does it build" check);
objects go to ``_build/`` next to this file, the library next to this file.
``--resource-usage`` also prints, per kernel, the registers, scratch
(spill) bytes, occupancy and LDS the compiler assigned (its
kernel-resource-usage remarks).  ``--sanitize`` builds the same library with
its host code under AddressSanitizer and UndefinedBehaviorSanitizer (device
code unchanged) into ``_build/sanitize/``; the ABI tests run against it.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtaylor_states.so")
SOURCES = ["tt_api.hip", "tt_decode.hip", "tt_prefill.hip", "tt_prefill_c16.hip", "tt_prefill_c32.hip",
           "tt_prefill_c128.hip", "tt_softmax.hip"]
ARCH = os.environ.get("TT_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(os.path.dirname(PKG), "include"),
]


def _compile(src: str, verbose: bool, remarks: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if remarks:
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    if remarks:
        _REMARKS[src] = r.stderr
    return obj


_REMARKS = {}
_FIELDS = {"VGPRs": "vgpr", "AGPRs": "agpr", "SGPRs": "sgpr", "ScratchSize [bytes/lane]": "scratch",
           "Occupancy [waves/SIMD]": "occupancy", "LDS Size [bytes/block]": "lds"}


def resource_usage():
    """[(source, demangled kernel, {field: value})] from the compiler's
    kernel-resource-usage remarks of the last build(resource=True)."""
    out = []
    for src, text in _REMARKS.items():
        cur = None
        for line in text.splitlines():
            m = re.search(r"Function Name: (\S+)", line)
            if m:
                name = subprocess.run(["c++filt", m.group(1)], capture_output=True, text=True).stdout.strip()
                name = re.sub(r"tt::\(anonymous namespace\)::", "", name)
                cur = {}
                out.append((src, re.sub(r"\(.*", "", name), cur))
                continue
            for key, field in _FIELDS.items():
                m = re.search(re.escape(key) + r": (\d+)", line)
                if m and cur is not None:
                    cur[field] = int(m.group(1))
    return out


SAN_BUILD = os.path.join(BUILD, "sanitize")
SAN_LIB = os.path.join(SAN_BUILD, "libtaylor_states_san.so")
# sanitizers for the host side of each translation unit only (GPU code is not
# built with them)
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-g"]


def build_sanitized(verbose: bool = False) -> str:
    """The library with host-side ASan and UBSan, rebuilt only when a source
    or header is newer than it.  Loading it needs the sanitizer runtime first
    in the process (LD_PRELOAD of clang's libclang_rt.asan)."""
    os.makedirs(SAN_BUILD, exist_ok=True)
    deps = [os.path.join(CSRC, f) for f in os.listdir(CSRC)]
    deps.append(os.path.join(os.path.dirname(PKG), "include", "taylor_states.h"))
    if os.path.exists(SAN_LIB) and os.path.getmtime(SAN_LIB) > max(os.path.getmtime(d) for d in deps):
        return SAN_LIB

    def compile_one(src: str) -> str:
        obj = os.path.join(SAN_BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *FLAGS, *SAN_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = SAN_LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


def build(verbose: bool = False, resource: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, resource), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized(verbose="-v" in sys.argv))
        sys.exit(0)
    lib = build(verbose="-v" in sys.argv, resource="--resource-usage" in sys.argv)
    if "--resource-usage" in sys.argv:
        print(f"{'source':15} {'vgpr':>4} {'agpr':>4} {'sgpr':>4} {'scratch':>7} {'occ':>3} {'lds':>6}  kernel")
        for src, name, f in resource_usage():
            print(f"{src:15} {f.get('vgpr', 0):4d} {f.get('agpr', 0):4d} {f.get('sgpr', 0):4d} "
                  f"{f.get('scratch', 0):7d} {f.get('occupancy', 0):3d} {f.get('lds', 0):6d}  {name}")
    else:
        print(lib)
