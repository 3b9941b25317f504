"""Compile the HIP/C++ sources into the in-tree shared library libthdattn.so.

Every source is built by hipcc for gfx950 only. Host-only files go through
hipcc too (they call the HIP runtime). Packed fp32 instructions are switched
off for device code.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libthdattn.so")
SOURCES = ["thd_plan.cpp", "thd_api.cpp", "thd_fwd.hip", "thd_bwd.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Werror", "-Wno-unused-command-line-argument",
          "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
DEVICE = ["-x", "hip", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-Wno-unknown-warning-option"]
# Per-file device flags. The forward: NaNs are not data there (inputs are
# finite; masked scores are -inf), and with the IEEE mode bit off v_max_f32
# needs no canonicalising copy of each MFMA result before the row-maximum tree
# (16 instructions per 64-key tile). The backward has no maxima and keeps the
# defaults (its dK/dV kernel is register-allocated to three workgroups per CU).
FILE_FLAGS = {"thd_fwd.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON + (DEVICE + FILE_FLAGS.get(src, []) if src.endswith(".hip")
                              else ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"])
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as pool:
        objs = list(pool.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    # Loading resolves every symbol now: a missing kernel launch stub fails the build here.
    import ctypes
    ctypes.CDLL(os.path.abspath(tmp))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


def resources() -> str:
    """Per-kernel register, LDS and scratch use of the gfx950 code (read from
    the assembler's kernel descriptors), as a Markdown table."""
    import re
    rows = []
    for src in SOURCES:
        if not src.endswith(".hip"):
            continue
        asm = os.path.join(BUILD, os.path.splitext(src)[0] + ".s")
        os.makedirs(BUILD, exist_ok=True)
        cmd = [HIPCC] + COMMON + DEVICE + FILE_FLAGS.get(src, []) + [
            "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", asm]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(res.stderr)
        text = open(asm).read()
        for name, body in re.findall(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", text, re.S):
            def field(key):
                m = re.search(r"\.amdhsa_" + key + r" (\d+)", body)
                return int(m.group(1)) if m else 0
            vgpr, acc = field("next_free_vgpr"), field("accum_offset")
            lds, scratch, sgpr = field("group_segment_fixed_size"), field("private_segment_fixed_size"), field("next_free_sgpr")
            demangled = subprocess.run(["c++filt", name], capture_output=True, text=True).stdout.strip()
            short = re.sub(r"thd::\(anonymous namespace\)::", "", demangled).replace("(thd::FwdParams)", "").replace("(thd::BwdParams)", "")
            waves = max(1, min(8, 512 // max(vgpr, 1)))
            rows.append(f"| `{short}` | {vgpr} | {max(vgpr - acc, 0)} | {sgpr} | {lds} | {scratch} | {waves} |")
    head = ("| kernel | VGPRs (arch + acc) | of which AGPRs | SGPRs | LDS bytes | scratch bytes | waves per SIMD by VGPRs |\n"
            "|---|---|---|---|---|---|---|")
    return head + "\n" + "\n".join(rows)


if __name__ == "__main__":
    if "--resources" in sys.argv:
        print(resources())
        sys.exit(0)
    build(verbose=True)
    sys.exit(0)
