"""Build libfp8gemm.so (gfx950) in-tree with hipcc.

    python -m fp8_block_scaled_x128_amd.build        # or: python fp8_block_scaled_x128_amd/build.py

Besides compiling, it checks the generated gfx950 assembly for two properties the kernels rely
on: M0 is written only by the direct-to-LDS load sequences (which set it themselves), and no
nested loop (the K loop, the split-K sums) spills to scratch memory.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libfp8gemm.so")
SOURCES = [os.path.join(CSRC, "fp8gemm_kernels.hip"), os.path.join(CSRC, "stream_kernels.hip"),
           os.path.join(CSRC, "quantize_kernels.hip"), os.path.join(CSRC, "fp8gemm_api.cpp")]
DEVICE_SOURCES = [p for p in SOURCES if p.endswith(".hip")]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 VALU ops are kept out of the device code on purpose.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                # MFMA results in VGPRs, so the promotion FMAs read them without AGPR copies
                "-mllvm", "-amdgpu-mfma-vgpr-form"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-result"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("is not a recognized feature for this target", "packed-fp32-ops")
    err = "\n".join(l for l in r.stderr.splitlines() if not any(n in l for n in noise))
    if r.returncode != 0:
        raise RuntimeError("command failed: %s\n%s" % (" ".join(cmd), err))
    return err


def check_isa(asm_text: str) -> None:
    """M0 may only be set by the LDS-DMA sequences, and no nested loop may touch scratch."""
    lines = asm_text.splitlines()
    for i, line in enumerate(lines):
        code = line.split(";", 1)[0]
        if re.search(r"\bm0\b", code):
            ok = (re.match(r"\s*s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)\s*$", code) and i + 2 < len(lines)
                  and "s_nop" in lines[i + 1] and "global_load_lds_dword" in lines[i + 2])
            if not ok:
                raise RuntimeError("unexpected use of M0 in generated code: line %d: %s" % (i + 1, line.strip()))
    # Spills are tolerated only outside nested loops: a value kept across the per-tile loop may be
    # reloaded once per tile, but nothing in the K loop (loop depth >= 2) may touch scratch.
    depth = 0
    for i, line in enumerate(lines):
        if re.match(r"^(\.LBB\w+:|; %bb\.\d+:)", line):
            m = re.search(r"Depth=(\d+)", line)
            depth = int(m.group(1)) if m else 0
        elif re.match(r"^\S+:", line):
            depth = 0
        code = line.split(";", 1)[0]
        if depth >= 2 and re.search(r"\bscratch_(load|store)", code):
            raise RuntimeError("scratch access inside a nested loop: line %d: %s" % (i + 1, line.strip()))


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    try:
        _run([HIPCC, "--offload-arch=" + ARCH] + COMMON + DEVICE_FLAGS + ["-shared", "-o", tmp] + SOURCES)
        with tempfile.TemporaryDirectory() as td:
            for src in DEVICE_SOURCES:
                asm = os.path.join(td, os.path.basename(src) + ".s")
                _run([HIPCC, "--offload-arch=" + ARCH] + COMMON + DEVICE_FLAGS +
                     ["--cuda-device-only", "-S", "-o", asm, src])
                check_isa(open(asm).read())
        os.replace(tmp, LIB)
    finally:
        if os.path.exists(tmp):
            os.remove(tmp)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
