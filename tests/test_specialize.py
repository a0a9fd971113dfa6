"""Run-time shape specialisation of the tiled kernel, on the CPU: hipRTC builds gfx950 code objects
without a GPU, so the generated code itself is checked here -- it compiles for every dense table
entry at the benchmark's N and K, names the requested constants, keeps the device-code rules of the
ahead-of-time build (no packed fp32 VALU instructions, M0 written only to address direct-to-LDS
loads, no scratch memory), and the entry points reject bad arguments before any device work."""
import os
import re
import subprocess
import sys
import tempfile

import pytest

import fp8_block_scaled_x128_amd as fg
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"
READELF = "/opt/rocm/llvm/bin/llvm-readelf"


def dense_entries():
    src = open(os.path.join(ROOT, "fp8_block_scaled_x128_amd", "csrc", "fp8gemm_kernels.hip")).read()
    return [tuple(int(x) for x in t) for t in
            re.findall(r"FP8GEMM_ENTRY\((\d+), (\d+), (\d+), (\d+), (\d+), kDense\)", src)]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fg.library_path()):
        from fp8_block_scaled_x128_amd import build
        build.build()
    return fg.lib()


def disassemble(code: bytes) -> str:
    with tempfile.NamedTemporaryFile(suffix=".co") as f:
        f.write(code)
        f.flush()
        return subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", f.name], capture_output=True, text=True,
                              check=True).stdout


def notes(code: bytes) -> str:
    with tempfile.NamedTemporaryFile(suffix=".co") as f:
        f.write(code)
        f.flush()
        return subprocess.run([READELF, "--notes", f.name], capture_output=True, text=True, check=True).stdout


def check_code(code: bytes, entry, what):
    bm, bn, wm, wn, st = entry
    asm = disassemble(code)
    lines = [l.split("//")[0].strip() for l in asm.splitlines()]
    ins = [l for l in lines if re.match(r"^[sv]_|^global_|^buffer_|^ds_|^scratch_", l)]
    assert not [l for l in ins if re.match(r"v_pk_(fma|mul|add)_f32", l)], what + ": packed fp32 VALU op"
    assert not [l for l in ins if l.startswith("scratch_")], what + ": scratch access"
    # M0: set only right before a direct-to-LDS load (s_mov_b32 m0, <scalar register>; s_nop 0;
    # global_load_lds_*) -- the register holds the LDS address; vcc_lo/hi serve as scalar registers too
    for i, l in enumerate(ins):
        if re.search(r"\bm0\b", l):
            assert re.match(r"s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)$", l), (what, l)
            assert ins[i + 1].startswith("s_nop") and ins[i + 2].startswith("global_load_lds_dword"), (what, l)
    n_mfma = sum(1 for l in ins if re.match(r"v_mfma_(scale_)?f32_16x16x128_f8f6f4", l))
    per_slice = (bm // wm // 16) * (bn // wn // 16)
    assert n_mfma > 0 and n_mfma % per_slice == 0, (what, n_mfma, per_slice)
    meta = notes(code)
    assert re.search(r"\.private_segment_fixed_size:\s+0\b", meta), what + ": uses scratch"
    vgpr = int(re.search(r"\.vgpr_count:\s+(\d+)", meta).group(1))
    assert vgpr <= 512, (what, vgpr)
    return n_mfma, vgpr


@pytest.mark.skipif(not os.path.exists(OBJDUMP), reason="llvm-objdump not installed")
@pytest.mark.parametrize("entry", dense_entries(), ids=lambda e: "%dx%d_w%dx%d_s%d" % e)
def test_code_object_per_dense_entry(lib, entry):
    """Each dense tiled entry specialised to a sweep shape (N = 2112 has a ragged N tail)."""
    N, K = (2112, 7168) if entry[0] != 256 else (4096, 7168)
    code, sym = fg.specialized_code_object(0, *entry, N, K)
    assert code[:4] == b"\x7fELF"
    assert "Li%dELi%dEE" % (N, K) in sym, sym          # the constants are in the kernel's name
    check_code(code, entry, sym)


def test_code_object_every_sweep_shape_of_the_prefill_tile(lib):
    """The 256x256 dense tile at every (N, K) of the dense sweep."""
    for N, K in W.SWEEP_NK:
        code, sym = fg.specialized_code_object(0, 256, 256, 4, 2, 2, N, K)
        check_code(code, (256, 256, 4, 2, 2), sym)


def test_code_object_argument_errors(lib):
    f = lib.fp8gemm_specialized_code_object
    import ctypes
    size = ctypes.c_size_t(0)
    assert f(0, 256, 256, 4, 2, 3, 4096, 7168, None, ctypes.byref(size), None, 0) == 2   # not in the table
    assert f(0, 256, 256, 4, 2, 2, 4096, 7000, None, ctypes.byref(size), None, 0) == 2   # K % 128
    assert f(0, 256, 256, 4, 2, 2, 0, 7168, None, ctypes.byref(size), None, 0) == 2      # N <= 0
    assert f(0, 256, 256, 4, 2, 2, 4096, 7168, None, None, None, 0) == 1                 # no size
    assert f(0, 64, 64, 1, 4, 4, 256, 512, None, ctypes.byref(size), None, 0) == 0 and size.value > 0
    small = ctypes.create_string_buffer(16)
    size2 = ctypes.c_size_t(16)
    assert f(0, 64, 64, 1, 4, 4, 256, 512, small, ctypes.byref(size2), None, 0) == 2     # buffer too small
    assert size2.value == size.value


FAKE = 1 << 20


def test_specialized_entry_validation_errors(lib):
    nt = lib.fp8gemm_nt_specialized
    ok = [FAKE, FAKE, FAKE, FAKE, FAKE]
    assert nt(*ok, -1, 8, 128, None) == 2
    assert nt(*ok, 8, 8, 100, None) == 2
    assert nt(*ok, 8, 8, 1 << 25, None) == 4
    assert nt(*ok, 0, 8, 128, None) == 0
    assert nt(None, FAKE, FAKE, FAKE, FAKE, 8, 8, 128, None) == 1
    assert nt(FAKE + 8, FAKE, FAKE, FAKE, FAKE, 8, 8, 128, None) == 3
    import ctypes
    ms = ctypes.c_double(0)
    assert lib.fp8gemm_specialize_nt(0, 8, 128, ctypes.byref(ms)) == 2
    assert lib.fp8gemm_specialize_nt(8, 8, 100, ctypes.byref(ms)) == 2
    assert lib.fp8gemm_specialized_count() == 0


ENV_CHURN = r"""
import ctypes, os, sys
sys.path.insert(0, sys.argv[1])
import fp8_block_scaled_x128_amd as fg
libc = ctypes.CDLL(None)
libc.dlmopen.restype = ctypes.c_void_p
libc.dlmopen.argtypes = [ctypes.c_long, ctypes.c_char_p, ctypes.c_int]
libc.dlsym.restype = ctypes.c_void_p
libc.dlsym.argtypes = [ctypes.c_void_p, ctypes.c_char_p]
RTLD_NOW, RTLD_NOLOAD = 2, 4
main_environ = lambda: ctypes.c_void_p.in_dll(libc, "environ").value

fg.specialized_code_object(0, 64, 64, 1, 4, 4, 256, 512)     # loads the compiler
ns = [lm for lm in range(1, 16) if libc.dlmopen(lm, b"libhiprtc.so.7", RTLD_NOW | RTLD_NOLOAD)]
assert len(ns) == 1, ns
slot = libc.dlsym(libc.dlmopen(ns[0], b"libc.so.6", RTLD_NOW | RTLD_NOLOAD), b"environ")
ns_environ = ctypes.c_void_p.from_address(slot)

for i in range(40):                                          # grow the environment: its array moves
    os.environ["FP8GEMM_TEST_CHURN_%d" % i] = "x" * (i + 1)
for i in range(40):
    os.environ.pop("FP8GEMM_TEST_CHURN_%d" % i)
os.environ["FP8GEMM_TEST_LATE"] = "1"
code, sym = fg.specialized_code_object(0, 64, 64, 1, 4, 4, 384, 512)
assert code[:4] == b"\x7fELF", sym
assert ns_environ.value == main_environ(), "the namespace reads a stale environment"

# an environment pointer the compiler cannot read (as a freed array may be) is replaced before
# the compile reads it
bad = (ctypes.c_void_p * 3)(0x10, 0x10, None)
ns_environ.value = ctypes.addressof(bad)
code, sym = fg.specialized_code_object(0, 64, 64, 1, 4, 4, 512, 512)
assert code[:4] == b"\x7fELF" and ns_environ.value == main_environ()
print("ok")
"""


def test_compile_after_the_environment_moved(lib):
    """The compiler lives in a linker namespace of its own, with its own C library, whose environment
    pointer is the process's array as it was at load time; setenv frees that array when it grows
    the environment, and every compile reads the environment.  Before each compile the namespace's
    pointer must be the process's current one (checked after a real move of the array, and after
    the pointer was set to memory that cannot be read).  Runs in a child process."""
    r = subprocess.run([sys.executable, "-c", ENV_CHURN, ROOT], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.returncode, r.stdout[-2000:], r.stderr[-2000:])
