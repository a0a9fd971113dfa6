"""The C-ABI library: it loads, exports every symbol include/fp8gemm.h declares, and rejects bad
arguments on the host before any device work.  CPU only (no GPU needed, no compute calls)."""
import ctypes
import os
import re

import pytest

import fp8_block_scaled_x128_amd as fg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8gemm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(fp8gemm_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fg.library_path()):
        from fp8_block_scaled_x128_amd import build
        build.build()
    return fg.lib()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("fp8gemm_nt", "fp8gemm_grouped_contiguous", "fp8gemm_grouped_masked",
              "fp8gemm_status_string", "fp8gemm_init", "fp8gemm_set_num_cus",
              "fp8gemm_last_config", "fp8gemm_read_device_error", "fp8gemm_quantize_1x128",
              "fp8gemm_quantize_1x128_masked"):
        assert n in names
    assert set(names) == set(fg.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in range(7):
        s = fg.status_string(code)
        assert s and s != "unknown status"
    assert fg.status_string(99) == "unknown status"


FAKE = 1 << 20          # aligned non-null address; never dereferenced by the validation paths


def test_dense_validation_errors(lib):
    nt = lib.fp8gemm_nt
    ok = [FAKE, FAKE, FAKE, FAKE, FAKE]
    assert nt(*ok, -1, 8, 128, None) == 2
    assert nt(*ok, 8, -1, 128, None) == 2
    assert nt(*ok, 8, 8, 100, None) == 2          # K not a multiple of 128
    assert nt(*ok, 8, 8, 0, None) == 2
    assert nt(*ok, 8, 8, 1 << 25, None) == 4      # K beyond the supported range
    assert nt(*ok, 0, 8, 128, None) == 0          # empty: a valid no-op
    assert nt(None, None, None, None, None, 0, 8, 128, None) == 0
    assert nt(None, FAKE, FAKE, FAKE, FAKE, 8, 8, 128, None) == 1
    assert nt(FAKE, FAKE, FAKE, FAKE, None, 8, 8, 128, None) == 1
    assert nt(FAKE + 8, FAKE, FAKE, FAKE, FAKE, 8, 8, 128, None) == 3
    assert nt(FAKE, FAKE + 2, FAKE, FAKE, FAKE, 8, 8, 128, None) == 3
    assert nt(FAKE, FAKE, FAKE, FAKE, FAKE + 4, 8, 8, 128, None) == 3


def test_grouped_validation_errors(lib):
    cg = lib.fp8gemm_grouped_contiguous
    assert cg(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 256, 64, 128, 0, None) == 2      # G <= 0
    assert cg(FAKE, FAKE, FAKE, FAKE, None, FAKE, 256, 64, 128, 2, None) == 1      # m_indices
    assert cg(FAKE, FAKE, FAKE, FAKE, FAKE + 2, FAKE, 256, 64, 128, 2, None) == 3
    assert cg(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 64, 128, 2, None) == 0
    mg = lib.fp8gemm_grouped_masked
    assert mg(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 64, 64, 128, -1, None) == 2  # expected_m < 0
    assert mg(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 64, 64, 128, 8, None) == 2
    assert mg(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, -1, 64, 128, 8, None) == 2
    assert mg(FAKE, FAKE, FAKE, FAKE, None, FAKE, 2, 64, 64, 128, 8, None) == 1
    assert mg(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 0, 64, 128, 8, None) == 0


def test_quantiser_validation_errors(lib):
    q = lib.fp8gemm_quantize_1x128
    assert q(FAKE, FAKE, FAKE, -1, 128, None) == 2
    assert q(FAKE, FAKE, FAKE, 8, 100, None) == 2          # K not a multiple of 128
    assert q(FAKE, FAKE, FAKE, 8, 0, None) == 2
    assert q(FAKE, FAKE, FAKE, 8, 1 << 25, None) == 4
    assert q(FAKE, FAKE, FAKE, 1 << 31, 128, None) == 4    # rows beyond the supported range
    assert q(FAKE, FAKE, FAKE, 1 << 24, 1 << 14, None) == 4  # 2^31 blocks of 128 values
    assert q(None, None, None, 0, 128, None) == 0          # empty: a valid no-op
    assert q(None, FAKE, FAKE, 8, 128, None) == 1
    assert q(FAKE, None, FAKE, 8, 128, None) == 1
    assert q(FAKE, FAKE, None, 8, 128, None) == 1
    assert q(FAKE + 8, FAKE, FAKE, 8, 128, None) == 3
    assert q(FAKE, FAKE + 8, FAKE, 8, 128, None) == 3
    assert q(FAKE, FAKE, FAKE + 2, 8, 128, None) == 3
    qm = lib.fp8gemm_quantize_1x128_masked
    assert qm(FAKE, FAKE, FAKE, FAKE, 0, 64, 128, None) == 2     # G <= 0
    assert qm(FAKE, FAKE, FAKE, FAKE, 2, -1, 128, None) == 2
    assert qm(FAKE, FAKE, FAKE, FAKE, 2, 64, 200, None) == 2
    assert qm(FAKE, FAKE, FAKE, FAKE, 2, 0, 128, None) == 0
    assert qm(FAKE, FAKE, FAKE, None, 2, 64, 128, None) == 1     # masked_m
    assert qm(FAKE, FAKE, FAKE, FAKE + 2, 2, 64, 128, None) == 3


def test_knobs(lib):
    assert lib.fp8gemm_set_num_cus(-3) == 2
    assert lib.fp8gemm_set_num_cus(64) == 0
    assert lib.fp8gemm_set_num_cus(0) == 0
    assert lib.fp8gemm_last_config(None, 16) == 1
    buf = ctypes.create_string_buffer(64)
    assert lib.fp8gemm_last_config(buf, 64) == 0
    assert lib.fp8gemm_read_device_error(None, None) == 1


def test_binding_rejects_bad_tensors():
    import torch
    A = torch.zeros((4, 128), dtype=torch.float32)
    with pytest.raises(TypeError):
        fg.gemm_nt(A, A, A, A)
    A8 = torch.zeros((4, 128), dtype=torch.uint8)
    sa = torch.zeros((4, 1), dtype=torch.float32)
    with pytest.raises(ValueError):          # host tensors are refused: no CPU path exists
        fg.gemm_nt(A8, sa, A8, sa)

    X = torch.zeros((4, 128), dtype=torch.float32)
    with pytest.raises(TypeError):           # activations must be bf16
        fg.quantize_1x128(X)
    with pytest.raises(ValueError):
        fg.quantize_1x128(X.to(torch.bfloat16))
