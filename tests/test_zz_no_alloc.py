"""GPU: fp8gemm_nt_noalloc, the dense NT GEMM whose split-K partials live in the library's static
device scratch, called through the C ABI.  Each call must give fp8gemm_nt's bits on the same
operands (same kernels, launch shape and summation order) and match the oracle within
|gpu - ref| <= 2^-7 |ref| + 1e-3 rms(ref); two calls in a row, the second on a smaller problem,
so the scratch left by the first must not leak into the second.  A launch needing more than the
scratch holds is refused before anything is enqueued."""
import os
import re
import sys

import numpy as np
import pytest

import oracle
import workloads as W
from parity import assert_close, gpu_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU runs deselect these with -m "not gpu"
    pytest.skip("needs a GPU", allow_module_level=True)

import fp8_block_scaled_x128_amd as fg  # noqa: E402

SENTINEL = 0x7FC1


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def abi_call(name, ops, D, M, N, K):
    """The entry point through ctypes with raw device pointers and torch's current stream."""
    fn = getattr(fg.lib(), name)
    rc = fn(*[t.data_ptr() for t in ops], D.data_ptr(), M, N, K, torch.cuda.current_stream().cuda_stream)
    cfg = fg.last_config()
    return rc, cfg


def split_of(cfg):
    return int(re.search(r"split=(\d+)", cfg).group(1))


def test_noalloc_matches_nt_two_calls_second_smaller():
    # 128 x 7168 x 16384: 56 tiles of 128 x 128, 4 K splits, 14.7 MB of partials; then
    # 64 x 2112 x 7168: 33 tiles of 64 x 64, 7 K splits, 3.8 MB
    for M, N, K, seed in ((128, 7168, 16384, 601), (64, 2112, 7168, 602)):
        say("noalloc case", M, N, K)
        d = W.dense(M, N, K, seed=seed)
        ops = (dev(d.A), dev(np.swapaxes(d.sa, 0, 1)), dev(d.B), dev(d.sb))
        D_ref = torch.full((M, N), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        D = torch.full((M, N), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        rc, cfg_ref = abi_call("fp8gemm_nt", ops, D_ref, M, N, K)
        assert rc == 0, cfg_ref
        rc, cfg = abi_call("fp8gemm_nt_noalloc", ops, D, M, N, K)
        assert rc == 0, cfg
        torch.cuda.synchronize()
        assert split_of(cfg) > 1, cfg                      # the scratch is used
        assert cfg == cfg_ref, (cfg, cfg_ref)
        got = gpu_bits(D)
        assert np.array_equal(got, gpu_bits(D_ref)), "noalloc differs from fp8gemm_nt (%s)" % cfg
        rep = assert_close(got, oracle.gemm_nt(d.A, d.sa, d.B, d.sb), what=cfg)
        assert fg.read_device_error() == 0
        say("noalloc", M, N, K, cfg, rep["bit_equal"])


def test_noalloc_refuses_launches_beyond_the_scratch():
    """A forced launch shape whose partials exceed the static scratch (16 MiB): 32 tiles of
    128 x 128 x 16 K splits = 32 MiB.  Refused on the host, D untouched; fp8gemm_nt takes it."""
    M, N, K = 128, 4096, 2048
    d = W.dense(M, N, K, seed=603)
    ops = (dev(d.A), dev(np.swapaxes(d.sa, 0, 1)), dev(d.B), dev(d.sb))
    D = torch.full((M, N), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    os.environ["FP8GEMM_FORCE_CONFIG"] = "128x128:2x4:3:16"
    try:
        rc, _ = abi_call("fp8gemm_nt_noalloc", ops, D, M, N, K)
        assert rc == 4                                     # FP8GEMM_ERR_UNSUPPORTED
        torch.cuda.synchronize()
        assert np.all(gpu_bits(D) == SENTINEL)
        rc, cfg = abi_call("fp8gemm_nt", ops, D, M, N, K)
        assert rc == 0 and split_of(cfg) == 16, cfg
    finally:
        os.environ.pop("FP8GEMM_FORCE_CONFIG", None)
    torch.cuda.synchronize()
    assert_close(gpu_bits(D), oracle.gemm_nt(d.A, d.sa, d.B, d.sb), what=cfg)
