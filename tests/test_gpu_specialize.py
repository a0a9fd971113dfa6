"""GPU: the run-time specialised dense kernel (N and K compiled in) against the ahead-of-time kernel
and the CPU oracle.  The two kernels share their body and arithmetic order, so with the same
schedule (whole tiles: the specialised kernels take no stream-K) their outputs must be identical
bit for bit on every shape; the oracle comparison uses the GEMM tolerance
|gpu - ref| <= 2^-7 |ref| + 1e-3 rms(ref)."""
import os
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


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def operands(M, N, K, seed):
    rng = np.random.default_rng(seed)
    Bq, sb = W.quantize_128x128(W.normal(rng, (N, K)))
    Aq, sa = W.acts(rng, M, K)
    return Aq, sa, Bq, sb


def run_both(Aq, sa, Bq, sb):
    """The table kernel and the specialised one on the same operands.  The specialised kernels
    keep whole tiles, so the table kernel runs with stream-K off here (with it, its leftover
    tiles sum their K blocks in another order)."""
    A, S, B, SB = dev(Aq), dev(np.ascontiguousarray(sa.T)), dev(Bq), dev(sb)
    os.environ["FP8GEMM_STREAMK"] = "0"
    try:
        d0 = fg.gemm_nt(A, S, B, SB)
        torch.cuda.synchronize()
        c0 = fg.last_config()
    finally:
        os.environ.pop("FP8GEMM_STREAMK", None)
    d1 = fg.gemm_nt_specialized(A, S, B, SB)
    torch.cuda.synchronize()
    c1 = fg.last_config()
    return gpu_bits(d0), gpu_bits(d1), c0, c1


@pytest.mark.parametrize("M,N,K", [(256, 512, 1024), (300, 1000, 384), (64, 2112, 7168), (128, 7168, 2048),
                                   (1000, 4096, 512), (4096, 2112, 1024), (2048, 4096, 2048), (17, 96, 128)])
def test_specialized_equals_table_kernel(M, N, K):
    """Every regime of the table: decode tiles with split-K, 128x128 tiles, the prefill tiles
    (256x160 for N = 2112), ragged M and N tails, K of one block."""
    Aq, sa, Bq, sb = operands(M, N, K, seed=M + N + K)
    b0, b1, c0, c1 = run_both(Aq, sa, Bq, sb)
    assert "specialized" in c1 and c1.replace(" specialized", "") == c0, (c0, c1)
    assert np.array_equal(b0, b1), "%s: %d outputs differ" % (c1, int((b0 != b1).sum()))
    say("specialized", M, N, K, c1)


def test_specialized_config0_parity_with_oracle():
    d = W.config0()
    A, S, B, SB = dev(d.A), dev(np.ascontiguousarray(d.sa.T)), dev(d.B), dev(d.sb)
    D = fg.gemm_nt_specialized(A, S, B, SB)
    ref = oracle.gemm_nt(d.A, d.sa, d.B, d.sb)
    assert_close(gpu_bits(D), ref, what="specialized config 0")


def test_specialize_ahead_caches_per_shape():
    before = fg.specialized_count()
    ms = fg.specialize_nt(512, 1536, 2560)
    assert ms > 0 and fg.specialized_count() == before + 1
    assert fg.specialize_nt(512, 1536, 2560) == 0.0 and fg.specialized_count() == before + 1
    # same launch shape and N, K from another M: the same kernel
    assert fg.specialize_nt(500, 1536, 2560) == 0.0
    Aq, sa, Bq, sb = operands(512, 1536, 2560, seed=9)
    b0, b1, _, c1 = run_both(Aq, sa, Bq, sb)
    assert fg.specialized_count() == before + 1, c1
    assert np.array_equal(b0, b1)
    say("specialize ahead: %.1f ms" % ms)


def test_specialized_side_stream_and_graph_replay():
    """A call enqueued on a side stream, and a captured graph of the specialised launch (the kernel
    is built before capture) replayed several times with eager work between the replays."""
    M, N, K = 1024, 2048, 1024
    Aq, sa, Bq, sb = operands(M, N, K, seed=5)
    A, S, B, SB = dev(Aq), dev(np.ascontiguousarray(sa.T)), dev(Bq), dev(sb)
    os.environ["FP8GEMM_STREAMK"] = "0"      # the specialised kernels keep whole tiles
    try:
        ref = gpu_bits(fg.gemm_nt(A, S, B, SB))
    finally:
        os.environ.pop("FP8GEMM_STREAMK", None)
    fg.specialize_nt(M, N, K)
    s = torch.cuda.Stream()
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    with torch.cuda.stream(s):
        fg.gemm_nt_specialized(A, S, B, SB, out=out, stream=s)
    s.synchronize()
    assert np.array_equal(gpu_bits(out), ref)
    g = torch.cuda.CUDAGraph()
    out2 = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    with torch.cuda.graph(g, stream=s):
        fg.gemm_nt_specialized(A, S, B, SB, out=out2, stream=s)
    for r in range(3):
        out2.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(gpu_bits(out2), ref), "replay %d" % r


@pytest.mark.slow
@pytest.mark.parametrize("nki", range(len(W.SWEEP_NK)))
def test_specialized_sweep_m4096_equals_table_kernel(nki):
    """The prefill sweep shapes at M = 4096, in the launch configuration the benchmark times."""
    N, K = W.SWEEP_NK[nki]
    mi = W.SWEEP_M.index(4096)
    d = W.sweep_case(mi, nki)
    b0, b1, c0, c1 = run_both(d.A, d.sa, d.B, d.sb)
    assert np.array_equal(b0, b1), "%s: %d outputs differ" % (c1, int((b0 != b1).sum()))
    say("specialized sweep", N, K, c1)
