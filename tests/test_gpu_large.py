"""GPU: operands larger than 4 GiB, so that every address past the first 2^32 bytes of A, of its
scales and of D is formed with 64-bit arithmetic.  A is 1,048,613 x 4352 E4M3 codes (4.56 GB,
random codes without the NaN patterns, drawn on the device), B a quantised N(0,1) weight with a
ragged N.  Sampled rows -- the first ones, rows on both sides of the 4 GiB offset of A, the last
ones -- are checked against the oracle with the GEMM tolerance; the rows past the end of D are
checked untouched."""
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


def test_dense_a_past_4gib():
    M, N, K = (1 << 20) + 37, 136, 4352
    assert M * K > (1 << 32)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2024)
    A = torch.randint(0, 256, (M, K), dtype=torch.uint8, device="cuda", generator=gen)
    A = torch.where((A & 0x7F) == 0x7F, A ^ 1, A)          # 0x7F / 0xFF (NaN) -> 0x7E / 0xFE
    sa = torch.rand((K // 128, M), device="cuda", generator=gen) * 0.01 + 0.001
    rng = np.random.default_rng(2025)
    Bq, sb = W.quantize_128x128(W.normal(rng, (N, K)))
    B = torch.from_numpy(Bq).cuda()
    sbd = torch.from_numpy(sb).cuda()
    # D with a guard band of sentinels after it
    pad = 4096
    buf = torch.full((M * N + pad,), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    D = buf[:M * N].view(M, N)
    fg.gemm_nt(A.view(torch.float8_e4m3fn), sa, B.view(torch.float8_e4m3fn), sbd, out=D)
    torch.cuda.synchronize()
    cfg = fg.last_config()
    assert fg.read_device_error() == 0
    edge = (1 << 32) // K                                  # first row of A at or past byte 2^32
    rows = np.unique(np.concatenate([np.arange(8), np.arange(edge - 8, edge + 8), np.arange(M - 40, M),
                                     rng.integers(0, M, size=16)]))
    idx = torch.from_numpy(rows).cuda()
    a_rows = A.index_select(0, idx).cpu().numpy()
    sa_rows = sa.index_select(1, idx).cpu().numpy().T       # [rows, K/128], as the oracle takes it
    ref = oracle.gemm_nt(a_rows, np.ascontiguousarray(sa_rows), Bq, sb)
    got = gpu_bits(D.index_select(0, idx))
    assert_close(got, ref, what="rows %d..%d of %d (%s)" % (rows[0], rows[-1], M, cfg))
    tail = gpu_bits(buf[M * N:])
    assert np.all(tail == np.uint16(SENTINEL)), "write past the end of D"
    say("large dense", M, N, K, cfg)


def test_masked_b_past_4gib():
    """Masked layout on the masked decode kernel with B at 40 x 7168 x 16384 E4M3 codes (4.70 GB):
    the groups whose weights start past byte 2^32 of B are checked against the oracle."""
    G, M_max, N, K = 40, 16, 7168, 16384
    assert G * N * K > (1 << 32)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2026)
    B = torch.randint(0, 256, (G, N, K), dtype=torch.uint8, device="cuda", generator=gen)
    B = torch.where((B & 0x7F) == 0x7F, B ^ 1, B)
    sb = torch.rand((G, N // 128, K // 128), device="cuda", generator=gen) * 0.01 + 0.001
    rng = np.random.default_rng(2027)
    mm = rng.integers(0, M_max + 1, size=G).astype(np.int32)
    mm[-1] = M_max
    Aq, sa = W.acts(rng, G * M_max, K)
    Aq = Aq.reshape(G, M_max, K)
    sa = sa.reshape(G, M_max, K // 128)
    A = torch.from_numpy(Aq).cuda()
    sad = torch.from_numpy(np.ascontiguousarray(np.swapaxes(sa, -1, -2))).cuda()
    D = torch.full((G, M_max, N), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    fg.grouped_masked(A.view(torch.float8_e4m3fn), sad, B.view(torch.float8_e4m3fn), sb,
                      torch.from_numpy(mm).cuda(), 8, out=D)
    torch.cuda.synchronize()
    cfg = fg.last_config()
    assert fg.read_device_error() == 0
    first_past = -(-(1 << 32) // (N * K))                  # first group whose B starts at or past byte 2^32
    groups = [0, first_past - 1, first_past, G - 1]
    for g in groups:
        c = int(mm[g])
        got = gpu_bits(D[g])
        assert np.all(got[c:] == np.uint16(SENTINEL)), "group %d: rows past the count written" % g
        if c == 0:
            continue
        ref, _ = oracle.grouped_masked(Aq[g:g + 1], sa[g:g + 1], B[g:g + 1].cpu().numpy(), sb[g:g + 1].cpu().numpy(),
                                       mm[g:g + 1])
        assert_close(got[None, :c], ref[:, :c], what="group %d (%s)" % (g, cfg))
    say("large masked", G, M_max, N, K, groups, mm[groups].tolist(), cfg)
