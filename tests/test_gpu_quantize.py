"""GPU parity of the 1x128 activation quantiser (HIP library through its C ABI) against the CPU
oracle: codes and scales bit-exact, on ragged shapes, every bf16 value of the E4M3 range, the
masked layout, the full-size activation matrix, and the quantiser feeding the GEMM."""
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

CODE_SENTINEL = 0x7F      # the E4M3 NaN code: never written by the quantiser
SCALE_SENTINEL = -1.0     # scales are positive


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def host_codes(t):
    return t.view(torch.uint8).cpu().numpy()


def quantize_gpu(bits):
    M, K = bits.shape
    codes = torch.full((M, K), CODE_SENTINEL, dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
    scales = torch.full((K // 128, M), SCALE_SENTINEL, dtype=torch.float32, device="cuda")
    fg.quantize_1x128(dev_bf16(bits), codes=codes, scales=scales)
    torch.cuda.synchronize()
    return host_codes(codes), scales.cpu().numpy().T


def assert_quant_equal(bits, what):
    codes, sa = quantize_gpu(bits)
    ref_codes, ref_sa = oracle.quantize_1x128(bits)
    bad = np.argwhere(codes != ref_codes)
    assert bad.size == 0, "%s: %d codes differ, first %s: gpu %#x oracle %#x (x bits %#06x)" % (
        what, len(bad), bad[0], codes[tuple(bad[0])], ref_codes[tuple(bad[0])], bits[tuple(bad[0])])
    bad = np.argwhere(sa.view(np.uint32) != ref_sa.view(np.uint32))
    assert bad.size == 0, "%s: %d scales differ, first %s: gpu %r oracle %r" % (
        what, len(bad), bad[0], sa[tuple(bad[0])], ref_sa[tuple(bad[0])])
    return codes, sa


@pytest.mark.parametrize("M,K", [(1, 128), (3, 256), (16, 512), (17, 640), (37, 640), (100, 1152),
                                 (257, 384), (1000, 2048)])
def test_quantize_bit_exact_ragged(M, K):
    """Row counts off the 16-row workgroup tile, K-block counts off the 4-block tile; blocks of
    magnitudes 2^-60..2^60, zero blocks, bf16 subnormals and signed zeros."""
    say("quantize", M, K)
    assert_quant_equal(W.stress_bf16(M, K, seed=M * 7 + K), "stress %dx%d" % (M, K))
    assert_quant_equal(W.activations_bf16(M, K, seed=M + K), "activations %dx%d" % (M, K))
    assert fg.last_config().startswith("quantize_1x128")


def test_every_bf16_value_of_the_e4m3_range():
    """Each block starts with 448 (so its scale is exactly 1 and x/s = x), followed by every bf16
    value of magnitude at most 448, both signs: the hardware conversion against the oracle's
    encoder on every rounding case, subnormals and ties included."""
    pos = np.arange(0, 0x43E1, dtype=np.uint16)              # +0 .. 448 (0x43E0)
    vals = np.concatenate([pos, pos | np.uint16(0x8000)])
    per = 127
    nblk = -(-vals.size // per)
    body = np.zeros(nblk * per, dtype=np.uint16)
    body[:vals.size] = vals
    bits = np.concatenate([np.full((nblk, 1), 0x43E0, np.uint16), body.reshape(nblk, per)], axis=1)
    say("all bf16 values", bits.shape)
    codes, sa = assert_quant_equal(bits, "all bf16 values in [-448, 448]")
    assert np.all(sa == 1.0)


def test_extreme_magnitudes():
    """Largest finite bf16 values, blocks of only subnormals, blocks just under and over the
    amax floor, single nonzero element blocks."""
    rng = np.random.default_rng(7)
    rows = []
    big = np.full(128, 0x7F7F, np.uint16)                     # largest finite bf16
    big[1::2] |= 0x8000
    rows.append(big)
    rows.append(rng.integers(1, 0x80, size=128).astype(np.uint16))              # subnormals
    for v in (9.9e-5, 1e-4, 1.01e-4, 3e-3):
        x = (rng.standard_normal(128) * v / 4).astype(np.float32)
        x[5] = v
        rows.append(W.bf16_bits(x))
    one = np.zeros(128, np.uint16)
    one[77] = W.bf16_bits(np.array([-3.0e-20], np.float32))[0]
    rows.append(one)
    bits = np.stack(rows)
    assert_quant_equal(bits, "extreme magnitudes")


def test_quantize_deterministic_and_respects_bounds():
    """Two calls give the same bits; nothing outside the outputs is written (guard bands)."""
    M, K = 33, 896
    bits = W.stress_bf16(M, K, seed=11)
    X = dev_bf16(bits)
    pad = 4096
    codes_buf = torch.full((M * K + 2 * pad,), CODE_SENTINEL, dtype=torch.uint8, device="cuda")
    sa_buf = torch.full(((K // 128) * M + 2 * pad,), SCALE_SENTINEL, dtype=torch.float32, device="cuda")
    codes = codes_buf[pad:pad + M * K].view(M, K).view(torch.float8_e4m3fn)
    scales = sa_buf[pad:pad + (K // 128) * M].view(K // 128, M)
    outs = []
    for _ in range(2):
        fg.quantize_1x128(X, codes=codes, scales=scales)
        torch.cuda.synchronize()
        outs.append((host_codes(codes).copy(), scales.cpu().numpy().copy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    cb, sb = codes_buf.cpu().numpy(), sa_buf.cpu().numpy()
    assert np.all(cb[:pad] == CODE_SENTINEL) and np.all(cb[pad + M * K:] == CODE_SENTINEL)
    assert np.all(sb[:pad] == SCALE_SENTINEL) and np.all(sb[pad + (K // 128) * M:] == SCALE_SENTINEL)
    ref_codes, ref_sa = oracle.quantize_1x128(bits)
    assert np.array_equal(outs[0][0], ref_codes) and np.array_equal(outs[0][1].T, ref_sa)


@pytest.mark.parametrize("mm,M_max,K", [([0, 1, 64, 200, 130], 200, 384), ([16, 15], 16, 128),
                                        ([256] * 3, 256, 1024)])
def test_quantize_masked_rows_past_count_untouched(mm, M_max, K):
    G = len(mm)
    bits = W.stress_bf16(G * M_max, K, seed=G * 100 + K).reshape(G, M_max, K)
    masked_m = torch.tensor(mm, dtype=torch.int32, device="cuda")
    codes = torch.full((G, M_max, K), CODE_SENTINEL, dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
    scales = torch.full((G, K // 128, M_max), SCALE_SENTINEL, dtype=torch.float32, device="cuda")
    fg.quantize_1x128_masked(dev_bf16(bits), masked_m, codes=codes, scales=scales)
    got_c = host_codes(codes)
    got_s = np.swapaxes(scales.cpu().numpy(), 1, 2)
    ref_c, ref_s = oracle.quantize_1x128(bits.reshape(G * M_max, K))
    ref_c, ref_s = ref_c.reshape(G, M_max, K), ref_s.reshape(G, M_max, K // 128)
    for g, c in enumerate(mm):
        assert np.array_equal(got_c[g, :c], ref_c[g, :c]), g
        assert np.array_equal(got_s[g, :c].view(np.uint32), ref_s[g, :c].view(np.uint32)), g
        assert np.all(got_c[g, c:] == CODE_SENTINEL) and np.all(got_s[g, c:] == SCALE_SENTINEL), g
    assert fg.read_device_error() == 0
    say("quantize masked", mm, fg.last_config())


def test_quantize_masked_count_out_of_range_clamps_and_flags():
    G, M_max, K = 3, 32, 256
    bits = W.stress_bf16(G * M_max, K, seed=5).reshape(G, M_max, K)
    masked_m = torch.tensor([40, -2, 7], dtype=torch.int32, device="cuda")
    codes, scales = fg.quantize_1x128_masked(dev_bf16(bits), masked_m)
    assert fg.read_device_error() == fg.DEVERR_BAD_COUNT
    ref_c, _ = oracle.quantize_1x128(bits.reshape(G * M_max, K))
    got = host_codes(codes).reshape(G * M_max, K)
    assert np.array_equal(got[:M_max], ref_c[:M_max])               # 40 clamped to M_max
    assert np.all(got[M_max:2 * M_max] == 0)                          # -2 taken as 0: untouched
    assert np.array_equal(got[2 * M_max:2 * M_max + 7], ref_c[2 * M_max:2 * M_max + 7])
    assert fg.read_device_error() == 0


def test_quantize_then_gemm_end_to_end():
    """bf16 activations -> GPU quantiser -> GPU GEMM (dense and contiguous) against oracle
    quantiser -> oracle GEMM, within the GEMM's tolerance."""
    M, N, K = 300, 384, 1024
    bits = W.activations_bf16(M, K, seed=21)
    rng = np.random.default_rng(22)
    Bq, sb = W.quantize_128x128(W.normal(rng, (N, K)))
    codes, scales = fg.quantize_1x128(dev_bf16(bits))
    D = fg.gemm_nt(codes, scales, torch.from_numpy(Bq).cuda(), torch.from_numpy(sb).cuda())
    ref_codes, ref_sa = oracle.quantize_1x128(bits)
    ref = oracle.gemm_nt(ref_codes, ref_sa, Bq, sb)
    assert_close(gpu_bits(D), ref, what="quantise -> gemm_nt")
    # contiguous: two groups, the second half padded
    G = 2
    Bg = np.stack([Bq, Bq[::-1].copy()])
    sbg = np.stack([sb, sb[::-1].copy()])
    m_idx = np.repeat(np.array([0, 1], np.int32), [128, M - 128])
    m_idx[256:] = -1
    Dc = fg.grouped_contiguous(codes, scales, torch.from_numpy(Bg).cuda(), torch.from_numpy(sbg).cuda(),
                               torch.from_numpy(m_idx).cuda())
    refc, valid = oracle.grouped_contiguous(ref_codes, ref_sa, Bg, sbg, m_idx)
    v = valid.astype(bool)
    assert_close(gpu_bits(Dc), refc, mask=np.broadcast_to(v[:, None], refc.shape), what="quantise -> contiguous")
    assert G == Bg.shape[0] and fg.read_device_error() == 0


def test_full_size_activation_matrix():
    """The benchmark's activation matrix (32768 x 7168), every code and scale against the oracle."""
    M, K = W.QUANT_M, W.QUANT_K
    say("full-size quantiser", M, K)
    bits = W.activations_bf16(M, K, seed=31)
    assert_quant_equal(bits, "full size %dx%d" % (M, K))
