"""Pins for the CPU oracle: facts fixed by the number formats and by mathematics, checked against
implementations that share nothing with the oracle (exact rationals, torch's format casts and
fp64 matmul, closed forms, invariants).  CPU only."""
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as W

# ------------------------------------------------------------------------------------------
# independent helpers: exact rational arithmetic and torch's casts
# ------------------------------------------------------------------------------------------

_DEC = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float().numpy()


def frac_of_code(c: int) -> Fraction:
    return Fraction(float(_DEC[c]))


def exact_bf16_bits(x: Fraction) -> int:
    """Round an exact rational to bf16 (round half to even), by rational arithmetic only."""
    if x == 0:
        return 0
    sign = 0x8000 if x < 0 else 0
    ax = abs(x)
    e = ax.numerator.bit_length() - ax.denominator.bit_length()
    while Fraction(2) ** e > ax:
        e -= 1
    while Fraction(2) ** (e + 1) <= ax:
        e += 1
    q = Fraction(2) ** (max(e, -126) - 7)
    n = ax / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * q
    if v >= Fraction(2) ** 128:
        return sign | 0x7F80
    bits = struct.unpack("<I", struct.pack("<f", float(v)))[0]
    return sign | (bits >> 16)


def bf16_tie_distance(x: Fraction) -> Fraction:
    """Relative distance from x to the nearest bf16 rounding boundary (midpoint)."""
    if x == 0:
        return Fraction(1)
    ax = abs(x)
    e = ax.numerator.bit_length() - ax.denominator.bit_length()
    while Fraction(2) ** e > ax:
        e -= 1
    while Fraction(2) ** (e + 1) <= ax:
        e += 1
    q = Fraction(2) ** (max(e, -126) - 7)
    n = ax / q
    frac = n - (n.numerator // n.denominator)
    return abs(frac - Fraction(1, 2)) * q / ax


def exact_gemm(A, sa, B, sb):
    """Exact rational dequantised product, sum_k (sa*dec(a)) * (sb*dec(b)), per output."""
    M, K = A.shape
    N = B.shape[0]
    out = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            s = Fraction(0)
            for k in range(K):
                s += (Fraction(float(sa[m, k // 128])) * frac_of_code(A[m, k]) *
                      Fraction(float(sb[n // 128, k // 128])) * frac_of_code(B[n, k]))
            out[m][n] = s
    return out


def code_of(v: float) -> int:
    return int(torch.tensor([v], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)[0])


# ------------------------------------------------------------------------------------------
# element formats
# ------------------------------------------------------------------------------------------

def _read_golden(path):
    rows = []
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line)
    return rows


def test_e4m3_anchors(golden_dir):
    rows = _read_golden(os.path.join(golden_dir, "e4m3_anchors.txt"))
    assert len(rows) >= 15
    for row in rows:
        code, val = row.split()
        got = oracle.e4m3_value(int(code, 16))
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), (code, got)


def test_e4m3_all_codes_match_library_decoder():
    for c in range(256):
        got, ref = oracle.e4m3_value(c), float(_DEC[c])
        if math.isnan(ref):
            assert math.isnan(got), c
        else:
            assert got == ref and math.copysign(1, got) == math.copysign(1, ref), (c, got, ref)


def test_bf16_golden_cases(golden_dir):
    rows = _read_golden(os.path.join(golden_dir, "bf16_rne.txt"))
    for row in rows:
        parts = row.split()
        hexpos = next(i for i, p in enumerate(parts) if p.startswith("0x"))
        x = float(eval(" ".join(parts[:hexpos]), {"__builtins__": {}}))
        want = int(parts[hexpos], 16)
        assert oracle.bf16_bits(x) == want, (row, hex(oracle.bf16_bits(x)))
    assert oracle.bf16_bits(float("nan")) == 0x7FC0


def test_bf16_matches_library_cast_on_fp32_values():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2**32, size=20000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    got = np.array([oracle.bf16_bits(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_single_rounding_against_exact_rationals():
    rng = np.random.default_rng(8)
    for _ in range(3000):
        m = int(rng.integers(1, 2**53))
        e = int(rng.integers(-190, 120))
        x = math.ldexp(m, e - 53) * (1 if rng.random() < 0.5 else -1)
        assert oracle.bf16_bits(x) == exact_bf16_bits(Fraction(x)), x


# ------------------------------------------------------------------------------------------
# whole products
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K,seed", [(3, 5, 128, 1), (4, 3, 256, 2), (2, 7, 384, 3), (5, 4, 200, 4),
                                        (1, 130, 128, 5)])
def test_brute_force_exact_rationals(M, N, K, seed):
    """Random codes over all non-NaN values (subnormals and +-448 included) and random scales:
    the oracle must equal the exactly rounded exact product, bit for bit."""
    rng = np.random.default_rng(seed)
    A = W.random_codes(rng, (M, K))
    B = W.random_codes(rng, (N, K))
    nkb, nnb = -(-K // 128), -(-N // 128)
    sa = np.exp(rng.standard_normal((M, nkb))).astype(np.float32)
    sb = np.exp(rng.standard_normal((nnb, nkb))).astype(np.float32) * np.float32(1e-3)
    D, acc = oracle.gemm_nt(A, sa, B, sb, with_acc=True)
    ex = exact_gemm(A, sa, B, sb)
    for m in range(M):
        for n in range(N):
            assert bf16_tie_distance(ex[m][n]) > Fraction(1, 10**12)  # no near-tie in these draws
            assert int(D[m, n]) == exact_bf16_bits(ex[m][n]), (m, n)
            assert abs(Fraction(acc[m, n]) - ex[m][n]) <= abs(ex[m][n]) * Fraction(1, 2**48) + Fraction(1, 2**200)


def test_integer_closed_forms():
    """Unit scales and small-integer codes: D[m][n] = K * a_m * b_n exactly."""
    one = np.float32(1.0)
    for K in (128, 256, 640):
        a_vals = np.array([-4, -3, -2, -1, 0, 1, 2, 3, 4], dtype=np.float32)
        b_vals = np.array([4, -3, 1, 2, 0, -1, 3], dtype=np.float32)
        A = np.array([[code_of(v)] * K for v in a_vals], dtype=np.uint8)
        B = np.array([[code_of(v)] * K for v in b_vals], dtype=np.uint8)
        sa = np.full((len(a_vals), K // 128), one, dtype=np.float32)
        sb = np.full((1, K // 128), one, dtype=np.float32)
        D = oracle.gemm_nt(A, sa, B, sb)
        want = (K * np.outer(a_vals, b_vals)).astype(np.float32)
        got = oracle.bf16_bits_to_float(D)
        assert np.array_equal(got, want)
    # all ones: D = K
    for K in (128, 1024, 7168):
        A = np.full((2, K), 0x38, dtype=np.uint8)
        B = np.full((3, K), 0x38, dtype=np.uint8)
        D = oracle.gemm_nt(A, np.ones((2, K // 128), np.float32), B, np.ones((1, K // 128), np.float32))
        assert np.all(oracle.bf16_bits_to_float(D) == np.float32(K)) or K > 256 * 256


def test_integer_rne_golden(golden_dir):
    rows = _read_golden(os.path.join(golden_dir, "gemm_integer_rne.txt"))
    for row in rows:
        K, fours, extra, want = row.split()
        K, fours, extra, want = int(K), int(fours), int(extra), float(want)
        a = np.zeros((1, K), dtype=np.uint8)
        a[0, :fours] = code_of(4.0)
        a[0, fours] = code_of(float(extra))
        B = np.full((5, K), code_of(1.0), dtype=np.uint8)
        D = oracle.gemm_nt(a, np.ones((1, K // 128), np.float32), B, np.ones((1, K // 128), np.float32))
        assert np.all(oracle.bf16_bits_to_float(D) == np.float32(want)), row


def test_power_of_two_scale_indexing_closed_form():
    """A and B all ones, power-of-two scales: D[m][n] = 128 * sum_kb sa[m][kb] * sb[n // 128][kb],
    exact.  Catches a wrong K-block or N-block index (N=300 has a partial third block)."""
    M, N, K = 6, 300, 640
    nkb, nnb = K // 128, -(-N // 128)
    sa = np.array([[2.0 ** ((m + kb) % 5 - 2) for kb in range(nkb)] for m in range(M)], np.float32)
    sb = np.array([[2.0 ** ((nb + 2 * kb) % 3 - 1) for kb in range(nkb)] for nb in range(nnb)], np.float32)
    A = np.full((M, K), 0x38, np.uint8)
    B = np.full((N, K), 0x38, np.uint8)
    D = oracle.gemm_nt(A, sa, B, sb)
    want = np.array([[128 * sum(sa[m, kb] * sb[n // 128, kb] for kb in range(nkb)) for n in range(N)]
                     for m in range(M)], np.float32)
    assert np.array_equal(oracle.bf16_bits_to_float(D), want)


def test_matches_library_fp64_matmul_of_dequantised_operands():
    """Special case reducing to a library routine: dequantise with torch's decoder and block
    expansion, multiply with torch's fp64 matmul (A . B^T), compare with the oracle's fp64 value."""
    rng = np.random.default_rng(11)
    M, N, K = 37, 200, 384
    d = W.dense(M, N, K, seed=11)
    Af = torch.from_numpy(d.A).view(torch.float8_e4m3fn).double() * torch.from_numpy(d.sa).double().repeat_interleave(128, 1)
    Bf = torch.from_numpy(d.B).view(torch.float8_e4m3fn).double() * \
        torch.from_numpy(d.sb).double().repeat_interleave(128, 0)[:N].repeat_interleave(128, 1)
    ref = (Af @ Bf.T).numpy()
    D, acc = oracle.gemm_nt(d.A, d.sa, d.B, d.sb, with_acc=True)
    bound = (Af.abs() @ Bf.abs().T).numpy() * 1e-13
    assert np.all(np.abs(acc - ref) <= bound)
    rb = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    # fp64 -> fp32 -> bf16 can double-round only at a near-tie; with these draws there are none
    assert np.mean(D == rb) > 0.9999
    del rng


# ------------------------------------------------------------------------------------------
# invariants of the grouped layouts
# ------------------------------------------------------------------------------------------

def test_row_permutation():
    d = W.dense(50, 70, 256, seed=21)
    perm = np.random.default_rng(21).permutation(50)
    D = oracle.gemm_nt(d.A, d.sa, d.B, d.sb)
    Dp = oracle.gemm_nt(d.A[perm], d.sa[perm], d.B, d.sb)
    assert np.array_equal(Dp, D[perm])


def test_scale_linearity():
    d = W.dense(8, 140, 256, seed=22)
    D = oracle.gemm_nt(d.A, d.sa, d.B, d.sb)
    sa2 = d.sa.copy()
    sa2[3] *= 2
    sb2 = d.sb.copy()
    sb2[1] *= 4
    D2 = oracle.gemm_nt(d.A, sa2, d.B, sb2)
    f, f2 = oracle.bf16_bits_to_float(D), oracle.bf16_bits_to_float(D2)
    scale = np.ones_like(f)
    scale[3] *= 2
    scale[:, 128:] *= 4
    assert np.array_equal(f2, f * scale)


def test_contiguous_equals_per_group_dense_and_ignores_padding():
    c = W.contiguous([100, 0, 130, 7], 256, 96, 256, seed=23, packed=True)
    D, valid = oracle.grouped_contiguous(c.A, c.sa, c.B, c.sb, c.m_indices)
    assert np.array_equal(valid.astype(bool), c.m_indices >= 0)
    for g in range(4):
        rows = np.nonzero(c.m_indices == g)[0]
        if rows.size:
            Dg = oracle.gemm_nt(c.A[rows], c.sa[rows], c.B[g], c.sb[g])
            assert np.array_equal(D[rows], Dg)
    # refill the padding rows: valid rows unchanged
    A2, sa2 = c.A.copy(), c.sa.copy()
    pad = c.m_indices < 0
    rng = np.random.default_rng(5)
    A2[pad] = W.random_codes(rng, (int(pad.sum()), A2.shape[1]))
    sa2[pad] = rng.random((int(pad.sum()), sa2.shape[1]), dtype=np.float32) + 1
    D2, _ = oracle.grouped_contiguous(A2, sa2, c.B, c.sb, c.m_indices)
    assert np.array_equal(D2[~pad], D[~pad])
    # an index outside [-1, G) is padding too
    mi = c.m_indices.copy()
    mi[0] = 4
    mi[1] = -7
    D3, v3 = oracle.grouped_contiguous(c.A, c.sa, c.B, c.sb, mi)
    assert v3[0] == 0 and v3[1] == 0 and np.array_equal(D3[2:][v3[2:] == 1], D[2:][v3[2:] == 1])


def test_masked_equals_per_group_dense_and_ignores_rows_past_count():
    mm = np.array([5, 0, 64, 3], np.int32)
    w = W.masked(mm, 64, 130, 256, seed=24)
    D, valid = oracle.grouped_masked(w.A, w.sa, w.B, w.sb, w.masked_m)
    for g in range(4):
        assert np.array_equal(valid[g], (np.arange(64) < mm[g]).astype(np.uint8))
        if mm[g]:
            Dg = oracle.gemm_nt(w.A[g, :mm[g]], w.sa[g, :mm[g]], w.B[g], w.sb[g])
            assert np.array_equal(D[g, :mm[g]], Dg)
    A2 = w.A.copy()
    A2[0, 5:] = W.random_codes(np.random.default_rng(9), (59, 256))
    D2, _ = oracle.grouped_masked(A2, w.sa, w.B, w.sb, w.masked_m)
    assert np.array_equal(D2[valid == 1], D[valid == 1])
    # counts outside [0, M_max] clamp
    D3, v3 = oracle.grouped_masked(w.A, w.sa, w.B, w.sb, np.array([-2, 0, 1000, 3], np.int32))
    assert v3[0].sum() == 0 and v3[2].sum() == 64 and np.array_equal(D3[2], D[2])


def test_contiguous_equals_concatenated_masked():
    """The same groups in both grouped layouts give the same valid outputs."""
    mm = np.array([40, 128, 1], np.int32)
    w = W.masked(mm, 128, 64, 128, seed=25)
    Ac = np.concatenate([w.A[g] for g in range(3)])
    sac = np.concatenate([w.sa[g] for g in range(3)])
    mi = np.concatenate([np.where(np.arange(128) < mm[g], g, -1) for g in range(3)]).astype(np.int32)
    Dm, vm = oracle.grouped_masked(w.A, w.sa, w.B, w.sb, mm)
    Dc, vc = oracle.grouped_contiguous(Ac, sac, w.B, w.sb, mi)
    assert np.array_equal(vm.reshape(-1), vc)
    assert np.array_equal(Dm.reshape(-1, 64)[vc == 1], Dc[vc == 1])


def test_elements_match_full_results():
    d = W.dense(33, 260, 384, seed=26)
    D = oracle.gemm_nt(d.A, d.sa, d.B, d.sb)
    rng = np.random.default_rng(26)
    r = rng.integers(0, 33, 500)
    c = rng.integers(0, 260, 500)
    got = oracle.elements(d.A, d.sa, d.B, d.sb, r, c, c // 128)
    assert np.array_equal(got, D[r, c])
    # grouped: flattened B rows g*N + n, sb rows g*ceil(N/128) + n//128
    w = W.masked(np.array([7, 9], np.int32), 16, 200, 256, seed=27)
    Dm, vm = oracle.grouped_masked(w.A, w.sa, w.B, w.sb, w.masked_m)
    g = np.array([0, 1, 1, 0]); rr = np.array([0, 8, 3, 6]); n = np.array([0, 199, 128, 77])
    got = oracle.elements(w.A.reshape(-1, 256), w.sa.reshape(-1, 2), w.B.reshape(-1, 256),
                          w.sb.reshape(-1, 2), g * 16 + rr, g * 200 + n, g * 2 + n // 128)
    assert np.array_equal(got, Dm[g, rr, n])


def test_quantiser_block_max_is_448():
    """Input recipe check: every quantised block holds a code of magnitude 448 (its amax)."""
    d = W.dense(64, 300, 512, seed=28)
    a = torch.from_numpy(d.A).view(torch.float8_e4m3fn).float().abs()
    assert torch.all(a.view(64, 4, 128).amax(-1) == 448)
    b = torch.from_numpy(d.B).view(torch.float8_e4m3fn).float().abs()
    for nb in range(3):
        blk = b[nb * 128:(nb + 1) * 128].view(-1, 4, 128).amax(dim=(0, 2))
        assert torch.all(blk == 448)
