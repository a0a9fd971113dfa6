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


# ------------------------------------------------------------------------------------------
# activation quantiser, 1x128 blocks
# ------------------------------------------------------------------------------------------

FLOOR = np.float32(1e-4)


def bf16_bits_exact(x) -> np.ndarray:
    """fp32 values that bf16 holds exactly -> their bf16 bit patterns (the top half of fp32)."""
    b = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "value not exact in bf16"
    return (b >> 16).astype(np.uint16)


def widen(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def test_e4m3_encoder_matches_library_cast_at_every_boundary():
    """Every E4M3 value and every rounding midpoint, with their two nearest fp32 neighbours on
    each side, plus log-uniform values, both signs: the oracle's encoder against torch's cast."""
    vals = _DEC[:0x7F].astype(np.float64)           # codes 0x00..0x7E: 0 .. 448 ascending
    assert np.all(np.diff(vals) > 0)
    mids = (vals[:-1] + vals[1:]) / 2
    pts = np.concatenate([vals, mids]).astype(np.float32)
    cand = [pts]
    up, dn = pts.copy(), pts.copy()
    for _ in range(2):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(0))
        cand += [up, dn]
    rng = np.random.default_rng(40)
    cand.append((2.0 ** rng.uniform(-16, math.log2(448), 4000)).astype(np.float32))
    x = np.concatenate(cand)
    x = x[x <= 448]
    x = np.concatenate([x, -x])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_code(float(v)) for v in x], dtype=np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(ref[i])) for i in bad[:8]]
    # above 448 the encoder saturates (torch's cast turns values past 464 into NaN instead)
    for v in (448.0, 455.9, 464.0, 470.0, 1e6):
        assert oracle.e4m3_code(v) == 0x7E and oracle.e4m3_code(-v) == 0xFE


def _read_quant_golden(path):
    blocks = []
    for line in _read_golden(path):
        f = line.split()
        if f[0] == "block":
            blocks.append((float(f[1]), float(f[2]), []))
        else:
            blocks[-1][2].append((float(f[0]), int(f[1], 16)))
    return blocks


def test_quantiser_golden_blocks(golden_dir):
    """Row 0: the hand-worked blocks side by side.  Row 1: an all-zero block, row 2: a block whose
    amax is below the floor; both take the floored scale fp32(fp32(1e-4)/448)."""
    blocks = _read_quant_golden(os.path.join(golden_dir, "quantize_1x128_blocks.txt"))
    assert len(blocks) == 2
    K = 128 * len(blocks)
    x = np.zeros((3, K), dtype=np.float32)
    want = np.zeros((3, K), dtype=np.uint8)
    for b, (amax, scale, elems) in enumerate(blocks):
        for j, (v, code) in enumerate(elems):
            x[0, 128 * b + j] = v
            want[0, 128 * b + j] = code
        assert np.abs(x[0, 128 * b:128 * b + 128]).max() == amax
    tiny = np.float32(2.0 ** -20)
    x[2, :] = tiny
    codes, sa = oracle.quantize_1x128(bf16_bits_exact(x))
    floored = np.float32(FLOOR / np.float32(448))            # numpy's IEEE fp32 division
    assert np.array_equal(sa[0], np.array([b[1] for b in blocks], np.float32))
    assert np.all(sa[1] == floored) and np.all(sa[2] == floored)
    assert np.array_equal(codes[0], want[0]) and np.all(codes[1] == 0)
    v = np.float32(tiny / floored)
    assert np.all(codes[2] == code_of(float(v)))


def test_quantiser_scale_layout_closed_form():
    """Block (m, kb) holds 2^(m+2kb-4) everywhere but one position (the block's last for a third
    of the blocks), which holds 448 times that (negative for odd m+kb): sa[m][kb] = 2^(m+2kb-4),
    codes 0x38 (1.0) and 0x7E / 0xFE."""
    M, nkb = 3, 3
    x = np.zeros((M, 128 * nkb), dtype=np.float32)
    want = np.zeros_like(x, dtype=np.uint8)
    for m in range(M):
        for kb in range(nkb):
            s = 2.0 ** (m + 2 * kb - 4)
            p = 127 if (m + kb) % 3 == 0 else (7 * m + 13 * kb) % 128
            x[m, 128 * kb:128 * kb + 128] = s
            want[m, 128 * kb:128 * kb + 128] = 0x38
            neg = (m + kb) % 2 == 1
            x[m, 128 * kb + p] = -448 * s if neg else 448 * s
            want[m, 128 * kb + p] = 0xFE if neg else 0x7E
    codes, sa = oracle.quantize_1x128(bf16_bits_exact(x))
    assert np.array_equal(sa, np.array([[2.0 ** (m + 2 * kb - 4) for kb in range(nkb)]
                                        for m in range(M)], np.float32))
    assert np.array_equal(codes, want)


def _quant_input(seed, M=37, K=640, lo=-60, hi=60):
    return W.stress_bf16(M, K, seed, lo=lo, hi=hi)


def test_quantiser_invariants():
    bits = _quant_input(41)
    M, K = bits.shape
    # a few blocks whose largest element is their last or their first
    x = widen(bits).copy()
    for m, kb, pos in ((0, 0, 127), (1, 2, 127), (2, 4, 0), (4, 3, 64)):
        blk = x[m, 128 * kb:128 * kb + 128]
        blk[pos] = -3 * np.abs(blk).max()
    bits = W.bf16_bits(x)
    xb = widen(bits).astype(np.float64)
    codes, sa = oracle.quantize_1x128(bits)
    dec = _DEC[codes].astype(np.float64)
    amax = np.abs(xb).reshape(M, -1, 128).max(axis=2)
    # the block maximum maps to +-448 unless the amax was floored
    big = amax >= FLOOR
    assert np.all(np.abs(dec).reshape(M, -1, 128).max(axis=2)[big] == 448)
    assert np.all(sa[~big] == np.float32(FLOOR / np.float32(448))) and (~big).sum() >= 2
    # no element is clipped by the saturation beyond the rounding of the scale
    ratio = np.abs(xb).reshape(M, -1, 128).max(axis=2) / sa.astype(np.float64)
    assert np.all(ratio <= 448 * (1 + 2.0 ** -22))
    # E4M3 rounding error: half a unit in the last place (2^-4 relative for normals, 2^-10 below
    # 2^-6), plus the fp32 rounding of x/s
    s = np.repeat(sa.astype(np.float64), 128, axis=1)
    err = np.abs(dec * s - xb)
    assert np.all(err <= ((2.0 ** -4 + 2.0 ** -23) * np.abs(xb) + 2.0 ** -10 * s) * (1 + 1e-12))
    # sign symmetry (zeros included: +0 -> 0x00, -0 -> 0x80)
    c2, s2 = oracle.quantize_1x128(bits ^ np.uint16(0x8000))
    assert np.array_equal(c2, codes ^ np.uint8(0x80)) and np.array_equal(s2, sa)
    assert np.any(codes == 0x80) and np.any(codes == 0x00)


def test_quantiser_power_of_two_invariance():
    """Scaling a row by 2^j scales every block's scale by 2^j and leaves the codes unchanged
    (magnitudes kept away from the floor and from bf16's range limits)."""
    bits = np.delete(_quant_input(42, lo=-4, hi=20), [3, 5, 6], axis=0)
    amax = np.abs(widen(bits)).reshape(bits.shape[0], -1, 128).max(axis=2)
    assert amax.min() * 2.0 ** -7 > 2 * FLOOR
    codes, sa = oracle.quantize_1x128(bits)
    for j in (-7, 3, 11):
        b2 = bf16_bits_exact(widen(bits) * np.float32(2.0 ** j))
        c2, s2 = oracle.quantize_1x128(b2)
        assert np.array_equal(c2, codes)
        assert np.array_equal(s2, sa * np.float32(2.0 ** j))


def test_quantiser_matches_library_composition():
    """Whole quantiser against the input recipe built from torch's fp32 division and float8 cast."""
    bits = _quant_input(43, M=64, K=1024)
    codes, sa = oracle.quantize_1x128(bits)
    c2, s2 = W.quantize_1x128(widen(bits))
    assert np.array_equal(codes, c2) and np.array_equal(sa, s2)


# ------------------------------------------------------------------------------------------
# SwiGLU and requantisation (between an MoE expert's two linear layers)
# ------------------------------------------------------------------------------------------

def _swiglu_input(seed, M, I, gate_scale=3.0):
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((M, I)).astype(np.float32) * np.float32(gate_scale)
    u = rng.standard_normal((M, I)).astype(np.float32)
    return W.bf16_bits(np.concatenate([g, u], axis=1))


def test_swiglu_matches_library_silu_and_quantiser():
    """h against torch's fp64 silu of the first half times the second half; codes and scales
    against the input recipe's quantiser (torch's fp32 division and float8 cast) on fp32(h)."""
    I = 640
    bits = _swiglu_input(51, 24, I)
    codes, sa, h = oracle.swiglu_quantize_1x128(bits)
    x = torch.from_numpy(widen(bits).astype(np.float64))
    ref = (torch.nn.functional.silu(x[:, :I]) * x[:, I:]).numpy()
    assert np.allclose(h, ref, rtol=1e-14, atol=0)
    c2, s2 = W.quantize_1x128(ref.astype(np.float32))
    assert np.array_equal(codes, c2) and np.array_equal(sa, s2)


def test_swiglu_closed_forms():
    """silu(0) = 0 and a zero up half gives 0; silu(x) - silu(-x) = x (sigmoid(x) + sigmoid(-x)
    = 1); silu(x) / silu(-x) = -e^x (sigmoid(x) / sigmoid(-x) = e^x); silu(x) -> x for large x."""
    gates = np.array([0.0, 1.1015625, -1.1015625, 1.5, -1.5, 7.0, -7.0, 2.0, 40.0], np.float32)
    ups = np.array([5.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 0.0, 1.0], np.float32)
    I = 128
    x = np.zeros((1, 2 * I), np.float32)
    x[0, :9], x[0, I:I + 9] = gates, ups
    _, _, h = oracle.swiglu_quantize_1x128(W.bf16_bits(x))
    h = h[0]
    assert h[0] == 0.0 and h[7] == 0.0
    for i in (1, 3, 5):
        t = float(gates[i])
        assert abs((h[i] - h[i + 1]) - t) <= 1e-15 * t
        assert abs(h[i] / h[i + 1] + math.exp(t)) <= 1e-14 * math.exp(t)
    assert abs(h[8] - 40.0) <= 40.0 * 1e-16 + 40.0 * math.exp(-40.0) * 1.01
    assert np.all(h[9:] == 0.0)


def test_swiglu_large_gate_is_the_quantiser_of_the_product():
    """gate = 32: sigmoid(32) = 1 - 1.3e-14, so fp32(h) = 32 * up exactly (a bf16 value), and the
    codes and scales equal the 1x128 quantiser's on 32 * up; gate = -120: h is a signed zero."""
    rng = np.random.default_rng(52)
    I = 384
    up = widen(W.bf16_bits(rng.standard_normal((6, I)).astype(np.float32)))
    x = np.concatenate([np.full((6, I), 32.0, np.float32), up], axis=1)
    codes, sa, h = oracle.swiglu_quantize_1x128(W.bf16_bits(x))
    c2, s2 = oracle.quantize_1x128(bf16_bits_exact(up * np.float32(32.0)))
    assert np.array_equal(codes, c2) and np.array_equal(sa, s2)
    x[:, :I] = -120.0
    codes, sa, h = oracle.swiglu_quantize_1x128(W.bf16_bits(x))
    assert np.all(np.abs(h) < 1e-40)
    assert np.all(sa == np.float32(FLOOR / np.float32(448)))
    assert np.all((codes & 0x7F) == 0)


def test_swiglu_quantiser_invariants():
    """Every block's largest code is +-448 (no floored block here); code * s is within half an
    E4M3 unit of fp32(h); flipping the sign of the up half flips every code's sign bit."""
    I = 512
    bits = _swiglu_input(53, 16, I, gate_scale=6.0)
    codes, sa, h = oracle.swiglu_quantize_1x128(bits)
    dec = _DEC[codes].astype(np.float64)
    assert np.all(np.abs(dec).reshape(16, -1, 128).max(axis=2) == 448)
    h32 = h.astype(np.float32).astype(np.float64)
    s = np.repeat(sa.astype(np.float64), 128, axis=1)
    err = np.abs(dec * s - h32)
    assert np.all(err <= ((2.0 ** -4 + 2.0 ** -23) * np.abs(h32) + 2.0 ** -10 * s) * (1 + 1e-12))
    flipped = bits.copy()
    flipped[:, I:] ^= np.uint16(0x8000)
    c2, s2, _ = oracle.swiglu_quantize_1x128(flipped)
    assert np.array_equal(c2, codes ^ np.uint8(0x80)) and np.array_equal(s2, sa)


# ------------------------------------------------------------------------------------------
# FP8 x FP4 (E2M1 elements, E8M0 scales per 32 values)
# ------------------------------------------------------------------------------------------

def test_e2m1_and_e8m0_values(golden_dir):
    """Every E2M1 code and E8M0 anchors against the published OCP MX definition."""
    n = 0
    for line in _read_golden(os.path.join(golden_dir, "e2m1_e8m0_values.txt")):
        kind, code, val = line.split()
        c = int(code, 16)
        if kind == "e2m1":
            got = oracle.e2m1_value(c)
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), (code, got)
        else:
            assert oracle.e8m0_value(c) == 2.0 ** int(val), (code, oracle.e8m0_value(c))
        n += 1
    assert n == 21
    assert math.isnan(oracle.e8m0_value(0xFF))


def _fp4_operands(seed, G=3, M_max=9, N=40, K=384, lo=123, hi=131):
    rng = np.random.default_rng(seed)
    A = W.random_codes(rng, (G, M_max, K))
    sa = np.exp(rng.standard_normal((G, M_max, K // 128))).astype(np.float32)
    B = rng.integers(0, 256, size=(G, N, K // 2), dtype=np.uint8)
    sb = rng.integers(lo, hi + 1, size=(G, N, K // 32)).astype(np.uint8)
    return A, sa, B, sb


def _fp4_values(B, sb):
    """Exact values e2m1(B) * 2^(sb - 127) as float32 [G, N, K] (independent of the oracle)."""
    table = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6], np.float32)
    codes = np.stack([B & 15, B >> 4], axis=-1).reshape(B.shape[0], B.shape[1], -1)
    scale = np.ldexp(np.float32(1), sb.astype(np.int32) - 127).astype(np.float32)
    return table[codes] * np.repeat(scale, 32, axis=-1)


def test_fp4_product_equals_fp8_product_of_the_same_values():
    """With E8M0 scales in [2^-4, 2^4] every scaled E2M1 value is an E4M3 value, so the FP4 product
    must equal the (pinned) FP8 product of those values with unit 128x128 scales, bit for bit."""
    A, sa, B, sb = _fp4_operands(71)
    G, M_max, K = A.shape
    N = B.shape[1]
    vals = _fp4_values(B, sb)
    B8 = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(_DEC[B8], vals)                         # exact in E4M3
    mm = np.array([9, 0, 4], np.int32)
    d4, v4 = oracle.grouped_masked_fp4(A, sa, B, sb, mm)
    d8, v8 = oracle.grouped_masked(A, sa, B8, np.ones((G, -(-N // 128), K // 128), np.float32), mm)
    assert np.array_equal(v4, v8)
    assert np.array_equal(d4[v4.astype(bool)], d8[v8.astype(bool)])


def test_fp4_brute_force_exact_rationals():
    """Tiny shapes with scales over a wide range: the exact rational sum, rounded once to bf16."""
    A, sa, B, sb = _fp4_operands(72, G=2, M_max=3, N=5, K=256, lo=100, hi=160)
    G, M_max, K = A.shape
    N = B.shape[1]
    vals = _fp4_values(B, sb).astype(np.float64)
    mm = np.array([3, 2], np.int32)
    d4, valid = oracle.grouped_masked_fp4(A, sa, B, sb, mm)
    for g in range(G):
        for m in range(mm[g]):
            for n in range(N):
                s = Fraction(0)
                for k in range(K):
                    s += Fraction(float(sa[g, m, k // 128])) * frac_of_code(A[g, m, k]) * Fraction(float(vals[g, n, k]))
                assert d4[g, m, n] == exact_bf16_bits(s), (g, m, n)


def test_fp4_rows_past_count_do_not_matter():
    A, sa, B, sb = _fp4_operands(73)
    mm = np.array([5, 9, 1], np.int32)
    d1, v = oracle.grouped_masked_fp4(A, sa, B, sb, mm)
    rng = np.random.default_rng(3)
    A2, sa2 = A.copy(), sa.copy()
    for g, c in enumerate(mm):
        A2[g, c:] = W.random_codes(rng, A2[g, c:].shape)
        sa2[g, c:] = 7.0
    d2, _ = oracle.grouped_masked_fp4(A2, sa2, B, sb, mm)
    vb = v.astype(bool)
    assert np.array_equal(d1[vb], d2[vb]) and np.all(d1[~vb] == 0)
