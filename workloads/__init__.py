"""Seeded synthetic inputs for the FP8 block-scaled GEMM (shared by the tests, the smoke check
and the benchmark).

This module only *makes inputs*: it draws N(0,1) fp32 values and quantises them to OCP E4M3
codes with fp32 block scales, and it lays out the grouped (MoE) variants.  It holds none of the
GEMM arithmetic; the oracle and the HIP library both consume the bytes produced here.

Quantisation recipe (input preparation; the pages only say "fine-grained scaling", page
"DeepSeek開源第三彈：V3/R1訓練推理關鍵秘籍，核心代碼僅300行", section 深入了解DeepGEMM):
  * A (activations) has one scale per 1x128 block of a row, B (weights) one per 128x128 block.
  * scale = fp32(amax / 448) over the block (448 = largest finite E4M3 value); the amax is
    floored at fp32(1e-4) so that an all-zero block keeps a finite scale (its codes are zero).
  * code = E4M3 round-to-nearest-even of fp32(x / scale), saturated to +-448 first (torch's
    cast would give NaN above 464; saturating is the plain quantiser).
The float8 cast is torch's library routine; random numbers come from numpy's PCG64
``default_rng(seed)``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

E4M3_MAX = 448.0
BLOCK = 128

# ---------------------------------------------------------------------------------------------
# Workload definitions (shapes and value recipes of the five measured configurations)
# ---------------------------------------------------------------------------------------------

#: Dense decode/prefill sweep over DeepSeek-V3-like projection shapes.
SWEEP_M = (64, 128, 4096)
SWEEP_NK = ((2112, 7168), (24576, 1536), (32768, 512), (7168, 16384), (4096, 7168), (7168, 2048))


@dataclass
class Dense:
    A: np.ndarray      # uint8 [M, K] E4M3 codes
    sa: np.ndarray     # float32 [M, K/128]
    B: np.ndarray      # uint8 [N, K]
    sb: np.ndarray     # float32 [ceil(N/128), K/128]

    @property
    def shape(self):
        return self.A.shape[0], self.B.shape[0], self.A.shape[1]


@dataclass
class Contiguous:
    A: np.ndarray          # uint8 [M_total, K]
    sa: np.ndarray         # float32 [M_total, K/128]
    B: np.ndarray          # uint8 [G, N, K]
    sb: np.ndarray         # float32 [G, ceil(N/128), K/128]
    m_indices: np.ndarray  # int32 [M_total], -1 = padding row
    counts: list = field(default_factory=list)  # valid rows per group


@dataclass
class Masked:
    A: np.ndarray          # uint8 [G, M_max, K]
    sa: np.ndarray         # float32 [G, M_max, K/128]
    B: np.ndarray          # uint8 [G, N, K]
    sb: np.ndarray         # float32 [G, ceil(N/128), K/128]
    masked_m: np.ndarray   # int32 [G]
    expected_m: int = 0


@dataclass
class MoeExpert:
    """One MoE expert layer per group on the masked layout: out = swiglu(A W1^T) W2^T."""
    A: np.ndarray          # uint8 [G, M_max, H]
    sa: np.ndarray         # float32 [G, M_max, H/128]
    W1: np.ndarray         # uint8 [G, 2I, H]     (gate rows [0, I), up rows [I, 2I))
    s1: np.ndarray         # float32 [G, 2I/128, H/128]
    W2: np.ndarray         # uint8 [G, H, I]
    s2: np.ndarray         # float32 [G, ceil(H/128), I/128]
    masked_m: np.ndarray   # int32 [G]
    expected_m: int = 0


# ---------------------------------------------------------------------------------------------
# Random draws and quantisation
# ---------------------------------------------------------------------------------------------

def normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def _cast_e4m3(y: torch.Tensor) -> torch.Tensor:
    """Saturating round-to-nearest-even fp32 -> E4M3 codes (uint8)."""
    y = torch.clamp(y, -E4M3_MAX, E4M3_MAX)
    return y.to(torch.float8_e4m3fn).view(torch.uint8)


def quantize_1x128(x: np.ndarray, chunk_rows: int = 8192):
    """x: float32 [R, K] -> (codes uint8 [R, K], scales float32 [R, ceil(K/128)])."""
    R, K = x.shape
    nkb = -(-K // BLOCK)
    codes = np.empty((R, K), dtype=np.uint8)
    scales = np.empty((R, nkb), dtype=np.float32)
    for r0 in range(0, R, chunk_rows):
        r1 = min(R, r0 + chunk_rows)
        t = torch.from_numpy(np.ascontiguousarray(x[r0:r1]))
        if K % BLOCK:
            t = torch.nn.functional.pad(t, (0, nkb * BLOCK - K))
        tb = t.view(r1 - r0, nkb, BLOCK)
        amax = tb.abs().amax(dim=2).clamp_min(1e-4)
        s = amax / E4M3_MAX
        q = _cast_e4m3(tb / s.unsqueeze(2)).reshape(r1 - r0, nkb * BLOCK)[:, :K]
        codes[r0:r1] = q.numpy()
        scales[r0:r1] = s.numpy()
    return codes, scales


def quantize_128x128(x: np.ndarray):
    """x: float32 [N, K] -> (codes uint8 [N, K], scales float32 [ceil(N/128), ceil(K/128)]).
    A partial last block (N or K not a multiple of 128) takes its amax over the rows/columns it has."""
    N, K = x.shape
    nnb, nkb = -(-N // BLOCK), -(-K // BLOCK)
    codes = np.empty((N, K), dtype=np.uint8)
    scales = np.empty((nnb, nkb), dtype=np.float32)
    for b in range(nnb):
        r0, r1 = b * BLOCK, min(N, (b + 1) * BLOCK)
        t = torch.from_numpy(np.ascontiguousarray(x[r0:r1]))
        if K % BLOCK:
            t = torch.nn.functional.pad(t, (0, nkb * BLOCK - K))
        tb = t.view(r1 - r0, nkb, BLOCK)
        amax = tb.abs().amax(dim=(0, 2)).clamp_min(1e-4)
        s = amax / E4M3_MAX
        q = _cast_e4m3(tb / s.view(1, nkb, 1)).reshape(r1 - r0, nkb * BLOCK)[:, :K]
        codes[r0:r1] = q.numpy()
        scales[b] = s.numpy()
    return codes, scales


def random_codes(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniform over the 254 non-NaN E4M3 codes (0x7F and 0xFF excluded)."""
    c = rng.integers(0, 254, size=shape, dtype=np.int32)
    c = c + (c >= 0x7F).astype(np.int32)           # skip 0x7F
    c = c + (c >= 0xFF).astype(np.int32)           # skip 0xFF (cannot be reached after shift)
    return c.astype(np.uint8)


def _weights(rng, N, K):
    return quantize_128x128(normal(rng, (N, K)))


def acts(rng, M, K, chunk_rows=4096):
    """A operand: N(0,1) rows quantised per 1x128 block -> (codes [M,K], scales [M, K/128])."""
    nkb = -(-K // BLOCK)
    codes = np.empty((M, K), dtype=np.uint8)
    scales = np.empty((M, nkb), dtype=np.float32)
    for r0 in range(0, M, chunk_rows):
        r1 = min(M, r0 + chunk_rows)
        codes[r0:r1], scales[r0:r1] = quantize_1x128(normal(rng, (r1 - r0, K)))
    return codes, scales


# ---------------------------------------------------------------------------------------------
# Workload builders
# ---------------------------------------------------------------------------------------------

def dense(M: int, N: int, K: int, seed: int, seed_b: int | None = None) -> Dense:
    """N(0,1) fp32 operands quantised per the recipe above.  B is drawn from ``seed_b`` when given
    (so that a sweep can share one weight matrix between several M)."""
    rng_b = np.random.default_rng(seed if seed_b is None else seed_b)
    rng_a = np.random.default_rng(seed) if seed_b is not None else rng_b
    B, sb = _weights(rng_b, N, K)
    A, sa = acts(rng_a, M, K)
    return Dense(A, sa, B, sb)


def sweep_seeds(mi: int, nki: int):
    """Seeds of the dense sweep case (M index mi, (N,K) index nki): (A seed, B seed)."""
    return 200 + 10 * mi + nki, 100 + nki


def sweep_case(mi: int, nki: int) -> Dense:
    M = SWEEP_M[mi]
    N, K = SWEEP_NK[nki]
    sa_seed, sb_seed = sweep_seeds(mi, nki)
    return dense(M, N, K, sa_seed, sb_seed)


def contiguous(counts, slot: int, N: int, K: int, seed: int, packed: bool = False) -> Contiguous:
    """Groups concatenated along M.  Group g has counts[g] valid rows followed by padding rows
    (m_indices = -1) up to the end of its slot.  ``packed``: the slot of group g is counts[g]
    rounded up to a multiple of 128 instead of the fixed ``slot``."""
    rng = np.random.default_rng(seed)
    G = len(counts)
    slots = [(-(-c // BLOCK)) * BLOCK if packed else slot for c in counts]
    M = int(sum(slots))
    m_idx = np.full((M,), -1, dtype=np.int32)
    r = 0
    for g, (c, s) in enumerate(zip(counts, slots)):
        assert 0 <= c <= s
        m_idx[r:r + c] = g
        r += s
    Bs, sbs = [], []
    for g in range(G):
        b, s = _weights(rng, N, K)
        Bs.append(b)
        sbs.append(s)
    A, sa = acts(rng, M, K)
    return Contiguous(A, sa, np.stack(Bs), np.stack(sbs), m_idx, list(counts))


def masked(masked_m, M_max: int, N: int, K: int, seed: int, expected_m: int = 0) -> Masked:
    """Group g has M_max rows of which the first masked_m[g] are valid.  Rows past masked_m hold
    uniform random non-NaN codes and random positive scales: they must not change any output."""
    rng = np.random.default_rng(seed)
    G = len(masked_m)
    nkb = -(-K // BLOCK)
    Bs, sbs = [], []
    for g in range(G):
        b, s = _weights(rng, N, K)
        Bs.append(b)
        sbs.append(s)
    A = np.empty((G, M_max, K), dtype=np.uint8)
    sa = np.empty((G, M_max, nkb), dtype=np.float32)
    for g in range(G):
        c = int(min(max(masked_m[g], 0), M_max))
        if c:
            A[g, :c], sa[g, :c] = acts(rng, c, K)
        if c < M_max:
            A[g, c:] = random_codes(rng, (M_max - c, K))
            sa[g, c:] = np.exp(rng.standard_normal((M_max - c, nkb))).astype(np.float32) * 0.01
    return Masked(A, sa, np.stack(Bs), np.stack(sbs), np.asarray(masked_m, dtype=np.int32),
                  expected_m)


# --- 4-bit weights: OCP MXFP4 (E2M1 elements, one E8M0 scale per 32 consecutive values) -------

E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


# Rounding thresholds on |x| / 2^e for E2M1 codes 1..7: the midpoints between neighbouring grid
# values; at a midpoint the even code (mantissa bit 0) wins, so a threshold that leads to an odd
# code is passed only strictly (">") and one that leads to an even code inclusively (">=").
_E2M1_UP = ((0.25, False), (0.75, True), (1.25, False), (1.75, True), (2.5, False), (3.5, True), (5.0, False))


def quantize_mxfp4(x: np.ndarray, chunk_rows: int = 1024):
    """x: float32 [R, K] (K a multiple of 32) -> (packed uint8 [R, K/2], scales uint8 [R, K/32]).
    Per 32-value block the shared exponent is floor(log2(amax)) - 2 (E2M1's largest exponent is
    2), so amax / 2^e lies in [4, 8); elements round to the nearest E2M1 value (ties to the even
    code), saturating at 6.  An all-zero block gets scale 2^0."""
    R, K = x.shape
    assert K % 32 == 0
    packed = np.empty((R, K // 2), dtype=np.uint8)
    scales = np.empty((R, K // 32), dtype=np.uint8)
    for r0 in range(0, R, chunk_rows):
        r1 = min(R, r0 + chunk_rows)
        xb = x[r0:r1].astype(np.float64).reshape(r1 - r0, K // 32, 32)
        amax = np.abs(xb).max(axis=2)
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, 0).astype(np.int64)
        e = np.clip(e, -127, 127)
        y = np.abs(xb) / np.ldexp(1.0, e)[:, :, None]
        code = np.zeros(y.shape, dtype=np.uint8)
        for t, inclusive in _E2M1_UP:
            code += (y >= t) if inclusive else (y > t)
        code |= np.where(xb < 0, 8, 0).astype(np.uint8)
        code = code.reshape(r1 - r0, K)
        packed[r0:r1] = code[:, 0::2] | (code[:, 1::2] << 4)
        scales[r0:r1] = (e + 127).astype(np.uint8)
    return packed, scales


@dataclass
class MaskedFp4:
    A: np.ndarray          # uint8 [G, M_max, K] E4M3
    sa: np.ndarray         # float32 [G, M_max, K/128]
    B: np.ndarray          # uint8 [G, N, K/2] E2M1 pairs
    sb: np.ndarray         # uint8 [G, N, K/32] E8M0
    masked_m: np.ndarray   # int32 [G]
    expected_m: int = 0


def masked_fp4(masked_m, M_max: int, N: int, K: int, seed: int, expected_m: int = 0) -> MaskedFp4:
    """As ``masked`` with the right operand N(0,1) quantised to MXFP4."""
    first = masked(masked_m, M_max, 128, K, seed, expected_m)      # A, sa and rows past the counts
    rng = np.random.default_rng(seed + 11)
    Bs, sbs = zip(*(quantize_mxfp4(normal(rng, (N, K))) for _ in range(len(masked_m))))
    return MaskedFp4(first.A, first.sa, np.stack(Bs), np.stack(sbs), first.masked_m, expected_m)


def config4_fp4() -> MaskedFp4:
    """The masked decode configuration with its weights in MXFP4: 16 groups, M_max=256,
    masked_m ~ Poisson(64), N=4096, K=7168."""
    return masked_fp4(config4_masked_m(), 256, 4096, 7168, seed=44, expected_m=64)


def moe_expert(masked_m, M_max: int, H: int, I: int, seed: int, expected_m: int = 0) -> MoeExpert:
    """Activations as in ``masked`` (hidden size H); both layers' weights N(0,1) quantised per
    128x128 block with their scales divided by sqrt(fan-in), so the first layer's outputs (the
    SwiGLU inputs) and the second layer's outputs are of order one."""
    first = masked(masked_m, M_max, 2 * I, H, seed, expected_m)
    rng = np.random.default_rng(seed + 7)
    W2, s2 = zip(*(_weights(rng, H, I) for _ in range(len(masked_m))))
    s1 = (first.sb / np.float32(np.sqrt(H))).astype(np.float32)
    s2 = (np.stack(s2) / np.float32(np.sqrt(I))).astype(np.float32)
    return MoeExpert(first.A, first.sa, first.B, s1, np.stack(W2), s2, first.masked_m, expected_m)


def moe_config4() -> MoeExpert:
    """The masked decode configuration as a whole DeepSeek-V3-sized expert layer: 16 groups,
    M_max=256, masked_m ~ Poisson(64), hidden size H=7168, expert intermediate size I=2048 (the
    first layer is the configuration's N=4096 x K=7168 GEMM, the second N=7168 x K=2048)."""
    return moe_expert(config4_masked_m(), 256, 7168, 2048, seed=40, expected_m=64)


def swiglu_input_bf16(M: int, I: int, seed: int) -> np.ndarray:
    """bf16 [M, 2I] first-layer outputs (gate | up): N(0,1) gates times 2 (over the curved part of
    silu, both signs), N(0,1) ups with 1% outlier channels of gain 16."""
    rng = np.random.default_rng(seed)
    gain = np.ones(I, dtype=np.float32)
    gain[rng.choice(I, size=max(1, I // 100), replace=False)] = 16.0
    g = normal(rng, (M, I)) * np.float32(2.0)
    u = normal(rng, (M, I)) * gain
    return bf16_bits(np.concatenate([g, u], axis=1))


# --- the five configurations -----------------------------------------------------------------

def config0() -> Dense:
    """Dense M=256, N=512, K=1024."""
    return dense(256, 512, 1024, seed=0)


def config2() -> Contiguous:
    """Contiguous MoE: 4 groups, slots of 8192 rows (M=32768), 5% of each slot padding (7782 valid
    + 410 rows of -1), N=4096, K=7168."""
    return contiguous([7782] * 4, 8192, 4096, 7168, seed=2)


def config3_counts(seed: int = 3):
    rng = np.random.default_rng(seed + 1000)
    return [int(x) for x in rng.integers(3000, 4096, size=8, endpoint=True)]


def config3() -> Contiguous:
    """Contiguous MoE down-projection: 8 groups, slots of 4096 rows (M=32768), valid rows per
    group uniform in [3000, 4096], the rest of each slot padding; N=7168, K=2048."""
    return contiguous(config3_counts(), 4096, 7168, 2048, seed=3)


def config4_masked_m(seed: int = 4):
    rng = np.random.default_rng(seed + 1000)
    return np.clip(rng.poisson(64, size=16), 0, 256).astype(np.int32)


def config4() -> Masked:
    """Masked MoE decode: 16 groups, M_max=256, masked_m ~ Poisson(64) clipped to [0, 256],
    expected_m=64, N=4096, K=7168."""
    return masked(config4_masked_m(), 256, 4096, 7168, seed=4, expected_m=64)


# --- bf16 activations: inputs of the 1x128 quantiser -----------------------------------------

#: Activation matrix quantised in the benchmark: the left operand of the contiguous MoE
#: configuration (32768 rows of K=7168).
QUANT_M, QUANT_K = 32768, 7168


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even (torch's cast)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def activations_bf16(M: int, K: int, seed: int, chunk_rows: int = 4096) -> np.ndarray:
    """Hidden-state-like bf16 activations [M,K] (bit patterns): N(0,1) times a per-channel gain,
    where 1% of the channels (chosen by the seed) carry a gain of 32 -- the outlier channels that
    make one scale per 128 values worth having."""
    rng = np.random.default_rng(seed)
    gain = np.ones(K, dtype=np.float32)
    gain[rng.choice(K, size=max(1, K // 100), replace=False)] = 32.0
    out = np.empty((M, K), dtype=np.uint16)
    for r0 in range(0, M, chunk_rows):
        r1 = min(M, r0 + chunk_rows)
        out[r0:r1] = bf16_bits(normal(rng, (r1 - r0, K)) * gain)
    return out


def stress_bf16(M: int, K: int, seed: int, lo: int = -60, hi: int = 60) -> np.ndarray:
    """bf16 rows [M,K] (bit patterns) whose 128-wide blocks span magnitudes 2^U[lo,hi] (N(0,1)
    values times a per-block power of two), with, where the shape has room, an all-zero block
    (row 3, block 1), a block of bf16 subnormals (row 5, block 0) and signed zeros (row 6)."""
    rng = np.random.default_rng(seed)
    nkb = -(-K // BLOCK)
    x = normal(rng, (M, K))
    mag = 2.0 ** rng.integers(lo, hi + 1, size=(M, nkb))
    x *= np.repeat(mag, BLOCK, axis=1)[:, :K].astype(np.float32)
    if M > 3 and nkb > 1:
        x[3, BLOCK:2 * BLOCK] = 0
    if M > 5:
        x[5, :BLOCK] *= np.float32(2.0 ** -128 / mag[5, 0])
    if M > 6:
        x[6, ::3] = -0.0
    return bf16_bits(x)


def quantize_work(rows: int, K: int):
    """Bytes the 1x128 quantiser must move: bf16 in, E4M3 codes and fp32 scales out."""
    return rows * K * 2 + rows * K + 4 * rows * (-(-K // BLOCK))


# --- algorithmic work counts (for throughput and roofline reporting) --------------------------

def dense_work(M, N, K):
    """(flop, bytes): 2MNK and A + sa + B + sb + D bytes."""
    nkb, nnb = -(-K // BLOCK), -(-N // BLOCK)
    return 2 * M * N * K, M * K + 4 * M * nkb + N * K + 4 * nnb * nkb + 2 * M * N


def swiglu_quantize_work(rows: int, I: int):
    """Bytes of the SwiGLU + requantisation step: bf16 gate and up in, E4M3 codes and fp32 scales
    out."""
    return rows * 2 * I * 2 + rows * I + 4 * rows * (-(-I // BLOCK))


def moe_expert_work(valid_rows_per_group, H, I, G):
    """(flop, bytes) of one masked expert layer: the first layer (N = 2I, K = H), the SwiGLU step
    and the second layer (N = H, K = I); masked counts as index bytes of both GEMMs."""
    f1, b1 = grouped_work(valid_rows_per_group, 2 * I, H, index_bytes=4 * G)
    f2, b2 = grouped_work(valid_rows_per_group, H, I, index_bytes=4 * G)
    rows = int(sum(valid_rows_per_group))
    return f1 + f2, b1 + swiglu_quantize_work(rows, I) + b2


def grouped_fp4_work(valid_rows_per_group, N, K, index_bytes):
    """(flop, bytes) of the masked GEMM with MXFP4 weights: B is K/2 bytes per row plus one E8M0
    byte per 32 values; A, its scales, D and the counts as in ``grouped_work``."""
    nkb = -(-K // BLOCK)
    rows = int(sum(valid_rows_per_group))
    groups = sum(1 for c in valid_rows_per_group if c > 0)
    flop = 2 * rows * N * K
    byts = rows * K + 4 * rows * nkb + groups * (N * K // 2 + N * K // 32) + 2 * rows * N + index_bytes
    return flop, byts


def grouped_work(valid_rows_per_group, N, K, index_bytes):
    nkb, nnb = -(-K // BLOCK), -(-N // BLOCK)
    rows = int(sum(valid_rows_per_group))
    groups = sum(1 for c in valid_rows_per_group if c > 0)
    flop = 2 * rows * N * K
    byts = rows * K + 4 * rows * nkb + groups * (N * K + 4 * nnb * nkb) + 2 * rows * N + index_bytes
    return flop, byts
