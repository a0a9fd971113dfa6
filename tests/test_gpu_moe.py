"""GPU parity of the MoE expert chain pieces: the fused SwiGLU + 1x128 requantisation kernel and
the masked expert layer (first grouped GEMM -> SwiGLU + requantise -> second grouped GEMM),
through the C ABI, against the CPU oracle.

SwiGLU is formed in fp64 by the oracle and in fp32 by the kernel (hardware exp2 and reciprocal),
so the activations agree to a few fp32 units in the last place, not bit for bit.  Where such a
difference decides an integer -- an E4M3 code -- several results are correct, and the tests
compare what is unique and check that the rest is valid:
  - scales: within 2^-20 relative of the oracle's (a few fp32 ulps of the block maximum);
  - codes: equal to the oracle's, except at elements whose exact h / s lies within 2^-16
    (relative) of the midpoint between two adjacent E4M3 values, where the other neighbour is
    accepted too; such elements must be rare.
The GEMM steps are compared with the GEMM tolerance |gpu - ref| <= 2^-7 |ref| + 1e-3 rms(ref)
against the oracle applied to the GPU's own inputs of that step."""
import sys

import numpy as np
import pytest

import oracle
import workloads as W
from parity import assert_close, assert_close_full, gpu_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU runs deselect these with -m "not gpu"
    pytest.skip("needs a GPU", allow_module_level=True)

import fp8_block_scaled_x128_amd as fg  # noqa: E402

_DEC = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float().numpy()
SENT_CODE = 0x7F          # an E4M3 NaN: the library never writes it
SENT_BF16 = 0x7FC1        # a bf16 NaN pattern the library never writes


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def bf16_dev(bits):
    return dev(bits.view(np.int16)).view(torch.bfloat16)


def assert_swiglu_codes(cg, sg, co, so, h, what):
    """GPU codes/scales (cg [R,I], sg [R,I/128]) against the oracle's (co, so, fp64 h)."""
    R, I = co.shape
    rel = np.abs(sg.astype(np.float64) / so.astype(np.float64) - 1.0)
    assert np.all(rel <= 2.0 ** -20), "%s: scales differ by up to %.3g relative" % (what, rel.max())
    diff = cg != co
    n = int(diff.sum())
    if n:
        s = np.repeat(so.astype(np.float64), 128, axis=1)[:, :I]
        v = np.abs(h.astype(np.float32).astype(np.float64) / s)[diff]
        a, b = cg[diff].astype(np.int32), co[diff].astype(np.int32)
        adjacent = ((a & 0x80) == (b & 0x80)) & (np.abs((a & 0x7F) - (b & 0x7F)) == 1)
        mid = (np.abs(_DEC[a]) + np.abs(_DEC[b])) / 2.0
        near = np.abs(v - mid) <= 2.0 ** -16 * mid
        assert np.all(adjacent & near), "%s: %d codes differ away from a rounding midpoint" % (
            what, int((~(adjacent & near)).sum()))
        assert n <= max(2, 1e-3 * co.size), "%s: %d of %d codes differ" % (what, n, co.size)
    return n


# ------------------------------------------------------------------------------------------
# SwiGLU + requantisation
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("M,I", [(1, 128), (17, 256), (257, 640), (1000, 2048)])
def test_swiglu_quantize_matches_oracle(M, I):
    """Rows off the 16-block workgroups, several blocks per row, outlier channels."""
    bits = W.swiglu_input_bf16(M, I, seed=M + I)
    codes, scales = fg.swiglu_quantize_1x128(bf16_dev(bits))
    torch.cuda.synchronize()
    co, so, h = oracle.swiglu_quantize_1x128(bits)
    cg = codes.view(torch.uint8).cpu().numpy()
    sg = scales.cpu().numpy().T
    n = assert_swiglu_codes(cg, sg, co, so, h, "swiglu %dx%d" % (M, I))
    say("swiglu", M, I, fg.last_config(), "codes off by one at midpoints:", n)


def test_swiglu_quantize_exact_cases():
    """gate = 32: sigmoid rounds to 1 in fp32, h = 32 * up exactly, so codes and scales are
    bit-exact; gate = -120: e^120 overflows, h is a signed zero and the block scale the floor."""
    rng = np.random.default_rng(61)
    I = 384
    up = (W.bf16_bits(rng.standard_normal((40, I)).astype(np.float32)).astype(np.uint32) << 16).view(np.float32)
    x = np.concatenate([np.full((40, I), 32.0, np.float32), up], axis=1)
    x[20:, :I] = -120.0
    bits = W.bf16_bits(x)
    codes, scales = fg.swiglu_quantize_1x128(bf16_dev(bits))
    torch.cuda.synchronize()
    co, so, _ = oracle.swiglu_quantize_1x128(bits)
    assert np.array_equal(codes.view(torch.uint8).cpu().numpy(), co)
    assert np.array_equal(scales.cpu().numpy().T, so)


def test_swiglu_quantize_masked_rows_and_counts():
    G, M_max, I = 4, 96, 512
    mm = np.array([0, 1, 50, 96], np.int32)
    bits = W.swiglu_input_bf16(G * M_max, I, seed=62).reshape(G, M_max, 2 * I)
    codes = torch.full((G, M_max, I), SENT_CODE, dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
    scales = torch.full((G, I // 128, M_max), float("nan"), dtype=torch.float32, device="cuda")
    fg.swiglu_quantize_1x128_masked(bf16_dev(bits), dev(mm), codes=codes, scales=scales)
    torch.cuda.synchronize()
    assert fg.read_device_error() == 0
    cg = codes.view(torch.uint8).cpu().numpy()
    sg = scales.cpu().numpy()
    for g in range(G):
        c = int(mm[g])
        assert np.all(cg[g, c:] == SENT_CODE) and np.all(np.isnan(sg[g, :, c:]))
        if c:
            co, so, h = oracle.swiglu_quantize_1x128(bits[g, :c])
            assert_swiglu_codes(cg[g, :c], sg[g, :, :c].T, co, so, h, "masked group %d" % g)
    # a count outside [0, M_max] is clamped and flagged
    bad = np.array([-3, 200, 0, 0], np.int32)
    fg.swiglu_quantize_1x128_masked(bf16_dev(bits), dev(bad), codes=codes, scales=scales)
    assert fg.read_device_error() & fg.DEVERR_BAD_COUNT
    cg2 = codes.view(torch.uint8).cpu().numpy()
    co, so, h = oracle.swiglu_quantize_1x128(bits[1])
    assert_swiglu_codes(cg2[1], scales.cpu().numpy()[1].T, co, so, h, "clamped count")


# ------------------------------------------------------------------------------------------
# the masked expert layer
# ------------------------------------------------------------------------------------------

def _sa_dev(sa):
    return dev(np.swapaxes(sa, -1, -2))


def _sentinel_bf16(shape):
    return torch.full(shape, SENT_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def _run_chain(e, G, M_max, H, I):
    Y1 = _sentinel_bf16((G, M_max, 2 * I))
    Hq = torch.full((G, M_max, I), SENT_CODE, dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
    sh = torch.full((G, I // 128, M_max), float("nan"), dtype=torch.float32, device="cuda")
    out = _sentinel_bf16((G, M_max, H))
    fg.moe_expert_masked(dev(e.A), _sa_dev(e.sa), dev(e.W1), dev(e.s1), dev(e.W2), dev(e.s2),
                         dev(e.masked_m), e.expected_m, out=out, workspace=(Y1, Hq, sh))
    torch.cuda.synchronize()
    return Y1, Hq, sh, out


@pytest.mark.parametrize("mm,M_max,H,I", [([70, 0, 33], 80, 256, 384), ([130, 5], 160, 384, 256)])
def test_moe_expert_chain_stagewise(mm, M_max, H, I):
    """Each step of the chain against the oracle applied to the GPU's own input of that step;
    rows past the counts untouched in every workspace and in the output; the chain entry point
    equals the three steps called one by one (bit for bit)."""
    mm = np.array(mm, np.int32)
    G = len(mm)
    e = W.moe_expert(mm, M_max, H, I, seed=int(mm.sum()) + H, expected_m=64)
    Y1, Hq, sh, out = _run_chain(e, G, M_max, H, I)
    assert fg.read_device_error() == 0
    y1 = gpu_bits(Y1)
    hq = Hq.view(torch.uint8).cpu().numpy()
    shn = sh.cpu().numpy()
    ob = gpu_bits(out)
    valid = np.arange(M_max)[None, :] < mm[:, None]
    # first layer
    ref1, _ = oracle.grouped_masked(e.A, e.sa, e.W1, e.s1, mm)
    v1 = np.broadcast_to(valid[:, :, None], ref1.shape)
    assert_close(y1, ref1, mask=v1, what="first layer")
    assert np.all(y1[~v1] == SENT_BF16)
    # SwiGLU + requantisation of the GPU's first-layer output
    for g in range(G):
        c = int(mm[g])
        assert np.all(hq[g, c:] == SENT_CODE) and np.all(np.isnan(shn[g, :, c:]))
        if c:
            co, so, h = oracle.swiglu_quantize_1x128(y1[g, :c])
            assert_swiglu_codes(hq[g, :c], shn[g, :, :c].T, co, so, h, "swiglu group %d" % g)
    # second layer on the GPU's codes and scales
    ref2, _ = oracle.grouped_masked(hq, np.swapaxes(np.nan_to_num(shn), -1, -2), e.W2, e.s2, mm)
    v2 = np.broadcast_to(valid[:, :, None], ref2.shape)
    assert_close(ob, ref2, mask=v2, what="second layer")
    assert np.all(ob[~v2] == SENT_BF16)
    # the three steps one by one
    Y1b = fg.grouped_masked(dev(e.A), _sa_dev(e.sa), dev(e.W1), dev(e.s1), dev(e.masked_m), e.expected_m)
    Hb, shb = fg.swiglu_quantize_1x128_masked(Y1b, dev(e.masked_m))
    outb = fg.grouped_masked(Hb, shb, dev(e.W2), dev(e.s2), dev(e.masked_m), e.expected_m)
    torch.cuda.synchronize()
    assert np.array_equal(gpu_bits(outb)[v2], ob[v2])
    say("chain", mm.tolist(), M_max, H, I, fg.last_config())


def test_moe_expert_chain_argument_errors():
    G, M_max, H, I = 2, 16, 256, 256
    e = W.moe_expert(np.array([3, 4], np.int32), M_max, H, I, seed=5)
    args = [dev(e.A), _sa_dev(e.sa), dev(e.W1), dev(e.s1), dev(e.W2), dev(e.s2), dev(e.masked_m)]
    with pytest.raises(ValueError):       # W2 of the wrong width
        fg.moe_expert_masked(*args[:4], dev(e.W2[:, :, :128]), args[5], args[6], 4)
    lib = fg.lib()
    p = [a.data_ptr() for a in args]
    ws = [torch.empty(x, dtype=torch.uint8, device="cuda") for x in (G * M_max * 2 * I * 2, G * M_max * I,
                                                                      G * M_max * I // 128 * 4, G * M_max * H * 2)]
    w = [t.data_ptr() for t in ws]
    assert lib.fp8gemm_moe_expert_masked(*p, *w, G, M_max, H, 200, 4, None) == 2     # I % 128
    assert lib.fp8gemm_moe_expert_masked(*p, *w, 0, M_max, H, I, 4, None) == 2      # G <= 0
    assert lib.fp8gemm_moe_expert_masked(*p[:6], None, *w, G, M_max, H, I, 4, None) == 1
    assert lib.fp8gemm_moe_expert_masked(*p, w[0] + 2, *w[1:], G, M_max, H, I, 4, None) == 3


@pytest.mark.slow
def test_moe_expert_chain_deepseek_v3_size():
    """The masked decode configuration as a whole expert layer (16 groups, M_max 256, about 64
    valid rows each, H = 7168, I = 2048): every valid output of both layers against the oracle on
    the GPU's own input to that layer (GEMM tolerance, rms over all valid outputs), and the
    SwiGLU + requantisation step on every valid row."""
    say("moe expert config 4")
    e = W.moe_config4()
    G, M_max, H = e.A.shape
    I = e.W2.shape[2]
    Y1, Hq, sh, out = _run_chain(e, G, M_max, H, I)
    lc = fg.last_config()
    assert fg.read_device_error() == 0
    valid = np.arange(M_max)[None, :] < e.masked_m[:, None]
    y1 = gpu_bits(Y1)
    ref1, _ = oracle.grouped_masked(e.A, e.sa, e.W1, e.s1, e.masked_m)
    rep1 = assert_close_full(y1, ref1, mask=np.broadcast_to(valid[:, :, None], y1.shape),
                             what="moe config 4 first layer [%s]" % lc)
    gi, ri = np.nonzero(valid)
    rows = gi * M_max + ri
    hq = Hq.view(torch.uint8).cpu().numpy().reshape(G * M_max, I)
    shn = np.nan_to_num(np.swapaxes(sh.cpu().numpy(), 1, 2)).reshape(G * M_max, I // 128)
    co, so, h = oracle.swiglu_quantize_1x128(y1.reshape(G * M_max, 2 * I)[rows])
    nd = assert_swiglu_codes(hq[rows], shn[rows], co, so, h, "swiglu, every valid row")
    ob = gpu_bits(out)
    ref2, _ = oracle.grouped_masked(hq.reshape(G, M_max, I), shn.reshape(G, M_max, I // 128), e.W2, e.s2,
                                    e.masked_m)
    rep2 = assert_close_full(ob, ref2, mask=np.broadcast_to(valid[:, :, None], ob.shape),
                             what="moe config 4 second layer [%s]" % lc)
    say("moe expert config 4 ok", lc, rep1["bit_equal"], nd, rep2["bit_equal"])
