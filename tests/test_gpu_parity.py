"""GPU parity: the HIP library (called through the C ABI) against the CPU oracle, element by
element, on seeded inputs.  Floating-point cases: |gpu - ref| <= 2^-7 |ref| + 1e-3 rms(ref);
integer-valued and power-of-two-scale cases: bit-exact."""
import os
import re
import sys

import numpy as np
import pytest

import oracle
import workloads as W
from parity import assert_bit_exact, assert_close, assert_close_full, gpu_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU runs deselect these with -m "not gpu"
    pytest.skip("needs a GPU", allow_module_level=True)

import fp8_block_scaled_x128_amd as fg  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SENTINEL = 0x7FC1   # a NaN pattern the library never writes


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def dev_sa(sa):
    """Scales of A as the library takes them: K-block-major ([.., K/128, rows])."""
    return dev(np.swapaxes(sa, -1, -2))


def run_dense(d, out=None):
    D = fg.gemm_nt(dev(d.A), dev_sa(d.sa), dev(d.B), dev(d.sb), out=out)
    torch.cuda.synchronize()
    return D


def sentinel_tensor(shape):
    t = torch.full(shape, SENTINEL, dtype=torch.int16, device="cuda")
    return t.view(torch.bfloat16)


def kernel_table():
    src = open(os.path.join(ROOT, "fp8_block_scaled_x128_amd", "csrc", "fp8gemm_kernels.hip")).read()
    return [(int(a), int(b), int(c), int(d), int(e), f) for a, b, c, d, e, f in
            re.findall(r"FP8GEMM_ENTRY\((\d+), (\d+), (\d+), (\d+), (\d+), (k\w+)\)", src)]


def stream_table():
    """Configurations of the masked decode kernel: (rows, waves, fragments, phase, depth)."""
    src = open(os.path.join(ROOT, "fp8_block_scaled_x128_amd", "csrc", "stream_kernels.hip")).read()
    return [tuple(int(x) for x in t) for t in
            re.findall(r"STREAM_ENTRY\((\d+), (\d+), (\d+), (\d+), (\d+)\)", src)]


def stream_id(e):
    return "mt%d_w%d_jn%d_kp%d_pf%d" % e[:5]


class forced:
    """Force the launch configuration of the calls inside the block (FP8GEMM_FORCE_CONFIG)."""

    def __init__(self, bm, bn, wm, wn, st, split):
        self.v = "%dx%d:%dx%d:%d:%d" % (bm, bn, wm, wn, st, split)

    def __enter__(self):
        os.environ["FP8GEMM_FORCE_CONFIG"] = self.v

    def __exit__(self, *exc):
        os.environ.pop("FP8GEMM_FORCE_CONFIG", None)


class forced_stream(forced):
    """Force a configuration of the masked decode kernel."""

    def __init__(self, mt, w, jn, kp, pf, split):
        self.v = "stream:%d:%d:%d:%d:%d:%d" % (mt, w, jn, kp, pf, split)


def int_codes(rng, shape, lo=-4, hi=4):
    vals = rng.integers(lo, hi + 1, size=shape).astype(np.float32)
    return torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# ------------------------------------------------------------------------------------------
# dense
# ------------------------------------------------------------------------------------------

def test_config0_full_parity():
    d = W.config0()
    D = run_dense(d)
    ref = oracle.gemm_nt(d.A, d.sa, d.B, d.sb)
    rep = assert_close(gpu_bits(D), ref, what="config 0")
    say("config0", fg.last_config(), rep)


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (3, 17, 256), (64, 64, 128), (65, 300, 640),
                                   (128, 2112, 1024), (130, 257, 384), (256, 512, 1024),
                                   (1030, 520, 1152), (64, 2112, 7168)])
def test_integer_inputs_bit_exact(M, N, K):
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    A, B = int_codes(rng, (M, K)), int_codes(rng, (N, K))
    sa = np.ones((M, K // 128), np.float32)
    sb = np.ones(((N + 127) // 128, K // 128), np.float32)
    d = W.Dense(A, sa, B, sb)
    D = run_dense(d)
    assert_bit_exact(gpu_bits(D), oracle.gemm_nt(A, sa, B, sb), what="integer %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K", [(70, 300, 640), (64, 2112, 1024), (257, 390, 1024), (2048, 384, 512)])
def test_power_of_two_scales_bit_exact(M, N, K):
    """Integer codes with power-of-two block scales: every term and sum is exact in fp32, so a
    wrong K-block or N-block scale index (N=300/390/2112 straddle 128-blocks) changes bits."""
    rng = np.random.default_rng(M + N + K)
    A, B = int_codes(rng, (M, K)), int_codes(rng, (N, K))
    sa = (2.0 ** rng.integers(-1, 2, size=(M, K // 128))).astype(np.float32)
    sb = (2.0 ** rng.integers(-1, 2, size=((N + 127) // 128, K // 128))).astype(np.float32)
    D = run_dense(W.Dense(A, sa, B, sb))
    assert_bit_exact(gpu_bits(D), oracle.gemm_nt(A, sa, B, sb), what="pow2 %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K", [(1, 7, 128), (5, 130, 256), (17, 33, 384), (64, 64, 128),
                                   (100, 300, 640), (129, 257, 256), (300, 520, 1152),
                                   (1024, 512, 512), (1100, 384, 256), (2048, 640, 384)])
def test_random_ragged_shapes(M, N, K):
    d = W.dense(M, N, K, seed=M + 1000 * N + K)
    D = run_dense(d)
    rep = assert_close(gpu_bits(D), oracle.gemm_nt(d.A, d.sa, d.B, d.sb), what="%dx%dx%d" % (M, N, K))
    say("ragged", M, N, K, fg.last_config(), rep["bit_equal"])


@pytest.mark.parametrize("entry", [e for e in kernel_table() if e[5] == "kDense"],
                         ids=lambda e: "%dx%d_w%dx%d_s%d" % e[:5])
@pytest.mark.parametrize("split", [1, 3])
def test_every_dense_kernel_config(entry, split):
    bm, bn, wm, wn, st, _ = entry
    M, N, K = 2 * bm + 5, 2 * bn + 17, 1152
    d = W.dense(M, N, K, seed=bm * bn + split)
    ref = oracle.gemm_nt(d.A, d.sa, d.B, d.sb)
    with forced(bm, bn, wm, wn, st, split):
        D = run_dense(d)
        cfg = fg.last_config()
    assert "tile=%dx%d" % (bm, bn) in cfg, cfg
    assert_close(gpu_bits(D), ref, what=cfg)
    # integer inputs through the same configuration are bit-exact
    rng = np.random.default_rng(5)
    A, B = int_codes(rng, (M, K)), int_codes(rng, (N, K))
    sa = (2.0 ** rng.integers(-1, 2, size=(M, K // 128))).astype(np.float32)
    sb = (2.0 ** rng.integers(-1, 2, size=((N + 127) // 128, K // 128))).astype(np.float32)
    ref2 = oracle.gemm_nt(A, sa, B, sb)
    with forced(bm, bn, wm, wn, st, split):
        D2 = run_dense(W.Dense(A, sa, B, sb))
    assert_bit_exact(gpu_bits(D2), ref2, what=cfg)
    # a 3-CU cap makes every workgroup loop over several tiles (stage reuse across tiles)
    fg.set_num_cus(3)
    try:
        with forced(bm, bn, wm, wn, st, split):
            D3 = run_dense(W.Dense(A, sa, B, sb))
            cfg3 = fg.last_config()
    finally:
        fg.set_num_cus(0)
    units, grid = (int(x) for x in re.search(r"units=(\d+) grid=(\d+)", cfg3).groups())
    assert units > grid, cfg3
    assert_bit_exact(gpu_bits(D3), ref2, what=cfg3)


def test_output_guard_band_and_determinism():
    """No write outside D (canaries around it) and identical bits on repeated calls (split-K)."""
    d = W.dense(64, 2112, 7168, seed=77)
    M, N = 64, 2112
    pad = 4096
    buf = sentinel_tensor((M * N + 2 * pad,))
    D = buf[pad:pad + M * N].view(M, N)
    run_dense(d, out=D)
    b = gpu_bits(buf)
    assert np.all(b[:pad] == SENTINEL) and np.all(b[-pad:] == SENTINEL)
    first = gpu_bits(D).copy()
    for _ in range(3):
        run_dense(d, out=D)
        assert np.array_equal(gpu_bits(D), first)
    say("determinism", fg.last_config())


def test_cu_cap_and_side_stream():
    """A CU cap shrinks the persistent grid (it may change the split-K choice, hence the order of
    the fp32 partial sums: compared within tolerance); a side stream gives the same bits."""
    d = W.dense(200, 700, 1024, seed=78)
    ref_oracle = oracle.gemm_nt(d.A, d.sa, d.B, d.sb)
    ref = gpu_bits(run_dense(d))
    fg.set_num_cus(24)
    try:
        D = run_dense(d)
        cfg = fg.last_config()
    finally:
        fg.set_num_cus(0)
    assert_close(gpu_bits(D), ref_oracle, what=cfg)
    assert "grid=" in cfg and int(cfg.split("grid=")[1]) <= 24
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        D2 = fg.gemm_nt(dev(d.A), dev_sa(d.sa), dev(d.B), dev(d.sb))
    s.synchronize()
    assert np.array_equal(gpu_bits(D2), ref)


class streamk_on:
    """Stream-K wherever leftover tiles exist, inside the block (FP8GEMM_STREAMK=1)."""

    def __enter__(self):
        os.environ["FP8GEMM_STREAMK"] = "1"

    def __exit__(self, *exc):
        os.environ.pop("FP8GEMM_STREAMK", None)


def streamk_cus(tiles, nkb, at_least):
    """The smallest CU cap >= at_least that leaves leftover tiles with at least one K block per
    workgroup."""
    P = at_least
    while tiles % P == 0 or (tiles % P) * nkb < P:
        P += 1
    return P


@pytest.mark.parametrize("bn", [256, 192, 160])
@pytest.mark.parametrize("M,N,K,cus", [(1100, 700, 1280, 4), (1100, 700, 1280, 7), (600, 1030, 3840, 4),
                                       (777, 1500, 7168, 5), (300, 300, 1024, 2), (300, 256, 256, 3)])
def test_stream_k_leftover_tiles(bn, M, N, K, cus):
    """Tiles past the last full round taken stream-K (forced on, small CU caps): each leftover
    tile's K blocks are spread over 1 to 7 workgroups whose partials the last to arrive sums in K
    order (with two, the later segment folds the earlier one into its own accumulators; with one,
    the tile is whole in one range); ragged M and N tails.  Parity with the oracle, identical bits on a second call, and
    exact results for integer inputs with power-of-two scales."""
    tiles = -(-M // 256) * -(-N // bn)
    P = streamk_cus(tiles, K // 128, cus)
    d = W.dense(M, N, K, seed=M + N + K + bn)
    ref = oracle.gemm_nt(d.A, d.sa, d.B, d.sb)
    rng = np.random.default_rng(M + bn)
    A, B = int_codes(rng, (M, K)), int_codes(rng, (N, K))
    sa = (2.0 ** rng.integers(-1, 2, size=(M, K // 128))).astype(np.float32)
    sb = (2.0 ** rng.integers(-1, 2, size=((N + 127) // 128, K // 128))).astype(np.float32)
    ref2 = oracle.gemm_nt(A, sa, B, sb)
    fg.set_num_cus(P)
    try:
        with forced(256, bn, 4, 2, 2, 1), streamk_on():
            D = run_dense(d)
            cfg = fg.last_config()
            again = gpu_bits(run_dense(d)).copy()
            D2 = run_dense(W.Dense(A, sa, B, sb))
    finally:
        fg.set_num_cus(0)
    assert "streamk_tiles=" in cfg and "grid=%d " % P in cfg, cfg
    rep = assert_close(gpu_bits(D), ref, what=cfg)
    assert np.array_equal(again, gpu_bits(D)), cfg
    assert_bit_exact(gpu_bits(D2), ref2, what=cfg)
    say("stream-K", M, N, K, "cus", P, cfg, rep["bit_equal"])


@pytest.mark.parametrize("bn", [256, 192, 160])
@pytest.mark.parametrize("M,N,K,cus", [(1100, 1500, 1024, 4), (1024, 2048, 128, 3), (777, 1000, 512, 2),
                                       (513, 1001, 384, 2), (2048, 2048, 256, 5)])
def test_several_whole_tiles_per_workgroup(bn, M, N, K, cus):
    """Dense 256-row tiles, several whole tiles per workgroup (small CU caps, stream-K off): each
    workgroup runs tile after tile through the same ring and staging area, whole tiles followed by
    ragged ones and the reverse, one-slice tiles (K = 128), and N not a multiple of 8.  Parity with
    the oracle, identical bits on a second call, and exact results for integer inputs with
    power-of-two scales."""
    d = W.dense(M, N, K, seed=M + 3 * N + K + bn)
    ref = oracle.gemm_nt(d.A, d.sa, d.B, d.sb)
    rng = np.random.default_rng(M + 7 * bn)
    A, B = int_codes(rng, (M, K)), int_codes(rng, (N, K))
    sa = (2.0 ** rng.integers(-1, 2, size=(M, K // 128))).astype(np.float32)
    sb = (2.0 ** rng.integers(-1, 2, size=((N + 127) // 128, K // 128))).astype(np.float32)
    ref2 = oracle.gemm_nt(A, sa, B, sb)
    fg.set_num_cus(cus)
    os.environ["FP8GEMM_STREAMK"] = "0"
    try:
        with forced(256, bn, 4, 2, 2, 1):
            D = run_dense(d)
            cfg = fg.last_config()
            again = gpu_bits(run_dense(d)).copy()
            D2 = run_dense(W.Dense(A, sa, B, sb))
    finally:
        os.environ.pop("FP8GEMM_STREAMK", None)
        fg.set_num_cus(0)
    units = int(cfg.split("units=")[1].split()[0])
    assert "streamk" not in cfg and units >= 2 * cus, cfg
    rep = assert_close(gpu_bits(D), ref, what=cfg)
    assert np.array_equal(again, gpu_bits(D)), cfg
    assert_bit_exact(gpu_bits(D2), ref2, what=cfg)
    say("tiles per workgroup", M, N, K, "cus", cus, cfg, rep["bit_equal"])


@pytest.mark.parametrize("M,N,K,tile,streamk", [(4096, 1536, 7168, "256x192", True),
                                                  (4096, 2112, 7168, "256x192", True),
                                                  (4096, 4096, 7168, "256x256", False),
                                                  (4096, 2112, 1024, "256x160", False)])
def test_prefill_tile_width_choice(M, N, K, tile, streamk):
    """The N tile width of large dense launches: the least estimated time of the busiest
    workgroup under the schedule the launch runs (whole tiles or stream-K), so 256 x 192 with
    stream-K where 1536 or 2112 columns leave 256 x 256 tiles a partial round at long K, and the
    narrower whole tiles at short K.  Parity with the oracle on the full output."""
    d = W.dense(M, N, K, seed=M + N + K + 7)
    D = run_dense(d)
    cfg = fg.last_config()
    assert ("tile=%s " % tile) in cfg and (("streamk_tiles=" in cfg) == streamk), cfg
    rep = assert_close(gpu_bits(D), oracle.gemm_nt(d.A, d.sa, d.B, d.sb), what=cfg)
    say("width", M, N, K, cfg, rep["bit_equal"])


@pytest.mark.parametrize("cus", [96, 200, 250])
@pytest.mark.parametrize("M,N,K", [(2048, 1536, 4096), (1280, 2112, 3584)])
def test_prefill_widths_under_a_cu_cap(M, N, K, cus):
    """The width choice and the stream-K plan work from the capped CU count (caps that are not a
    multiple of 8 also switch the XCD remap off): the launch stays within the cap and matches the
    oracle, and a second call gives the same bits."""
    d = W.dense(M, N, K, seed=M + N + K + cus)
    ref = oracle.gemm_nt(d.A, d.sa, d.B, d.sb)
    fg.set_num_cus(cus)
    try:
        D = run_dense(d)
        cfg = fg.last_config()
        again = gpu_bits(run_dense(d)).copy()
    finally:
        fg.set_num_cus(0)
    assert "tile=256x" in cfg and int(cfg.split("grid=")[1].split()[0]) <= cus, cfg
    rep = assert_close(gpu_bits(D), ref, what=cfg)
    assert np.array_equal(again, gpu_bits(D)), cfg
    say("capped widths", M, N, K, cus, cfg, rep["bit_equal"])


def test_stream_k_off_matches_oracle_too():
    """The same leftover tiles as whole tiles (FP8GEMM_STREAMK=0): the schedule is a choice, both
    within tolerance of the oracle."""
    d = W.dense(1100, 700, 1280, seed=5)
    ref = oracle.gemm_nt(d.A, d.sa, d.B, d.sb)
    fg.set_num_cus(7)
    os.environ["FP8GEMM_STREAMK"] = "0"
    try:
        with forced(256, 256, 4, 2, 2, 1):
            D = run_dense(d)
            cfg = fg.last_config()
    finally:
        os.environ.pop("FP8GEMM_STREAMK", None)
        fg.set_num_cus(0)
    assert "streamk" not in cfg, cfg
    assert_close(gpu_bits(D), ref, what=cfg)


# ------------------------------------------------------------------------------------------
# grouped: contiguous
# ------------------------------------------------------------------------------------------

def run_contig(c, out=None):
    D = fg.grouped_contiguous(dev(c.A), dev_sa(c.sa), dev(c.B), dev(c.sb), dev(c.m_indices), out=out)
    torch.cuda.synchronize()
    return D


@pytest.mark.parametrize("counts,N,K", [([100, 0, 257, 128, 3], 320, 512), ([128], 256, 256),
                                        ([1, 1, 1], 64, 128), ([700, 300], 2112, 1024)])
def test_contiguous_parity_and_padding_untouched(counts, N, K):
    c = W.contiguous(counts, 0, N, K, seed=sum(counts) + N, packed=True)
    M = c.A.shape[0]
    out = sentinel_tensor((M, N))
    D = run_contig(c, out=out)
    ref, valid = oracle.grouped_contiguous(c.A, c.sa, c.B, c.sb, c.m_indices)
    v = valid.astype(bool)
    got = gpu_bits(D)
    rep = assert_close(got, ref, mask=v[:, None].repeat(N, 1), what="contiguous %s" % counts)
    assert np.all(got[~v] == SENTINEL), "padding rows were written"
    # refill the padding rows with other data: valid outputs keep their bits
    A2, sa2 = c.A.copy(), c.sa.copy()
    rng = np.random.default_rng(3)
    A2[~v] = W.random_codes(rng, (int((~v).sum()), K))
    sa2[~v] = 1e3
    D2 = run_contig(W.Contiguous(A2, sa2, c.B, c.sb, c.m_indices))
    assert np.array_equal(gpu_bits(D2)[v], got[v])
    assert fg.read_device_error() == 0
    say("contiguous", counts, fg.last_config(), rep["bit_equal"])


@pytest.mark.parametrize("entry", [e for e in kernel_table() if e[5] == "kContiguous"],
                         ids=lambda e: "%dx%d_w%dx%d_s%d" % e[:5])
@pytest.mark.parametrize("split", [1, 2])
def test_every_contiguous_kernel_config(entry, split):
    bm, bn, wm, wn, st, _ = entry
    c = W.contiguous([130, 0, 250], 0, 2 * bn + 40, 640, seed=bm + bn + split, packed=True)
    ref, valid = oracle.grouped_contiguous(c.A, c.sa, c.B, c.sb, c.m_indices)
    with forced(bm, bn, wm, wn, st, split):
        D = run_contig(c)
        cfg = fg.last_config()
    assert "tile=%dx%d" % (bm, bn) in cfg, cfg
    v = valid.astype(bool)
    assert_close(gpu_bits(D), ref, mask=v[:, None].repeat(D.shape[1], 1), what=cfg)


@pytest.mark.parametrize("split", [1, 2])
def test_contiguous_256_row_tiles_spanning_two_groups(split):
    """256-row tiles whose two 128-row blocks belong to different groups run one pass per group
    (rows of the other group not stored); tiles of one group, padding-only blocks, a ragged
    end; a 2-CU cap (several tiles per workgroup, passes reusing the LDS ring)."""
    c = W.contiguous([100, 0, 3, 128, 60, 250, 7], 0, 520, 640, seed=97 + split, packed=True)
    M, N = c.A.shape[0], 520
    ref, valid = oracle.grouped_contiguous(c.A, c.sa, c.B, c.sb, c.m_indices)
    v = valid.astype(bool)
    for cap in (0, 2):
        fg.set_num_cus(cap)
        try:
            with forced(256, 256, 4, 2, 2, split):
                D = run_contig(c, out=sentinel_tensor((M, N)))
                cfg = fg.last_config()
        finally:
            fg.set_num_cus(0)
        assert "tile=256x256" in cfg, cfg
        got = gpu_bits(D)
        assert_close(got, ref, mask=v[:, None].repeat(N, 1), what=cfg)
        assert np.all(got[~v] == SENTINEL), "padding rows were written"
    # integer codes, power-of-two scales: bit-exact through the two-pass tiles
    rng = np.random.default_rng(11)
    A, B = int_codes(rng, c.A.shape), int_codes(rng, c.B.shape)
    sa = (2.0 ** rng.integers(-1, 2, size=c.sa.shape)).astype(np.float32)
    sb = (2.0 ** rng.integers(-1, 2, size=c.sb.shape)).astype(np.float32)
    c2 = W.Contiguous(A, sa, B, sb, c.m_indices)
    ref2, _ = oracle.grouped_contiguous(A, sa, B, sb, c.m_indices)
    with forced(256, 256, 4, 2, 2, split):
        D2 = run_contig(c2)
    assert_bit_exact(gpu_bits(D2)[v], ref2[v], what="contiguous 256-row tiles, integer inputs")
    assert fg.read_device_error() == 0
    say("contiguous 256-row tiles", cfg)


def test_contiguous_equals_per_group_dense():
    c = W.contiguous([256, 384], 0, 512, 1024, seed=91, packed=True)
    D = gpu_bits(run_contig(c))
    for g in range(2):
        rows = np.nonzero(c.m_indices == g)[0]
        Dg = run_dense(W.Dense(c.A[rows], c.sa[rows], c.B[g], c.sb[g]))
        # the same rows through the dense entry point: equal within tolerance (launch shapes differ)
        assert_close(D[rows], gpu_bits(Dg), what="group %d" % g)


def test_contiguous_bad_index_flags_and_is_padding():
    c = W.contiguous([128, 128], 0, 128, 256, seed=92, packed=True)
    mi = c.m_indices.copy()
    mi[5] = 7           # out of range
    mi[200] = 0         # a group-0 row inside group 1's block
    out = sentinel_tensor(c.A.shape[:1] + (128,))
    D = fg.grouped_contiguous(dev(c.A), dev_sa(c.sa), dev(c.B), dev(c.sb), dev(mi), out=out)
    err = fg.read_device_error()
    assert err & fg.DEVERR_BAD_INDEX
    got = gpu_bits(D)
    assert np.all(got[5] == SENTINEL) and np.all(got[200] == SENTINEL)
    ref, valid = oracle.grouped_contiguous(c.A, c.sa, c.B, c.sb, c.m_indices)
    keep = np.ones(256, bool)
    keep[[5, 200]] = False
    assert_close(got[keep], ref[keep], what="bad index rows excluded")
    assert fg.read_device_error() == 0      # cleared by the read


# ------------------------------------------------------------------------------------------
# grouped: masked
# ------------------------------------------------------------------------------------------

def run_masked(w, expected_m, out=None):
    D = fg.grouped_masked(dev(w.A), dev_sa(w.sa), dev(w.B), dev(w.sb), dev(w.masked_m), expected_m, out=out)
    torch.cuda.synchronize()
    return D


@pytest.mark.parametrize("mm,M_max,N,K", [([0, 1, 64, 200, 130], 200, 192, 384),
                                          ([64, 64], 64, 4096, 256), ([3], 256, 100, 128)])
def test_masked_parity_rows_past_count_untouched(mm, M_max, N, K):
    w = W.masked(np.array(mm, np.int32), M_max, N, K, seed=sum(mm) + N)
    G = len(mm)
    ref, valid = oracle.grouped_masked(w.A, w.sa, w.B, w.sb, w.masked_m)
    v = valid.astype(bool)
    results = []
    for em in (1, 64, M_max):
        out = sentinel_tensor((G, M_max, N))
        D = run_masked(w, em, out=out)
        got = gpu_bits(D)
        assert_close(got, ref, mask=np.broadcast_to(v[:, :, None], got.shape), what="masked em=%d" % em)
        assert np.all(got[~v] == SENTINEL)
        results.append(got)
    assert fg.read_device_error() == 0
    say("masked", mm, fg.last_config())


@pytest.mark.parametrize("entry", [e for e in kernel_table() if e[5] == "kMasked"],
                         ids=lambda e: "%dx%d_w%dx%d_s%d" % e[:5])
@pytest.mark.parametrize("split", [1, 3])
def test_every_masked_kernel_config(entry, split):
    bm, bn, wm, wn, st, _ = entry
    w = W.masked(np.array([bm + 3, 0, 17, 2 * bm], np.int32), 2 * bm, 2 * bn + 24, 768, seed=bm * 3 + split)
    ref, valid = oracle.grouped_masked(w.A, w.sa, w.B, w.sb, w.masked_m)
    with forced(bm, bn, wm, wn, st, split):
        D = run_masked(w, 64)
        cfg = fg.last_config()
    assert "tile=%dx%d" % (bm, bn) in cfg, cfg
    got = gpu_bits(D)
    assert_close(got, ref, mask=np.broadcast_to(valid.astype(bool)[:, :, None], got.shape), what=cfg)


@pytest.mark.parametrize("entry", stream_table(), ids=stream_id)
@pytest.mark.parametrize("split", [1, 3])
def test_every_masked_decode_config(entry, split):
    """The masked decode kernel: counts past one tile (a second M tile), zero, a ragged last
    sub-tile and a full group; N off the tile and scale-block grid; K = 6 blocks (a short last
    A phase for 4-block phases); integer inputs bit-exact; one CU (several units per workgroup)."""
    mt, w, jn, kp, pf = entry
    bn = 16 * jn * w
    M_max = 2 * mt
    w_ = W.masked(np.array([mt + 3, 0, 17, M_max], np.int32), M_max, 2 * bn + 24, 768, seed=mt * 3 + split + bn)
    ref, valid = oracle.grouped_masked(w_.A, w_.sa, w_.B, w_.sb, w_.masked_m)
    out = sentinel_tensor((4, M_max, 2 * bn + 24))
    with forced_stream(mt, w, jn, kp, pf, split):
        D = run_masked(w_, 64, out=out)
        cfg = fg.last_config()
    assert "stream tile=%dx%d" % (mt, bn) in cfg, cfg
    got = gpu_bits(D)
    v = np.broadcast_to(valid.astype(bool)[:, :, None], got.shape)
    assert_close(got, ref, mask=v, what=cfg)
    assert np.all(got[~v] == SENTINEL), "rows past the count were written"
    # integer codes with power-of-two scales: exact, so bit-exact; rows past the counts hold
    # other codes (they must not leak into valid rows)
    rng = np.random.default_rng(mt + split)
    G, K, N = 4, 768, 2 * bn + 24
    A = int_codes(rng, (G, M_max, K))
    Bq = int_codes(rng, (G, N, K))
    sa = (2.0 ** rng.integers(-1, 2, size=(G, M_max, K // 128))).astype(np.float32)
    sb = (2.0 ** rng.integers(-1, 2, size=(G, (N + 127) // 128, K // 128))).astype(np.float32)
    mm = np.array([mt - 5, 1, mt + 17, 0], np.int32)
    ref2, valid2 = oracle.grouped_masked(A, sa, Bq, sb, mm)
    v2 = np.broadcast_to(valid2.astype(bool)[:, :, None], ref2.shape)
    fg.set_num_cus(1)
    try:
        with forced_stream(mt, w, jn, kp, pf, split):
            D2 = run_masked(W.Masked(A, sa, Bq, sb, mm, 64), 64, out=sentinel_tensor((G, M_max, N)))
            cfg2 = fg.last_config()
    finally:
        fg.set_num_cus(0)
    got2 = gpu_bits(D2)
    assert np.array_equal(got2[v2], ref2[v2]), cfg2
    assert np.all(got2[~v2] == SENTINEL)
    units, grid = (int(x) for x in re.search(r"units=(\d+) grid=(\d+)", cfg2).groups())
    assert units > grid, cfg2
    say("masked decode", cfg, cfg2)


def test_masked_count_out_of_range_clamps_and_flags():
    w = W.masked(np.array([64, 10], np.int32), 64, 128, 256, seed=93)
    mm = np.array([1000, -5], np.int32)
    D = fg.grouped_masked(dev(w.A), dev_sa(w.sa), dev(w.B), dev(w.sb), dev(mm), 64,
                          out=sentinel_tensor((2, 64, 128)))
    assert fg.read_device_error() & fg.DEVERR_BAD_COUNT
    ref, valid = oracle.grouped_masked(w.A, w.sa, w.B, w.sb, mm)
    got = gpu_bits(D)
    assert np.all(got[1] == SENTINEL)
    assert_close(got[0], ref[0], what="clamped count")


# ------------------------------------------------------------------------------------------
# full-size workloads: every valid output against the oracle
# ------------------------------------------------------------------------------------------
# Each call runs in the launch configuration the benchmark times (the library's own choice).
# rms(ref) in the tolerance is taken over all valid outputs of the call; each test records the
# share of bit-equal outputs and the bf16 ulp-distance histogram (printed; appended as a JSON
# line to $FP8GEMM_PARITY_REPORT when set).


@pytest.mark.slow
@pytest.mark.parametrize("mi", range(len(W.SWEEP_M)))
@pytest.mark.parametrize("nki", range(len(W.SWEEP_NK)))
def test_sweep_full_size(mi, nki):
    M, (N, K) = W.SWEEP_M[mi], W.SWEEP_NK[nki]
    say("sweep case", M, N, K)
    d = W.sweep_case(mi, nki)
    D = run_dense(d)
    cfg = fg.last_config()
    got = gpu_bits(D)
    ref = oracle.gemm_nt(d.A, d.sa, d.B, d.sb)
    rep = assert_close_full(got, ref, what="sweep %dx%dx%d [%s]" % (M, N, K, cfg))
    say("sweep", M, N, K, cfg, rep["bit_equal"], rep["ulp_histogram"])


@pytest.mark.slow
@pytest.mark.parametrize("cfg", [2, 3])
def test_contiguous_configs_full_size(cfg):
    say("contiguous config", cfg)
    c = W.config2() if cfg == 2 else W.config3()
    N = c.B.shape[1]
    out = sentinel_tensor((c.A.shape[0], N))
    D = run_contig(c, out=out)
    lc = fg.last_config()
    got = gpu_bits(D)
    valid = c.m_indices >= 0
    assert np.all(got[~valid] == SENTINEL)
    assert fg.read_device_error() == 0
    ref, v = oracle.grouped_contiguous(c.A, c.sa, c.B, c.sb, c.m_indices)
    assert np.array_equal(v.astype(bool), valid)
    rep = assert_close_full(got, ref, mask=np.broadcast_to(valid[:, None], got.shape),
                            what="contiguous config %d [%s]" % (cfg, lc))
    say("contiguous config", cfg, lc, rep["bit_equal"], rep["ulp_histogram"])


@pytest.mark.slow
def test_masked_config4_full_size():
    say("masked config 4")
    w = W.config4()
    G, M_max, K = w.A.shape
    N = w.B.shape[1]
    out = sentinel_tensor((G, M_max, N))
    D = run_masked(w, w.expected_m, out=out)
    lc = fg.last_config()
    got = gpu_bits(D)
    valid = np.arange(M_max)[None, :] < w.masked_m[:, None]
    v = np.broadcast_to(valid[:, :, None], got.shape)
    assert np.all(got[~v] == SENTINEL)
    assert fg.read_device_error() == 0
    ref, _ = oracle.grouped_masked(w.A, w.sa, w.B, w.sb, w.masked_m)
    rep = assert_close_full(got, ref, mask=v, what="masked config 4 [%s]" % lc)
    say("masked config 4", lc, rep["bit_equal"], rep["ulp_histogram"])
