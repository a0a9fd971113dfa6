"""GPU: every entry point captured in a HIP graph and replayed.

Each call is made once eagerly on a stream into zeroed outputs, then captured on the same stream
(so its split-K workspace already exists), then the graph is replayed several times.  Between
replays the outputs are zeroed again by ordinary eager work and the device is synchronised.
Every replay must reproduce the eager result bit for bit.  The cases include split-K launches
(whose arrival counters the kernels reset themselves, with no memset node in the graph), the
masked decode kernel, E2M1 weights, the quantisers and the whole expert layer."""
import os
import sys

import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU runs deselect these with -m "not gpu"
    pytest.skip("needs a GPU", allow_module_level=True)

import fp8_block_scaled_x128_amd as fg  # noqa: E402

REPLAYS = 3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def dev_sa(sa):
    return dev(np.swapaxes(sa, -1, -2))


def bf16_dev(bits):
    return dev(bits.view(np.int16)).view(torch.bfloat16)


def raw(t):
    return t.detach().contiguous().view(torch.uint8).cpu().numpy().copy()


def replay_matches_eager(name, call, outs):
    """call(stream) writes the tensors in `outs`."""
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call(s)
    s.synchronize()
    ref = [raw(t) for t in outs]
    cfg = fg.last_config()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(s)
    for r in range(REPLAYS):
        for t in outs:      # back to the contents before the eager call (rows a call leaves alone stay so)
            t.view(torch.uint8).zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, t in enumerate(outs):
            got = raw(t)
            assert np.array_equal(got, ref[k]), "%s, replay %d, output %d: %d bytes differ (%s)" % (
                name, r, k, int((got != ref[k]).sum()), cfg)
    assert fg.read_device_error() == 0
    del g
    say("graph", name, cfg)


@pytest.mark.parametrize("M,N,K", [(64, 2112, 7168), (100, 700, 1024), (1024, 512, 512), (300, 1000, 384)])
def test_dense(M, N, K):
    d = W.dense(M, N, K, seed=M + N + K)
    ops = (dev(d.A), dev_sa(d.sa), dev(d.B), dev(d.sb))
    D = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    replay_matches_eager("dense %dx%dx%d" % (M, N, K), lambda s: fg.gemm_nt(*ops, out=D, stream=s), [D])


def test_contiguous():
    c = W.contiguous([100, 0, 3, 128, 60, 250, 7], 0, 520, 640, seed=31, packed=True)
    ops = (dev(c.A), dev_sa(c.sa), dev(c.B), dev(c.sb), dev(c.m_indices))
    D = torch.zeros((c.A.shape[0], 520), dtype=torch.bfloat16, device="cuda")
    replay_matches_eager("contiguous", lambda s: fg.grouped_contiguous(*ops, out=D, stream=s), [D])


@pytest.mark.parametrize("mm,M_max,N,K", [([37, 64], 64, 512, 2048), ([0, 1, 64, 200, 130], 200, 192, 384),
                                          ([70, 90, 5, 128], 128, 1024, 1024)])
def test_masked(mm, M_max, N, K):
    w = W.masked(np.array(mm, np.int32), M_max, N, K, seed=sum(mm) + N)
    ops = (dev(w.A), dev_sa(w.sa), dev(w.B), dev(w.sb), dev(w.masked_m))
    D = torch.zeros((len(mm), M_max, N), dtype=torch.bfloat16, device="cuda")
    replay_matches_eager("masked %s" % mm, lambda s: fg.grouped_masked(*ops, 64, out=D, stream=s), [D])


@pytest.mark.parametrize("mm,M_max,N,K", [([32, 20], 32, 160, 512), ([0, 1, 64, 200, 130], 200, 192, 384)])
def test_fp8fp4_masked(mm, M_max, N, K):
    w = W.masked_fp4(np.array(mm, np.int32), M_max, N, K, seed=sum(mm) + N + 5)
    ops = (dev(w.A), dev_sa(w.sa), dev(w.B), dev(w.sb), dev(w.masked_m))
    D = torch.zeros((len(mm), M_max, N), dtype=torch.bfloat16, device="cuda")
    replay_matches_eager("fp8xfp4 masked %s" % mm, lambda s: fg.fp8fp4_grouped_masked(*ops, 64, out=D, stream=s),
                         [D])


def test_quantisers():
    X = bf16_dev(W.activations_bf16(300, 1024, seed=7))
    codes = torch.zeros((300, 1024), dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
    scales = torch.zeros((8, 300), dtype=torch.float32, device="cuda")
    replay_matches_eager("quantize", lambda s: fg.quantize_1x128(X, codes=codes, scales=scales, stream=s),
                         [codes, scales])
    G, M_max, K = 3, 40, 512
    Xm = bf16_dev(W.activations_bf16(G * M_max, K, seed=8).reshape(G, M_max, K))
    mm = dev(np.array([40, 0, 17], np.int32))
    cm = torch.zeros((G, M_max, K), dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
    sm = torch.zeros((G, K // 128, M_max), dtype=torch.float32, device="cuda")
    replay_matches_eager("quantize masked",
                         lambda s: fg.quantize_1x128_masked(Xm, mm, codes=cm, scales=sm, stream=s), [cm, sm])
    Y = bf16_dev(W.swiglu_input_bf16(257, 640, seed=9))
    cy = torch.zeros((257, 640), dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
    sy = torch.zeros((5, 257), dtype=torch.float32, device="cuda")
    replay_matches_eager("swiglu quantize", lambda s: fg.swiglu_quantize_1x128(Y, codes=cy, scales=sy, stream=s),
                         [cy, sy])


def test_moe_expert_chain():
    mm = np.array([70, 0, 33], np.int32)
    G, M_max, H, I = 3, 80, 256, 384
    e = W.moe_expert(mm, M_max, H, I, seed=11, expected_m=64)
    ops = (dev(e.A), dev_sa(e.sa), dev(e.W1), dev(e.s1), dev(e.W2), dev(e.s2), dev(e.masked_m))
    out = torch.zeros((G, M_max, H), dtype=torch.bfloat16, device="cuda")
    ws = (torch.zeros((G, M_max, 2 * I), dtype=torch.bfloat16, device="cuda"),
          torch.zeros((G, M_max, I), dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn),
          torch.zeros((G, I // 128, M_max), dtype=torch.float32, device="cuda"))
    replay_matches_eager("moe expert chain",
                         lambda s: fg.moe_expert_masked(*ops, 64, out=out, workspace=ws, stream=s), [out])


def test_split_k_graph_survives_a_larger_call():
    """A split-K call captured on a prepared stream keeps its workspace: a larger split-K call on
    the same stream afterwards (more and wider partial tiles) neither frees nor moves it, so the
    graph's replays still give the bits of the first replay, which match the oracle."""
    import oracle
    from parity import assert_close, gpu_bits

    s = torch.cuda.Stream()
    fg.prepare_stream(s)
    small = W.dense(64, 2112, 7168, seed=501)
    ops = (dev(small.A), dev_sa(small.sa), dev(small.B), dev(small.sb))
    D = torch.zeros((64, 2112), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):        # no eager call first: the prepared stream suffices
        fg.gemm_nt(*ops, out=D, stream=s)
    cfg_small = fg.last_config()
    assert "split=1 " not in cfg_small, cfg_small
    g.replay()
    torch.cuda.synchronize()
    ref = raw(D)
    assert_close(gpu_bits(D), oracle.gemm_nt(small.A, small.sa, small.B, small.sb), what=cfg_small)
    big = W.dense(128, 7168, 16384, seed=502)
    with torch.cuda.stream(s):
        D2 = fg.gemm_nt(dev(big.A), dev_sa(big.sa), dev(big.B), dev(big.sb), stream=s)
    s.synchronize()
    cfg_big = fg.last_config()
    assert "split=1 " not in cfg_big, cfg_big
    assert_close(gpu_bits(D2), oracle.gemm_nt(big.A, big.sa, big.B, big.sb), what=cfg_big)
    for r in range(REPLAYS):
        D.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(raw(D), ref), "replay %d after a larger split-K call (%s, %s)" % (r, cfg_small, cfg_big)
    del g
    say("graph survives larger call", cfg_small, "|", cfg_big)


def test_split_k_capture_on_unprepared_stream_is_refused():
    """A split-K call captured on a stream that has no workspace yet returns UNSUPPORTED before
    anything is enqueued (the library allocates nothing during capture); after
    fp8gemm_prepare_stream the same capture succeeds."""
    import ctypes

    hip = ctypes.CDLL("libamdhip64.so")
    lib = fg.lib()
    d = W.dense(64, 2112, 1024, seed=503)
    ops = (dev(d.A), dev_sa(d.sa), dev(d.B), dev(d.sb))
    D = torch.zeros((64, 2112), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    s = ctypes.c_void_p()
    assert hip.hipStreamCreate(ctypes.byref(s)) == 0
    try:
        def capture():
            graph = ctypes.c_void_p()
            assert hip.hipStreamBeginCapture(s, 2) == 0          # relaxed mode
            rc = lib.fp8gemm_nt(*[t.data_ptr() for t in ops], D.data_ptr(), 64, 2112, 1024, s)
            assert hip.hipStreamEndCapture(s, ctypes.byref(graph)) == 0
            assert hip.hipGraphDestroy(graph) == 0
            return rc
        assert capture() == 4                                    # FP8GEMM_ERR_UNSUPPORTED
        assert lib.fp8gemm_prepare_stream(s) == 0
        assert capture() == 0
    finally:
        assert hip.hipStreamSynchronize(s) == 0
        assert hip.hipStreamDestroy(s) == 0
    say("unprepared capture refused, prepared capture accepted")


def test_stream_k_graph_replays():
    """A stream-K launch (leftover 256 x 256 tiles spread over 7 workgroups each, forced on a
    7-CU cap) captured after an eager call on the same stream: every replay gives the eager bits,
    so the arrival counters are back at zero after each launch."""
    d = W.dense(1100, 700, 1280, seed=504)
    ops = (dev(d.A), dev_sa(d.sa), dev(d.B), dev(d.sb))
    D = torch.zeros((1100, 700), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    os.environ["FP8GEMM_STREAMK"] = "1"
    os.environ["FP8GEMM_FORCE_CONFIG"] = "256x256:4x2:2:1"
    fg.set_num_cus(7)
    try:
        replay_matches_eager("stream-K 1100x700x1280", lambda s: fg.gemm_nt(*ops, out=D, stream=s), [D])
        cfg = fg.last_config()
    finally:
        fg.set_num_cus(0)
        os.environ.pop("FP8GEMM_FORCE_CONFIG", None)
        os.environ.pop("FP8GEMM_STREAMK", None)
    assert "streamk_tiles=" in cfg, cfg


def test_default_stream_k_graph_replays():
    """A launch that takes stream-K by the library's own choice (2048 x 4096 x 7168 on the whole
    device: 256-row tiles in less than one round), captured and replayed several times with eager
    work between the replays: every replay gives the eager bits."""
    M, N, K = 2048, 4096, 7168
    d = W.dense(M, N, K, seed=506)
    ops = (dev(d.A), dev_sa(d.sa), dev(d.B), dev(d.sb))
    D = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    replay_matches_eager("default stream-K %dx%dx%d" % (M, N, K), lambda s: fg.gemm_nt(*ops, out=D, stream=s), [D])
    cfg = fg.last_config()
    assert "streamk_tiles=" in cfg, cfg


def test_stream_k_capture_on_unprepared_stream_keeps_whole_tiles():
    """Stream-K needs the stream's workspace, which is never allocated during capture: on a
    stream with none, the captured launch keeps whole tiles (no error) and its graph computes the
    product; once the stream is prepared, the same capture takes stream-K."""
    import ctypes

    import oracle
    from parity import assert_close, gpu_bits

    hip = ctypes.CDLL("libamdhip64.so")
    lib = fg.lib()
    M, N, K = 1100, 700, 1280
    d = W.dense(M, N, K, seed=505)
    ops = (dev(d.A), dev_sa(d.sa), dev(d.B), dev(d.sb))
    D = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    ref = oracle.gemm_nt(d.A, d.sa, d.B, d.sb)
    torch.cuda.synchronize()
    s = ctypes.c_void_p()
    assert hip.hipStreamCreate(ctypes.byref(s)) == 0
    os.environ["FP8GEMM_STREAMK"] = "1"
    os.environ["FP8GEMM_FORCE_CONFIG"] = "256x256:4x2:2:1"
    fg.set_num_cus(7)
    try:
        def capture_and_run():
            graph, exe = ctypes.c_void_p(), ctypes.c_void_p()
            assert hip.hipStreamBeginCapture(s, 2) == 0          # relaxed mode
            rc = lib.fp8gemm_nt(*[t.data_ptr() for t in ops], D.data_ptr(), M, N, K, s)
            assert hip.hipStreamEndCapture(s, ctypes.byref(graph)) == 0
            cfg = fg.last_config()
            if rc == 0:
                assert hip.hipGraphInstantiate(ctypes.byref(exe), graph, None, None, 0) == 0
                assert hip.hipGraphLaunch(exe, s) == 0
                assert hip.hipStreamSynchronize(s) == 0
                assert hip.hipGraphExecDestroy(exe) == 0
            assert hip.hipGraphDestroy(graph) == 0
            return rc, cfg
        rc, cfg = capture_and_run()
        assert rc == 0 and "streamk" not in cfg, (rc, cfg)
        assert_close(gpu_bits(D), ref, what=cfg)
        assert lib.fp8gemm_prepare_stream(s) == 0
        D.zero_()
        torch.cuda.synchronize()
        rc, cfg = capture_and_run()
        assert rc == 0 and "streamk_tiles=" in cfg, (rc, cfg)
        assert_close(gpu_bits(D), ref, what=cfg)
    finally:
        fg.set_num_cus(0)
        os.environ.pop("FP8GEMM_FORCE_CONFIG", None)
        os.environ.pop("FP8GEMM_STREAMK", None)
        assert hip.hipStreamSynchronize(s) == 0
        assert hip.hipStreamDestroy(s) == 0
    say("unprepared capture keeps whole tiles, prepared capture takes stream-K")
