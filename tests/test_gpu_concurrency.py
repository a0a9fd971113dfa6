"""GPU: the library used from several host threads at once, each thread on a stream of its own.

The split-K workspace and its arrival counters are kept per stream, the dispatcher's device state
is built once under a lock, and the last-configuration string is kept per thread.  So calls made
concurrently must give the same bits, and report the same launch configuration, as the same calls
made one at a time.  The cases are chosen so that each one splits K across workgroups: dense decode
shapes, a masked call whose groups times N tiles leave most CUs idle, and a dense 256-row-tile
shape that takes stream-K (2048 x 4096 x 7168: 208 tiles of 256 x 160, 45 K blocks per workgroup
on 256 CUs)."""
import sys
import threading

import numpy as np
import pytest

import workloads as W
from parity import gpu_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU runs deselect these with -m "not gpu"
    pytest.skip("needs a GPU", allow_module_level=True)

import fp8_block_scaled_x128_amd as fg  # noqa: E402

THREADS = 4
REPS = 6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def dev_sa(sa):
    return dev(np.swapaxes(sa, -1, -2))


def make_cases():
    """(name, call(stream, out), output shape) for each case; every call splits K."""
    cases = []
    for M, N, K, seed in ((64, 2112, 7168, 81), (64, 4096, 7168, 82), (128, 2112, 7168, 83), (100, 700, 1024, 84),
                          (2048, 4096, 7168, 86)):
        d = W.dense(M, N, K, seed=seed)
        ops = (dev(d.A), dev_sa(d.sa), dev(d.B), dev(d.sb))
        cases.append(("dense %dx%dx%d" % (M, N, K),
                      lambda s, out, ops=ops: fg.gemm_nt(*ops, out=out, stream=s), (M, N)))
    w = W.masked(np.array([37, 64], np.int32), 64, 512, 2048, seed=85)
    mops = (dev(w.A), dev_sa(w.sa), dev(w.B), dev(w.sb), dev(w.masked_m))
    cases.append(("masked 2x64x512x2048",
                  lambda s, out, ops=mops: fg.grouped_masked(*ops, 64, out=out, stream=s), (2, 64, 512)))
    return cases


def test_threads_on_their_own_streams_match_sequential_calls():
    cases = make_cases()
    ref, ref_cfg = [], []
    for name, call, shape in cases:
        out = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
        call(torch.cuda.current_stream(), out)
        torch.cuda.synchronize()
        ref.append(gpu_bits(out).copy())
        ref_cfg.append(fg.last_config())
        assert "split=1 " not in ref_cfg[-1] or "streamk_tiles=" in ref_cfg[-1], (name, ref_cfg[-1])
        if name == "dense 2048x4096x7168":
            assert "streamk_tiles=" in ref_cfg[-1], ref_cfg[-1]
        say(name, ref_cfg[-1])

    results, errors = {}, []

    def worker(t):
        try:
            s = torch.cuda.Stream()
            done = []
            with torch.cuda.stream(s):
                for r in range(REPS):
                    i = (t + r) % len(cases)
                    name, call, shape = cases[i]
                    out = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
                    call(s, out)
                    done.append((i, out, fg.last_config()))
            s.synchronize()
            results[t] = [(i, gpu_bits(out).copy(), cfg) for i, out, cfg in done]
        except Exception as e:  # reported below, in the main thread
            errors.append("thread %d: %r" % (t, e))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(THREADS)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    assert not errors, errors
    assert sorted(results) == list(range(THREADS))
    for t, done in results.items():
        for i, bits, cfg in done:
            assert cfg == ref_cfg[i], (t, cases[i][0], cfg, ref_cfg[i])
            assert np.array_equal(bits, ref[i]), "thread %d, %s: %d outputs differ" % (
                t, cases[i][0], int((bits != ref[i]).sum()))
    say("concurrent calls: %d threads x %d calls, all bit-identical to the sequential calls" % (THREADS, REPS))
