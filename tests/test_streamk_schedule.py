"""The stream-K schedule of the dense 256-row tiles, restated in Python from its definition and
checked for the invariants the kernel relies on: the leftover tiles' K blocks are covered exactly
once, in order; a workgroup's range touches at most two tiles (segments 0 and 1, partial slots
2w and 2w + 1); a tile's segments come from consecutive workgroups, so the last to arrive can find
every partial (the owner of its first and last K block bound them); run segment 1 first, the
segments read K block j or j + (blocks per tile - blocks of the range) at step j whenever no tile
has more than two segments; and the host's choice takes stream-K only where it saves enough K
blocks.  No GPU is needed."""
import itertools

import pytest


def sk_start(w, per, extra):
    return w * per + min(w, extra)


def sk_owner(g, per, extra):
    big = extra * (per + 1)
    return g // (per + 1) if g < big else extra + (g - big) // per


def schedule(tiles, P, nkb):
    """(full rounds of whole tiles, leftover tiles, per, extra, segments) as the host and the
    kernel cut them; segments[w] = [(tile, kb0, nks), ...] for workgroup w."""
    full, R = divmod(tiles, P)
    per, extra = divmod(R * nkb, P)
    segs = {}
    for w in range(P):
        r0, r1 = sk_start(w, per, extra), sk_start(w + 1, per, extra)
        out = []
        for seg in (0, 1):
            g = r0 if seg == 0 else (r0 // nkb + 1) * nkb
            if g >= r1:
                continue
            t = g // nkb
            kb0 = g - t * nkb
            out.append((t, kb0, min(nkb - kb0, r1 - g), seg))
        segs[w] = out
    return full, R, per, extra, segs


CASES = [(T, P, nkb) for T, P, nkb in itertools.product(
    [1, 2, 5, 9, 17, 63, 191, 224, 257, 300, 448], [1, 3, 4, 7, 8, 64, 256], [1, 2, 3, 10, 16, 56, 128])]


@pytest.mark.parametrize("T,P,nkb", CASES)
def test_every_leftover_block_is_covered_once_and_in_order(T, P, nkb):
    full, R, per, extra, segs = schedule(T, P, nkb)
    if R == 0 or per < 1:
        return                      # the host keeps whole tiles then
    assert sk_start(P, per, extra) == R * nkb
    covered = []
    for w in range(P):
        assert len(segs[w]) <= 2
        for t, kb0, nks, seg in segs[w]:
            assert 0 <= t < R and 0 <= kb0 and nks >= 1 and kb0 + nks <= nkb
            covered.extend(t * nkb + k for k in range(kb0, kb0 + nks))
            assert 0 <= 2 * w + seg < 2 * P            # partial slot inside the workspace
    assert covered == list(range(R * nkb))


@pytest.mark.parametrize("T,P,nkb", CASES)
def test_a_tiles_segments_are_those_of_its_first_to_its_last_owner(T, P, nkb):
    full, R, per, extra, segs = schedule(T, P, nkb)
    if R == 0 or per < 1:
        return
    for t in range(R):
        wa, wb = sk_owner(t * nkb, per, extra), sk_owner(t * nkb + nkb - 1, per, extra)
        owners = [w for w in range(P) for (tt, _, _, _) in segs[w] if tt == t]
        assert owners == list(range(wa, wb + 1))
        # the slot the reducer computes for each owner is the one that owner wrote
        kb = 0
        for w in range(wa, wb + 1):
            seg = 0 if sk_start(w, per, extra) // nkb == t else 1
            (tt, kb0, nks, s), = [x for x in segs[w] if x[0] == t]
            assert s == seg and kb0 == kb
            kb += nks
        assert kb == nkb


def test_the_leftover_of_the_largest_sweep_shape_takes_stream_k():
    # 4096 x 7168 x 16384 in 256 x 256 tiles on 256 CUs: 448 tiles, 1.75 rounds
    full, R, per, extra, _ = schedule(16 * 28, 256, 128)
    assert (full, R, per, extra) == (1, 192, 96, 0)
    saved = 128 - per - (1 if extra else 0)
    assert saved >= 12                              # the host's threshold for 256 x 256 tiles
    # and the short-K shapes of the same tile count keep whole tiles
    full, R, per, extra, _ = schedule(16 * 28, 256, 16)
    assert 16 - per - (1 if extra else 0) < 12
    # 4096 x 2112 x 7168 in 256 x 160 tiles: 224 tiles, no full round, 7 blocks saved (threshold 6)
    full, R, per, extra, _ = schedule(16 * 14, 256, 56)
    assert (full, R) == (0, 224) and 56 - per - (1 if extra else 0) == 7 and 3 * per >= 56
    # 1024 x 2048 x 1024 in 256 x 160 tiles: 52 tiles of 8 K blocks, 1-2 blocks per workgroup --
    # 6 blocks saved, but a range is under a third of a tile: whole tiles
    full, R, per, extra, _ = schedule(4 * 13, 256, 8)
    assert 8 - per - (1 if extra else 0) >= 6 and 3 * per < 8


def steps(segs_w, nkb):
    """(step, K block) pairs of one workgroup, its segment 1 first as the kernel runs them."""
    out, j = [], 0
    for t, kb0, nks, seg in sorted(segs_w, key=lambda x: -x[3]):
        for k in range(kb0, kb0 + nks):
            out.append((j, k))
            j += 1
    return out


@pytest.mark.parametrize("T,P,nkb", CASES)
def test_two_k_phases_when_tiles_have_at_most_two_segments(T, P, nkb):
    full, R, per, extra, segs = schedule(T, P, nkb)
    if R == 0 or per < 1:
        return
    owners = {}
    for w in range(P):
        for t, _, _, _ in segs[w]:
            owners.setdefault(t, []).append(w)
    if max(len(o) for o in owners.values()) > 2:
        return
    for w in range(P):
        length = sk_start(w + 1, per, extra) - sk_start(w, per, extra)
        for j, k in steps(segs[w], nkb):
            assert k in (j, j + nkb - length), (w, j, k)
    # a tile then has two segments from consecutive workgroups (the later one folds the other in),
    # or one, when a range of per + 1 blocks is exactly a tile
    for t, o in owners.items():
        w_a, w_b = sk_owner(t * nkb, per, extra), sk_owner(t * nkb + nkb - 1, per, extra)
        assert o == sorted({w_a, w_b}) and w_b - w_a == len(o) - 1


def test_the_largest_sweep_shape_runs_in_two_phases():
    # 4096 x 7168 x 16384: 192 leftover tiles of 128 K blocks on 256 workgroups of 96 blocks each
    full, R, per, extra, segs = schedule(16 * 28, 256, 128)
    phases = set()
    for w in range(256):
        for j, k in steps(segs[w], 128):
            phases.add(k - j)
    assert phases == {0, 32}
