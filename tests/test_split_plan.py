"""Model of the decode kernel's balanced split, checked exhaustively on small
cases on the CPU: every 32-token chunk is covered by exactly one worker, the
pieces the merge waits for are exactly the workers that contribute to the
sequence, and partial-result slots are unique and inside the workspace the
host sizes (workers + sequences). Fixed partitions likewise."""

import itertools

import numpy as np
import pytest

CHUNK = 32


def balanced_plan(lengths, W):
    n = [(L + CHUNK - 1) // CHUNK if L > 0 else 0 for L in lengths]
    pref = np.concatenate([[0], np.cumsum(n)]).astype(np.int64)
    T = int(pref[-1])
    if T == 0:
        return {}, {}
    Wn = min(W, T)
    owner = lambda c: ((c + 1) * Wn - 1) // T  # noqa: E731
    pieces, expected = {}, {}
    for w in range(Wn):
        start, end = w * T // Wn, (w + 1) * T // Wn
        assert start < end
        # first sequence whose chunk range contains `start`
        s = int(np.searchsorted(pref, start, side="right") - 1)
        c = int(pref[s])
        while s < len(lengths) and c < end:
            if n[s] == 0:
                s += 1
                continue
            c0, c1 = max(start, c), min(end, c + n[s])
            first, last = owner(c), owner(c + n[s] - 1)
            pieces.setdefault(s, []).append((w, c0, c1, w + s))
            expected[s] = (first, last)
            c += n[s]
            s += 1
    return pieces, expected


@pytest.mark.parametrize("W", [1, 2, 3, 5, 8, 13, 64, 1000])
def test_balanced_split_covers_each_chunk_once(W):
    rng = np.random.default_rng(W)
    for trial in range(60):
        S = int(rng.integers(1, 12))
        lengths = rng.integers(0, 300, size=S).tolist()
        if trial % 7 == 0:
            lengths[0] = 0
        pieces, expected = balanced_plan(lengths, W)
        slots = set()
        for s, L in enumerate(lengths):
            n = (L + CHUNK - 1) // CHUNK
            if n == 0:
                assert s not in pieces
                continue
            got = sorted(pieces[s])
            covered = [c for (_, c0, c1, _) in got for c in range(c0, c1)]
            base = min(c0 for (_, c0, _, _) in got)
            assert covered == list(range(base, base + n))
            first, last = expected[s]
            workers = [w for (w, _, _, _) in got]
            assert workers == list(range(first, last + 1)), (lengths, W)
            for (_, _, _, slot) in got:
                assert slot not in slots and 0 <= slot < W + S
                slots.add(slot)


def test_fixed_partitions_cover_each_token_once():
    for L, P in itertools.product([1, 31, 32, 33, 511, 512, 513, 5000], [32, 64, 512]):
        max_parts = (L + P - 1) // P
        covered = []
        for part in range(max_parts):
            t0, t1 = part * P, min((part + 1) * P, L)
            if t0 < L:
                covered.extend(range(t0, t1))
        assert covered == list(range(L))


def partition_stream_plan(lengths, W, pc):
    """Fixed partitions of pc chunks taken in ranges: worker w runs every
    partition whose first chunk lies in its chunk range [w*T/Wn, (w+1)*T/Wn),
    walking the sequences from the one holding its first chunk, as the
    kernel's partition stream does."""
    n = [(L + CHUNK - 1) // CHUNK if L > 0 else 0 for L in lengths]
    pref = np.concatenate([[0], np.cumsum(n)]).astype(np.int64)
    T = int(pref[-1])
    runs = []
    if T == 0:
        return runs
    Wn = min(W, T)
    for w in range(Wn):
        start, end = w * T // Wn, (w + 1) * T // Wn
        s = int(np.searchsorted(pref, start, side="right") - 1)
        c, k = int(pref[s]), 0
        while s < len(lengths) and c < end:
            npart = (n[s] + pc - 1) // pc
            if c + k * pc < start:
                k = (start - c + pc - 1) // pc
            if k < npart:
                if c + k * pc >= end:
                    break
                runs.append((w, s, k))
                k += 1
                continue
            c += n[s]
            s += 1
            k = 0
    return runs


@pytest.mark.parametrize("W", [1, 2, 3, 7, 16, 128, 5000])
@pytest.mark.parametrize("pc", [1, 2, 16, 1000])
def test_partition_stream_runs_each_partition_once(W, pc):
    rng = np.random.default_rng(W * 7 + pc)
    for trial in range(40):
        S = int(rng.integers(1, 10))
        lengths = rng.integers(0, 2000, size=S).tolist()
        if trial % 5 == 0:
            lengths[-1] = 0
        runs = partition_stream_plan(lengths, W, pc)
        want = sorted((s, k) for s, L in enumerate(lengths)
                      for k in range(((L + CHUNK - 1) // CHUNK + pc - 1) // pc))
        assert sorted((s, k) for (_, s, k) in runs) == want
        # each worker's partitions come in stream order
        for w in {r[0] for r in runs}:
            mine = [(s, k) for (ww, s, k) in runs if ww == w]
            assert mine == sorted(mine)


def prefill_tile_map(q_start, total_q, qt, grid):
    """The prompt-phase kernel's tile map: workgroup x takes tile T-1-x of the
    tiles laid end to end over the sequences (ceil(n / qt) each; none for a
    sequence whose rows are not inside [0, total_q) in order)."""
    S = len(q_start) - 1
    nt = [(b - a + qt - 1) // qt if (a >= 0 and b > a and b <= total_q) else 0
          for a, b in zip(q_start[:-1], q_start[1:])]
    pref = np.concatenate([[0], np.cumsum(nt)]).astype(np.int64)
    T = int(pref[-1])
    out = []
    for x in range(grid):
        if x >= T:
            continue
        tile = T - 1 - x
        s = int(np.searchsorted(pref, tile, side="right") - 1)
        out.append((s, tile - int(pref[s])))
    assert S >= 0
    return out, nt


@pytest.mark.parametrize("g", [1, 2, 3, 4, 5, 8])
def test_prefill_tile_map_covers_each_tile_once(g):
    qt = max(1, 16 // g)
    rng = np.random.default_rng(g)
    for trial in range(50):
        S = int(rng.integers(1, 200))
        n = rng.integers(0, 300, size=S)
        if trial % 4 == 0:
            n[rng.integers(0, S)] = 0
        q_start = np.concatenate([[0], np.cumsum(n)]).astype(np.int64)
        total_q = int(q_start[-1])
        grid = -(-total_q // qt) + S               # the host's launch bound
        tiles, nt = prefill_tile_map(q_start.tolist(), total_q, qt, grid)
        assert sorted(tiles) == [(s, k) for s in range(S) for k in range(nt[s])]
        # the tile's queries stay inside the sequence's rows and its 16 columns
        for s, k in tiles:
            nq = min(qt, int(n[s]) - k * qt)
            assert 1 <= nq <= qt and nq * g <= 16
