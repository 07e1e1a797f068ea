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


# ---------------------------------------------------------------------------
# Shared mode: the plan launch (families, work items, worker ranges) and the
# workers' walk over the items, modelled as the kernels do them.
# ---------------------------------------------------------------------------

MIN_CHUNKS = 2  # a shorter common prefix does not form a family


def family_max(group):
    return 2 * (16 // group)


def shared_plan(lengths, tables, B, F, W):
    """Items [seq, members, fam or t0, t1, first chunk] and worker ranges, as
    the plan kernel lays them out."""
    S = len(lengths)
    nblk = [-(-L // B) for L in lengths]
    c = [0] * S
    for s in range(1, S):
        n = min(nblk[s], nblk[s - 1])
        k = 0
        while k < n and tables[s][k] == tables[s - 1][k]:
            k += 1
        c[s] = k
    link = [s > 0 and c[s] * B >= MIN_CHUNKS * CHUNK for s in range(S)]
    run = [0] * S
    for s in range(S):
        run[s] = s if not link[s] else run[s - 1]
    leader = [run[s] + F * ((s - run[s]) // F) for s in range(S)]
    fam_sf, fam_members = {}, {}
    for s in range(S):
        if leader[s] != s:
            continue
        g = 1
        cb, ml = 1 << 40, lengths[s] - 1
        while g < F and s + g < S and leader[s + g] == s:
            cb, ml = min(cb, c[s + g]), min(ml, lengths[s + g] - 1)
            g += 1
        sf = (min(cb * B, ml) // CHUNK) * CHUNK if g > 1 else 0
        if g < 2 or sf < MIN_CHUNKS * CHUNK:
            g, sf = 1, 0
        fam_members[s] = g
        for j in range(g):
            fam_sf[s + j] = sf
    items, chunk = [], 0
    fam = 0
    for s in range(S):
        sf = fam_sf[s]
        if leader[s] == s and fam_members[s] > 1:
            items.append((s, fam_members[s], fam, sf, chunk))   # t1 = sf
            chunk += sf // CHUNK
            fam += 1
        n = -(-(lengths[s] - sf) // CHUNK) if lengths[s] > sf else 0
        items.append((s, 1, sf, lengths[s], chunk))
        chunk += n
    return items, chunk, fam_sf


# the plan's cost estimate, in sixteenths of a one-group chunk
COST_CHUNK, COST_GROUP_CHUNK, COST_MEMBER_END, COST_ITEM_END = 16, 0, 8, 4


def item_chunks(it):
    seq, members, f_or_t0, t1, c = it
    t0 = 0 if members > 1 else f_or_t0
    return -(-(t1 - t0) // CHUNK) if t1 > t0 else 0


def shared_bounds(items, T, W, group):
    """Worker boundaries of the plan: boundary b where the estimated cost
    reaches b C / W', pulled towards the even split so that every worker
    keeps a chunk."""
    per = 16 // group
    cost, start_cost = 0, []
    rates = []
    for it in items:
        n, m = item_chunks(it), it[1]
        rate = COST_CHUNK + COST_GROUP_CHUNK * (-(-m // per)) if m > 1 else COST_CHUNK
        start_cost.append(cost)
        rates.append(rate)
        if m > 1:
            cost += n * rate + COST_MEMBER_END * m + COST_ITEM_END
        elif n > 0:
            cost += n * rate + COST_ITEM_END
    C, Wn = cost, min(W, T)
    starts = [it[4] for it in items] + [T]
    bounds = []
    for b in range(Wn + 1):
        x = T
        if b < Wn:
            X = b * C // Wn
            lo = max(i for i in range(len(items)) if start_cost[i] <= X)
            n = starts[lo + 1] - starts[lo]
            x = starts[lo] + min(n, (X - start_cost[lo]) // rates[lo])
        bounds.append(x * (T - Wn) // T + b)
    return bounds


def shared_walk(lengths, tables, B, group, W):
    S = len(lengths)
    F = family_max(group)
    items, T, fam_sf = shared_plan(lengths, tables, B, F, W)
    starts = [it[4] for it in items]
    pieces = {s: [] for s in range(S)}
    meta = {}
    if T == 0:
        return pieces, meta, fam_sf, F, 0
    Wn = min(W, T)
    bounds = shared_bounds(items, T, W, group)
    assert bounds[0] == 0 and bounds[-1] == T and all(b > a for a, b in zip(bounds, bounds[1:]))
    owner = lambda c: int(np.searchsorted(bounds, c, side="right") - 1)  # noqa: E731
    wmax = -(-2048 // 8)  # workspace bound used with 8 KV heads below
    fam_base = wmax + 2 * S
    for w in range(Wn):
        start, end = bounds[w], bounds[w + 1]
        i = int(np.searchsorted(starts, start, side="right") - 1)
        while i < len(items) and items[i][4] < end:
            seq, members, f_or_t0, t1, c = items[i]
            t0 = 0 if members > 1 else f_or_t0
            n = -(-(t1 - t0) // CHUNK) if t1 > t0 else 0
            if n == 0:
                i += 1
                continue
            c0, c1 = max(start, c), min(end, c + n)
            first, last = owner(c), owner(c + n - 1)
            a, b = t0 + (c0 - c) * CHUNK, min(t0 + (c1 - c) * CHUNK, t1)
            if members > 1:
                for m in range(members):
                    slot = fam_base + (w + f_or_t0) * F + m
                    pieces[seq + m].append(("fam", a, b, slot))
                    if c0 == c:
                        meta.setdefault(seq + m, {})["fam"] = (fam_base + (first + f_or_t0) * F + m, last - first + 1)
            else:
                pieces[seq].append(("own", a, b, w + i))
                if c0 == c:
                    meta.setdefault(seq, {})["own"] = (first + i, last - first + 1)
                    if t0 == 0:
                        meta[seq]["fam"] = (0, 0)
            i += 1
    return pieces, meta, fam_sf, F, fam_base


def forked_tables(rng, S, B):
    """Sequences forked from a few prompts (adjacent forks share the prompt's
    blocks, then diverge), with some lone sequences and some empty ones."""
    lengths, tables, nxt = [], [], [0]

    def fresh(k):
        out = list(range(nxt[0], nxt[0] + k))
        nxt[0] += k
        return out

    s = 0
    while s < S:
        forks = int(rng.integers(1, 12))
        plen = int(rng.integers(0, 400))
        prompt = fresh(-(-plen // B))
        for _ in range(min(forks, S - s)):
            own = int(rng.integers(0, 200))
            L = plen + own
            if plen % B and own:
                base = prompt[:-1] + fresh(1)   # copy-on-write of the partial last block
            else:
                base = list(prompt)
            tbl = base + fresh(-(-L // B) - len(base))
            lengths.append(L)
            tables.append(tbl)
            s += 1
    return lengths, tables


@pytest.mark.parametrize("B,group,W", [(16, 4, 128), (16, 4, 3), (8, 1, 64), (32, 8, 17), (16, 2, 1000),
                                       (128, 4, 50)])
def test_shared_plan_covers_each_token_once(B, group, W):
    rng = np.random.default_rng(B * 7 + group * 3 + W)
    for trial in range(40):
        S = int(rng.integers(1, 40))
        lengths, tables = forked_tables(rng, S, B)
        pieces, meta, fam_sf, F, fam_base = shared_walk(lengths, tables, B, group, W)
        slots = set()
        for s, L in enumerate(lengths):
            got = sorted(pieces[s], key=lambda x: x[1])
            covered = [t for (_, a, b, _) in got for t in range(a, b)]
            assert covered == list(range(L)), (lengths, s)
            sf = fam_sf[s]
            assert sf % CHUNK == 0 and (sf == 0 or sf <= L - 1)
            # a family's common prefix lies in blocks every member maps alike
            for (kind, a, b, _) in got:
                if kind == "fam":
                    leader = s
                    while leader > 0 and fam_sf.get(leader - 1) == sf and tables[leader - 1][:(b + B - 1) // B] == tables[s][:(b + B - 1) // B]:
                        leader -= 1
                    assert tables[leader][:(b + B - 1) // B] == tables[s][:(b + B - 1) // B]
            for (_, _, _, slot) in got:
                assert slot not in slots
                slots.add(slot)
            if L == 0:
                continue
            # the merge record names exactly the pieces that exist
            fam_first, fam_n = meta[s]["fam"]
            own_first, own_n = meta[s]["own"]
            fam_slots = sorted(x[3] for x in got if x[0] == "fam")
            own_slots = sorted(x[3] for x in got if x[0] == "own")
            assert fam_slots == [fam_first + k * F for k in range(fam_n)]
            assert own_slots == [own_first + k for k in range(own_n)]
            assert all(x < fam_base for x in own_slots)
            assert all(x < fam_base + (-(-2048 // 8) + len(lengths) // 2 + 1) * F for x in fam_slots)


def test_shared_plan_families_of_the_sampling_workload():
    # 32 prompts of 1016 tokens x 8 samples (B = 16): each prompt's samples
    # form one family (8 = 2 groups x 4 members at g = 4) over the first 992
    # tokens (the partial last prompt block is each sample's own copy)
    from paged_kv_cache_131_amd import workloads as wl

    ps = wl.ParallelSamplingWorkload(prompt_len=1016, values=False)
    st = ps.step()
    lengths = st.context_lens.tolist()
    tables = [list(st.block_tables[s, :-(-L // 16)]) for s, L in enumerate(lengths)]
    items, T, fam_sf = shared_plan(lengths, tables, 16, family_max(4), 128)
    fams = [it for it in items if it[1] > 1]
    assert len(fams) == 32 and all(it[1] == 8 and it[3] == 992 for it in fams)
    assert T == 32 * 31 + sum(-(-(L - 992) // CHUNK) for L in lengths)


def test_shared_bounds_weigh_families():
    # the sampling step's shape (32 prompts of 1016 tokens, 8 forks each
    # 256 tokens further on, B = 16, g = 4): families over 992 tokens, own
    # tails of 9 chunks. A worker on a family prefix gets fewer chunks than
    # one on the forks' own tails, every worker at least one.
    B, lengths, tables, nxt = 16, [], [], 0
    for _ in range(32):
        prompt = list(range(nxt, nxt + 63))
        nxt += 63
        for _ in range(8):
            L = 1016 + 256
            rest = -(-L // B) - 63
            tables.append(prompt + list(range(nxt, nxt + rest)))
            nxt += rest
            lengths.append(L)
    items, T, fam_sf = shared_plan(lengths, tables, B, family_max(4), 128)
    assert T == 32 * 31 + 256 * 9 and set(fam_sf.values()) == {992}
    bounds = shared_bounds(items, T, 128, 4)
    fam_chunks = set()
    for it in items:
        if it[1] > 1:
            fam_chunks.update(range(it[4], it[4] + item_chunks(it)))
    sizes = np.diff(bounds)
    on_fam = [w for w in range(128) if all(c in fam_chunks for c in range(bounds[w], bounds[w + 1]))]
    on_own = [w for w in range(128) if not any(c in fam_chunks for c in range(bounds[w], bounds[w + 1]))]
    assert on_fam and on_own and sizes.min() >= 1
    assert max(sizes[on_fam]) < min(sizes[on_own])
