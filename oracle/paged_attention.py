"""Plain, slow, float64 reference for paged decode attention, the slot-mapped KV
write, the copy-on-write block copy, the swap of whole blocks to and from
host memory, and the prompt-phase (prefill) attention over the paged cache.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py. The library never calls it.

Sources (web pages on the SOSP'23 PagedAttention paper):
  [notes-zh] "PagedAttention 论文精读笔记" (pagedattention-sosp23-notes)
  [deep-dive] "paged-attention은 도대체 뭘 최적화 하는 것일까" (hrletsgo.me)
  [review-en] "PagedAttention paper review" (junupark.xyz)
  [review-kr] "Efficient Memory Management for Large Language Model Serving
              with PagedAttention Review" (dimensionstp.github.io)

Storage conventions (the library's ABI; the pages fix none of this):
  k_cache  [num_blocks][num_kv_heads][block_size][head_dim]   token-major tile
  v_cache  [num_blocks][num_kv_heads][head_dim][block_size]   token-minor tile,
           as an array shape; inside each tile the elements are sub-tiles
           [block_size/Bs][head_dim][Bs] with Bs = 32 when block_size is a
           multiple of 32 above 32, else Bs = block_size (plain
           [head_dim][block_size]; see v_slot)
  q        [num_seqs][num_heads][head_dim]
  block_tables [num_seqs][max_blocks_per_seq] int32, context_lens [num_seqs]
Element types: "f32" (numpy float32), "f16" (numpy float16) and "bf16"
(numpy uint16 holding the raw bfloat16 bit pattern). Every floating-point
step runs in float64 after an exact widening of the stored values.

Every function here is pinned by tests marked "not gpu" (worked examples from
the pages, closed forms, a library attention routine on contiguous data,
brute force and invariants); see tests/test_oracle_pins.py.
"""

from __future__ import annotations

import math

import numpy as np

ELEMENT_TYPES = ("f32", "f16", "bf16")


def to_float64(x: np.ndarray, etype: str) -> np.ndarray:
    """Exact widening of stored elements to float64.

    bf16 is the upper half of an IEEE binary32, so shifting the 16 raw bits
    left by 16 gives the same value as a binary32, which float64 holds exactly.
    """
    if etype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if etype == "f16":
        return np.asarray(x, dtype=np.float16).astype(np.float64)
    if etype == "bf16":
        raw = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return raw.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown element type {etype!r}")


# --------------------------------------------------------------------------
# Address translation: [deep-dive] §14 (steps a kernel takes) and §17
# (pseudocode: logical block = index // BLOCK_SIZE, offset = index %
# BLOCK_SIZE, physical block = block_table[logical block]).
# --------------------------------------------------------------------------

def translate(block_table_row, token_index: int, block_size: int):
    """Logical token position -> (physical block, offset in block)."""
    logical_block = token_index // block_size
    offset = token_index % block_size
    return int(block_table_row[logical_block]), offset


def v_slot(block_size: int, head_dim: int, offset: int):
    """Where the channels of in-block token `offset` lie in a V tile held as
    a [head_dim][block_size] array: the tile's elements are sub-tiles
    [block_size/Bs][head_dim][Bs], Bs = 32 for a multiple of 32 above 32,
    else Bs = block_size, so channel c of the token is flat element
    ((offset // Bs) * head_dim + c) * Bs + offset % Bs. Returns (rows,
    columns) index arrays of that array."""
    sub = 32 if block_size > 32 and block_size % 32 == 0 else block_size
    flat = ((offset // sub) * head_dim + np.arange(head_dim)) * sub + offset % sub
    return flat // block_size, flat % block_size


def write_kv(k_cache, v_cache, k_new, v_new, slot_mapping, block_size, inplace=False):
    """Slot-mapped store of new K/V rows ("fused reshape and block write",
    [review-kr] §3-2(5); new KV goes into its physical block, [notes-zh] §5.3).

    k_new, v_new: [num_tokens][num_kv_heads][head_dim] raw stored elements.
    slot_mapping[n] = physical_block * block_size + offset; a negative slot
    means "no write" (padding token). Returns new pools (the given ones,
    modified, when inplace=True). This is pure data movement, so the result is
    compared bit for bit.
    """
    k_out = k_cache if inplace else np.array(k_cache, copy=True)
    v_out = v_cache if inplace else np.array(v_cache, copy=True)
    for n, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        phys, off = divmod(int(slot), block_size)
        rows, cols = v_slot(block_size, v_out.shape[2], off)
        for h in range(k_out.shape[1]):
            k_out[phys, h, off, :] = k_new[n, h, :]
            v_out[phys, h, rows, cols] = v_new[n, h, :]
    return k_out, v_out


def copy_blocks(k_cache, v_cache, block_mapping, inplace=False):
    """Copy-on-write block copy ([notes-zh] §6.1: allocate a new physical
    block and copy the original block's data into it; batched as one fused
    copy, [review-kr] §3-2(5)). Whole blocks: every KV head, every slot, K and
    V. Pairs are applied in list order. Returns new pools (the given ones when
    inplace=True).
    """
    k_out = k_cache if inplace else np.array(k_cache, copy=True)
    v_out = v_cache if inplace else np.array(v_cache, copy=True)
    for src, dst in np.asarray(block_mapping).reshape(-1, 2).tolist():
        k_out[dst] = k_out[src]
        v_out[dst] = v_out[src]
    return k_out, v_out


def swap_out(k_cache, v_cache, host, block_mapping, inplace=False):
    """Swapping out ([notes-zh] §7.4: the blocks of an evicted sequence group
    are copied to CPU RAM, into slots a CPU block allocator hands out). For
    each (device block, host slot) pair, in list order, host slot j receives
    the block's whole K tile, every KV head, then its whole V tile, each
    flattened in the pool's own element order: host is
    [slots][2][num_kv_heads * block_size * head_dim]. Returns the new swap
    space (the given one when inplace=True)."""
    out = host if inplace else np.array(host, copy=True)
    for blk, slot in np.asarray(block_mapping).reshape(-1, 2).tolist():
        out[slot, 0] = k_cache[blk].reshape(-1)
        out[slot, 1] = v_cache[blk].reshape(-1)
    return out


def swap_in(k_cache, v_cache, host, block_mapping, inplace=False):
    """Swapping in ([notes-zh] §7.4: a resumed group's blocks are loaded back
    into GPU blocks, not necessarily the ones they left). For each (device
    block, host slot) pair, in list order, the block's K and V tiles are
    restored from the slot's two images. Returns new pools (the given ones
    when inplace=True)."""
    k_out = k_cache if inplace else np.array(k_cache, copy=True)
    v_out = v_cache if inplace else np.array(v_cache, copy=True)
    for blk, slot in np.asarray(block_mapping).reshape(-1, 2).tolist():
        k_out[blk] = host[slot, 0].reshape(k_out.shape[1:])
        v_out[blk] = host[slot, 1].reshape(v_out.shape[1:])
    return k_out, v_out


def gather_sequence(k_cache, v_cache, block_table_row, context_len, kv_head,
                    block_size, etype):
    """Token-by-token gather of one sequence's K and V for one KV head into
    contiguous float64 [L][head_dim] arrays, by block-table lookup."""
    head_dim = k_cache.shape[3]
    keys = np.empty((context_len, head_dim), dtype=np.float64)
    values = np.empty((context_len, head_dim), dtype=np.float64)
    for t in range(context_len):
        phys, off = translate(block_table_row, t, block_size)
        keys[t] = to_float64(k_cache[phys, kv_head, off, :], etype)
        rows, cols = v_slot(block_size, head_dim, off)
        values[t] = to_float64(v_cache[phys, kv_head, rows, cols], etype)
    return keys, values


def _check_shapes(q, k_cache, v_cache):
    num_heads = q.shape[1]
    num_kv_heads = k_cache.shape[1]
    if num_heads % num_kv_heads:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    if v_cache.shape[:2] != k_cache.shape[:2] or v_cache.shape[2] != k_cache.shape[3]:
        raise ValueError("v_cache must be [blocks][kv_heads][head_dim][block_size]")
    return num_heads // num_kv_heads


def decode_probabilities(q_row, keys, scale):
    """a_j = exp(scale * q.k_j) / sum_t exp(scale * q.k_t) ([notes-zh] §2.1,
    attention-score equation; the max is subtracted first, which leaves the
    ratio unchanged)."""
    scores = scale * (keys @ q_row)
    e = np.exp(scores - scores.max())
    return e / e.sum()


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
           etype, seqs=None, heads=None):
    """Exact single-query decode attention over a paged KV cache.

    For sequence s and query head h (grouped-query reading: KV head h // g with
    g = num_heads / num_kv_heads), with L = context_lens[s]:
        a_t = softmax_t(scale * q[s,h] . k_t),  o[s,h] = sum_t a_t v_t,
    where k_t, v_t are found through the block table ([notes-zh] §2.1 and
    §4.2; [deep-dive] §8: the paged layout does not change the result).

    Returns float64 [num_seqs][num_heads][head_dim]. With `seqs`/`heads`
    given, only those (s, h) pairs are computed (others stay NaN).
    """
    group = _check_shapes(q, k_cache, v_cache)
    num_seqs, num_heads, head_dim = q.shape
    out = np.full((num_seqs, num_heads, head_dim), np.nan, dtype=np.float64)
    seq_list = range(num_seqs) if seqs is None else seqs
    for s in seq_list:
        L = int(context_lens[s])
        if L < 1:
            raise ValueError(f"context length {L} of sequence {s}: attention over an empty context is undefined")
        head_list = range(num_heads) if heads is None else heads
        cache = {}
        for h in head_list:
            kvh = h // group
            if kvh not in cache:
                cache[kvh] = gather_sequence(k_cache, v_cache, block_tables[s], L,
                                             kvh, block_size, etype)
            keys, values = cache[kvh]
            a = decode_probabilities(to_float64(q[s, h], etype), keys, scale)
            out[s, h] = a @ values
    return out


def prefill(q, q_start, k_cache, v_cache, block_tables, context_lens, scale, block_size,
            etype, seqs=None):
    """Prompt-phase attention over a paged KV cache ([notes-zh] §2.2: every
    prompt token is processed at once and its K/V cached; §2.1: token i
    attends to tokens 1..i). Sequence s owns query rows q_start[s] ..
    q_start[s+1]-1 of q ([total_q][num_heads][head_dim]); with L =
    context_lens[s] and n of them, query j sits at position p = L - n + j (the
    last n tokens of the context; n = L for a whole prompt, fewer when the
    first tokens were cached before) and reads the cached tokens t <= p:
        a_t = softmax_{t <= p}(scale * q_j,h . k_t),  o_j,h = sum_{t <= p} a_t v_t,
    k_t, v_t found through the block table, grouped heads as in decode.

    Returns float64 [total_q][num_heads][head_dim]; rows of sequences not in
    `seqs` stay NaN.
    """
    group = _check_shapes(q, k_cache, v_cache)
    total_q, num_heads, head_dim = q.shape
    q_start = np.asarray(q_start)
    out = np.full((total_q, num_heads, head_dim), np.nan, dtype=np.float64)
    seq_list = range(len(q_start) - 1) if seqs is None else seqs
    for s in seq_list:
        L = int(context_lens[s])
        q0, q1 = int(q_start[s]), int(q_start[s + 1])
        n = q1 - q0
        if n < 1:
            continue
        if n > L:
            raise ValueError(f"sequence {s}: {n} queries but only {L} cached tokens")
        for kvh in range(num_heads // group):
            keys, values = gather_sequence(k_cache, v_cache, block_tables[s], L, kvh, block_size, etype)
            for j in range(n):
                p = L - n + j
                for h in range(kvh * group, (kvh + 1) * group):
                    a = decode_probabilities(to_float64(q[q0 + j, h], etype), keys[:p + 1], scale)
                    out[q0 + j, h] = a @ values[:p + 1]
    return out


def decode_blockwise(q, k_cache, v_cache, block_tables, context_lens, scale,
                     block_size, etype):
    """The block-wise form of the same attention ([notes-zh] §4.2): the
    context is cut into ceil(L/B) logical blocks K_j, V_j, the score row A_ij
    is formed per block, normalised by the sum over every block's
    exponentials, and o = sum_j V_j A_ij^T. The pages' denominator prints a
    vector; it is read as the scalar sum of every token's exponential (the
    only reading under which the block form equals the token form).
    """
    group = _check_shapes(q, k_cache, v_cache)
    num_seqs, num_heads, head_dim = q.shape
    out = np.empty((num_seqs, num_heads, head_dim), dtype=np.float64)
    for s in range(num_seqs):
        L = int(context_lens[s])
        nblk = -(-L // block_size)
        for h in range(num_heads):
            kvh = h // group
            qv = to_float64(q[s, h], etype)
            block_scores, block_values = [], []
            for j in range(nblk):
                phys = int(block_tables[s][j])
                used = min(block_size, L - j * block_size)
                Kj = to_float64(k_cache[phys, kvh, :used, :], etype)      # [used][d]
                cols_of = [v_slot(block_size, head_dim, off) for off in range(used)]
                Vj = np.stack([to_float64(v_cache[phys, kvh, r, c], etype) for r, c in cols_of], axis=1)  # [d][used]
                block_scores.append(scale * (Kj @ qv))
                block_values.append(Vj)
            top = max(sc.max() for sc in block_scores)
            exps = [np.exp(sc - top) for sc in block_scores]
            denom = sum(e.sum() for e in exps)
            o = np.zeros(head_dim)
            for Vj, e in zip(block_values, exps):
                o += Vj @ (e / denom)                                   # V_j A_ij^T
            out[s, h] = o
    return out


def decode_partitioned(q, k_cache, v_cache, block_tables, context_lens, scale,
                       block_size, etype, partition_size):
    """Attention computed partition by partition and then combined
    ([review-en] "How does this work?": compute per block, combine the
    partial results). Each partition p of `partition_size` tokens yields its
    local max m_p, local sum l_p = sum exp(s - m_p) and local output
    o_p = sum exp(s - m_p) v / l_p; the combination rescales by exp(m_p - M)
    with M = max_p m_p. Returns (out, partials) where partials[s][h] is the
    list of (m_p, l_p, o_p) in partition order.
    """
    group = _check_shapes(q, k_cache, v_cache)
    num_seqs, num_heads, head_dim = q.shape
    out = np.empty((num_seqs, num_heads, head_dim), dtype=np.float64)
    partials = []
    for s in range(num_seqs):
        L = int(context_lens[s])
        per_seq = []
        for h in range(num_heads):
            keys, values = gather_sequence(k_cache, v_cache, block_tables[s], L,
                                           h // group, block_size, etype)
            qv = to_float64(q[s, h], etype)
            parts = []
            for start in range(0, L, partition_size):
                sc = scale * (keys[start:start + partition_size] @ qv)
                m = sc.max()
                e = np.exp(sc - m)
                l = e.sum()
                parts.append((m, l, (e @ values[start:start + partition_size]) / l))
            M = max(m for m, _, _ in parts)
            weights = [l * math.exp(m - M) for m, l, _ in parts]
            total = sum(weights)
            out[s, h] = sum(wt * o for wt, (_, _, o) in zip(weights, parts)) / total
            per_seq.append(parts)
        partials.append(per_seq)
    return out, partials


def bruteforce_decode(q, k_cache, v_cache, block_tables, context_lens, scale,
                      block_size, etype):
    """Pure-Python loops (math.exp, no arrays in the arithmetic) for tiny
    inputs: every index is resolved one token at a time."""
    num_seqs, num_heads, head_dim = q.shape
    num_kv_heads = k_cache.shape[1]
    group = num_heads // num_kv_heads
    qf = to_float64(q, etype).tolist()
    kf = to_float64(k_cache, etype).tolist()
    vf = to_float64(v_cache, etype).tolist()
    out = [[[0.0] * head_dim for _ in range(num_heads)] for _ in range(num_seqs)]
    for s in range(num_seqs):
        L = int(context_lens[s])
        for h in range(num_heads):
            kvh = h // group
            scores = []
            for t in range(L):
                phys = int(block_tables[s][t // block_size])
                off = t % block_size
                dot = 0.0
                for i in range(head_dim):
                    dot += qf[s][h][i] * kf[phys][kvh][off][i]
                scores.append(scale * dot)
            top = max(scores)
            weights = [math.exp(x - top) for x in scores]
            total = sum(weights)
            sub = 32 if block_size > 32 and block_size % 32 == 0 else block_size
            for i in range(head_dim):
                acc = 0.0
                for t in range(L):
                    phys = int(block_tables[s][t // block_size])
                    off = t % block_size
                    flat = ((off // sub) * head_dim + i) * sub + off % sub
                    acc += weights[t] * vf[phys][kvh][flat // block_size][flat % block_size]
                out[s][h][i] = acc / total
    return np.array(out, dtype=np.float64)
