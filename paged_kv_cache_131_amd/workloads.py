"""Seeded synthetic inputs for paged decode attention.

This module holds no attention arithmetic: it draws random numbers, rounds
them to the stored element type, places sequences into a shuffled block pool
and poisons every slot the decode must not read with NaN. The same arrays feed
both the CPU oracle (in tests) and the device library.

Recipe per workload k (seed 1000 + k): numpy.random.SeedSequence(seed) spawns
six streams, used in this order: lengths, pool permutation, q, K pool, V pool,
new-token K/V. Values are float32 standard normals times `value_scale`,
rounded to nearest-even into the stored type; an array is drawn in slices of
2**22 elements, slice i from the i-th child of its stream (so slices can be
drawn in parallel and the values do not depend on the thread count). Pools hold 10% more blocks than
the sequences need (the tiny workload has a fixed pool of 32) and hand them out
in the order of a seeded permutation, as on-demand allocation from a shuffled
free pool would.

Stored element types: "f32" -> float32, "f16" -> float16, "bf16" -> uint16
holding the raw bfloat16 bits.
"""

from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

from .block_manager import BlockManager

STORED_DTYPE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
ELEMENT_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
# quiet NaNs with a payload, so that bit-exact copies can be told apart from
# re-generated NaNs
POISON_BITS = {"f32": 0x7FC00123, "f16": 0x7E23, "bf16": 0x7FC3}
_SLICE = 1 << 22  # values drawn per slice (bounds temporary memory)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns raw bits.
    Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def round_to(x: np.ndarray, etype: str) -> np.ndarray:
    if etype == "f32":
        return np.asarray(x, dtype=np.float32)
    if etype == "f16":
        return np.asarray(x, dtype=np.float32).astype(np.float16)
    if etype == "bf16":
        return bf16_bits_from_f32(x)
    raise ValueError(etype)


def poison_value(etype: str):
    bits = POISON_BITS[etype]
    if etype == "f32":
        return np.array([bits], dtype=np.uint32).view(np.float32)[0]
    if etype == "f16":
        return np.array([bits], dtype=np.uint16).view(np.float16)[0]
    return np.uint16(bits)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def set_v_tokens(v_cache: np.ndarray, block: int, first: int, value) -> None:
    """Set in-block tokens first.. of a block's V tiles (every KV head, every
    channel) to value. A V tile, held as a [head_dim][block_size] array, is
    stored as sub-tiles [block_size/Bs][head_dim][Bs] with Bs = 32 for a
    multiple of 32 above 32, else Bs = block_size (plain [head_dim][block_size])."""
    Hkv, d, B = v_cache.shape[1:]
    Bs = 32 if B > 32 and B % 32 == 0 else B
    tiles = v_cache[block].reshape(Hkv, B // Bs, d, Bs)
    for t in range(first, B):
        tiles[:, t // Bs, :, t % Bs] = value


def random_stored(seq: np.random.SeedSequence, shape, etype: str, value_scale: float) -> np.ndarray:
    """Standard normals * value_scale rounded to `etype`; slice i of 2**22
    values comes from the i-th child of `seq`."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=STORED_DTYPE[etype])
    nslices = -(-n // _SLICE)
    children = seq.spawn(nslices)

    def fill(i):
        lo, hi = i * _SLICE, min(n, (i + 1) * _SLICE)
        x = np.random.default_rng(children[i]).standard_normal(hi - lo, dtype=np.float32)
        if value_scale != 1.0:
            x *= np.float32(value_scale)
        out[lo:hi] = round_to(x, etype)

    if nslices <= 1:
        for i in range(nslices):
            fill(i)
    else:
        with ThreadPoolExecutor(_threads()) as pool:
            list(pool.map(fill, range(nslices)))
    return out.reshape(shape)


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    index: int                 # seed = 1000 + index
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    etype: str
    value_scale: float
    lengths: tuple             # ("fixed", values) | ("uniform", lo, hi) | ("lognormal", median, sigma, lo, hi)
    max_len: int               # upper bound of the length law: sizes block tables
    pool_blocks: int = 0       # 0 = ceil(1.1 * blocks needed)
    partition_size: int = -1   # -1 = balanced split; -2 = shared split (forks read their common blocks once)

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


CONFIGS = {
    "tiny": DecodeConfig("tiny", 1, 4, 2, 2, 64, 16, "f32", 1.0,
                         ("fixed", (5, 17, 33, 64)), 64, pool_blocks=32),
    "opt13b": DecodeConfig("opt13b", 2, 64, 40, 40, 128, 16, "f16", 0.5,
                           ("uniform", 128, 2048), 2048),
    "llama3_8b": DecodeConfig("llama3_8b", 3, 256, 32, 8, 128, 16, "bf16", 1.0,
                              ("lognormal", 800.0, 1.0, 16, 8192), 8192),
    "long_context": DecodeConfig("long_context", 5, 16, 64, 8, 128, 32, "bf16", 1.0,
                                 ("uniform", 32768, 131072), 131072, partition_size=512),
}


def draw_lengths(cfg: DecodeConfig, rng: np.random.Generator) -> np.ndarray:
    kind = cfg.lengths[0]
    if kind == "fixed":
        lens = np.array(cfg.lengths[1], dtype=np.int64)
    elif kind == "uniform":
        lens = rng.integers(cfg.lengths[1], cfg.lengths[2] + 1, size=cfg.num_seqs)
    elif kind == "lognormal":
        median, sigma, lo, hi = cfg.lengths[1:]
        lens = np.rint(np.exp(rng.normal(math.log(median), sigma, size=cfg.num_seqs)))
        lens = np.clip(lens, lo, hi)
    else:
        raise ValueError(kind)
    return lens.astype(np.int32)


@dataclass
class DecodeWorkload:
    """One decode step's inputs. `k_cache`/`v_cache` hold the context's first
    L-1 tokens; the new token (position L-1) arrives in `k_new`/`v_new` and is
    stored at `slot_mapping` before the decode reads it."""
    cfg: DecodeConfig
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    block_tables: np.ndarray
    context_lens: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray
    slot_mapping: np.ndarray
    num_blocks: int
    poison_block: int
    used_blocks: np.ndarray = field(default=None)
    # Copy-on-write replay (a shared prefix that ends inside a block): the
    # pools then hold the state before the copies. Apply copy_pairs, then
    # store pre_k/pre_v at pre_slots (the tokens that landed in the copies),
    # then the new token.
    copy_pairs: np.ndarray = field(default=None)
    pre_slots: np.ndarray = field(default=None)
    pre_k: np.ndarray = field(default=None)
    pre_v: np.ndarray = field(default=None)

    @property
    def etype(self):
        return self.cfg.etype

    @property
    def max_blocks_per_seq(self):
        return self.block_tables.shape[1]

    @property
    def max_context_len(self):
        return int(self.context_lens.max())

    def kv_bytes(self) -> int:
        c = self.cfg
        return int(self.context_lens.astype(np.int64).sum()) * c.num_kv_heads * c.head_dim * 2 * ELEMENT_BYTES[c.etype]


def make_decode_workload(cfg: DecodeConfig, lengths=None, poison: bool = True,
                         values: bool = True, contiguous: bool = False, reserved: bool = False) -> DecodeWorkload:
    """Draw one decode step's inputs. With values=False only the integer
    inputs (lengths, block tables, slot mapping) are produced. contiguous=True
    hands the pool's blocks out in order (sequence s's blocks adjacent, after
    those of s-1) instead of in the seeded shuffled order. reserved=True gives
    every sequence a region of max_blocks blocks of its own (sequence s's
    logical block i is block s * max_blocks + i), the maximum-length
    reservation that paging replaces; the pool then holds num_seqs *
    max_blocks blocks plus one never handed out."""
    if contiguous and reserved:
        raise ValueError("contiguous and reserved are two different layouts")
    seqs = np.random.SeedSequence(1000 + cfg.index).spawn(6)
    rng_len, rng_pool = np.random.default_rng(seqs[0]), np.random.default_rng(seqs[1])
    ss_q, ss_k, ss_v, ss_new = seqs[2:]
    lens = draw_lengths(cfg, rng_len) if lengths is None else np.asarray(lengths, dtype=np.int32)
    if lens.shape != (cfg.num_seqs,) or lens.min() < 1:
        raise ValueError("one positive length per sequence is required")
    B = cfg.block_size
    nblk = -(-lens.astype(np.int64) // B)
    need = int(nblk.sum())
    max_blocks = max(-(-cfg.max_len // B), int(nblk.max()))
    if reserved:
        num_blocks = cfg.num_seqs * max_blocks + 1
        poison_block = num_blocks - 1
        tables = np.full((cfg.num_seqs, max_blocks), poison_block, dtype=np.int32)
        for s in range(cfg.num_seqs):
            tables[s, :nblk[s]] = s * max_blocks + np.arange(nblk[s], dtype=np.int32)
        used = np.concatenate([tables[s, :nblk[s]] for s in range(cfg.num_seqs)])
        handed = np.zeros(num_blocks, dtype=bool)
        handed[used] = True
        unused = np.flatnonzero(~handed).astype(np.int32)
    else:
        num_blocks = cfg.pool_blocks if cfg.pool_blocks else math.ceil(1.1 * need)
        if num_blocks <= need:
            raise ValueError("pool too small to leave a spare block for poisoned padding")
        perm = rng_pool.permutation(num_blocks).astype(np.int32)
        if contiguous:
            perm = np.arange(num_blocks, dtype=np.int32)
        poison_block = int(perm[need])             # first block never handed out
        tables = np.full((cfg.num_seqs, max_blocks), poison_block, dtype=np.int32)
        pos = 0
        for s in range(cfg.num_seqs):
            tables[s, :nblk[s]] = perm[pos:pos + nblk[s]]
            pos += int(nblk[s])
        used = perm[:need]
        unused = perm[need:]

    Hkv, d = cfg.num_kv_heads, cfg.head_dim
    last_pos = lens.astype(np.int64) - 1
    slots = (tables[np.arange(cfg.num_seqs), last_pos // B].astype(np.int64) * B + last_pos % B).astype(np.int32)
    if not values:
        return DecodeWorkload(cfg, None, None, None, tables, lens.copy(), None, None, slots,
                              num_blocks, poison_block, used)
    q = random_stored(ss_q, (cfg.num_seqs, cfg.num_heads, d), cfg.etype, cfg.value_scale)
    k_cache = random_stored(ss_k, (num_blocks, Hkv, B, d), cfg.etype, cfg.value_scale)
    v_cache = random_stored(ss_v, (num_blocks, Hkv, d, B), cfg.etype, cfg.value_scale)
    kn_ss, vn_ss = ss_new.spawn(2)
    k_new = random_stored(kn_ss, (cfg.num_seqs, Hkv, d), cfg.etype, cfg.value_scale)
    v_new = random_stored(vn_ss, (cfg.num_seqs, Hkv, d), cfg.etype, cfg.value_scale)

    if poison:
        pv = poison_value(cfg.etype)
        k_cache[unused] = pv
        v_cache[unused] = pv
        for s in range(cfg.num_seqs):
            last = tables[s, nblk[s] - 1]
            off = (int(lens[s]) - 1) % B          # the new token's slot and the rest
            k_cache[last, :, off:, :] = pv
            set_v_tokens(v_cache, last, off, pv)
    return DecodeWorkload(cfg, q, k_cache, v_cache, tables, lens.copy(), k_new, v_new,
                          slots, num_blocks, poison_block, used)


# --------------------------------------------------------------------------
# Parallel sampling with a shared prompt (32 prompts x 8 samples).
# --------------------------------------------------------------------------

PARALLEL_SAMPLING = DecodeConfig("parallel_sampling", 4, 256, 32, 8, 128, 16, "bf16", 1.0,
                                 ("fixed", ()), 1024 + 256, partition_size=-2)


@dataclass
class SamplingStep:
    step: int
    block_mapping: np.ndarray     # [num_pairs][2] int32 (src, dst), applied before the write
    slot_mapping: np.ndarray      # [num_seqs] int32
    k_new: np.ndarray
    v_new: np.ndarray
    q: np.ndarray
    block_tables: np.ndarray      # [num_seqs][max_blocks] int32
    context_lens: np.ndarray      # [num_seqs] int32 (after this step's token)


class ParallelSamplingWorkload:
    """Prompts are prefilled once, then every prompt is forked into
    `samples` sequences sharing its blocks; each step appends one token per
    sample through the block manager (copy-on-write of a shared partial
    block, on-demand allocation otherwise)."""

    def __init__(self, prompt_len: int = 1024, num_prompts: int = 32, samples: int = 8,
                 new_tokens: int = 256, cfg: DecodeConfig = PARALLEL_SAMPLING, poison: bool = True,
                 values: bool = True):
        self.cfg = cfg
        self.prompt_len, self.num_prompts, self.samples, self.new_tokens = prompt_len, num_prompts, samples, new_tokens
        self.values = values
        seqs = np.random.SeedSequence(1000 + cfg.index).spawn(6)
        rng_pool = np.random.default_rng(seqs[1])
        ss_k, ss_v = seqs[3], seqs[4]
        self.ss_q, self.ss_new = seqs[2], seqs[5]
        B = cfg.block_size
        used = self._dry_run_blocks()
        self.num_blocks = math.ceil(1.1 * used)
        perm = rng_pool.permutation(self.num_blocks)
        self.bm = BlockManager(self.num_blocks, B, free_order=perm)
        self.max_blocks = -(-(prompt_len + new_tokens) // B)
        Hkv, d = cfg.num_kv_heads, cfg.head_dim
        self.k_cache = self.v_cache = None
        if values:
            self.k_cache = random_stored(ss_k, (self.num_blocks, Hkv, B, d), cfg.etype, cfg.value_scale)
            self.v_cache = random_stored(ss_v, (self.num_blocks, Hkv, d, B), cfg.etype, cfg.value_scale)
        self.seqs = []
        prompt_blocks = []
        for _ in range(num_prompts):
            parent = self.bm.new_sequence()
            for _ in range(prompt_len):
                self.bm.append_token(parent)
            prompt_blocks.extend(parent.block_table)
            self.seqs.append(parent)
            for _ in range(samples - 1):
                self.seqs.append(self.bm.fork(parent))
        # order: prompt-major, sample index ascending (parent is sample 0)
        self.seqs = [self.seqs[p * samples + i] for p in range(num_prompts) for i in range(samples)]
        self.poison_block = int(self.bm.free[-1])   # handed out last, if ever
        if poison and values:
            pv = poison_value(cfg.etype)
            held = np.zeros(self.num_blocks, dtype=bool)
            held[prompt_blocks] = True
            self.k_cache[~held] = pv
            self.v_cache[~held] = pv
            tail = prompt_len % B
            if tail:
                for p in range(num_prompts):
                    last = self.seqs[p * samples].block_table[-1]
                    self.k_cache[last, :, tail:, :] = pv
                    set_v_tokens(self.v_cache, last, tail, pv)
        self.step_index = 0

    def _dry_run_blocks(self) -> int:
        B = self.cfg.block_size
        prompt = -(-self.prompt_len // B)
        own_tokens_first_block = 0 if self.prompt_len % B == 0 else B - self.prompt_len % B
        per_sample_new = -(-max(0, self.new_tokens - own_tokens_first_block) // B)
        copies = (self.samples - 1) if (self.prompt_len % B and self.new_tokens) else 0
        return self.num_prompts * (prompt + copies + self.samples * per_sample_new)

    @property
    def num_seqs(self):
        return self.num_prompts * self.samples

    def step(self) -> SamplingStep:
        if self.step_index >= self.new_tokens:
            raise StopIteration
        self.step_index += 1
        cfg = self.cfg
        slots, pairs = [], []
        for seq in self.seqs:
            slot, copy = self.bm.append_token(seq)
            slots.append(slot)
            if copy is not None:
                pairs.append(copy)
        S, Hkv, d = self.num_seqs, cfg.num_kv_heads, cfg.head_dim
        q = k_new = v_new = None
        if self.values:
            # step t draws from child t-1 of the q and new-token streams
            q_ss = self.ss_q.spawn(1)[0]
            kn_ss, vn_ss = self.ss_new.spawn(1)[0].spawn(2)
            q = random_stored(q_ss, (S, cfg.num_heads, d), cfg.etype, cfg.value_scale)
            k_new = random_stored(kn_ss, (S, Hkv, d), cfg.etype, cfg.value_scale)
            v_new = random_stored(vn_ss, (S, Hkv, d), cfg.etype, cfg.value_scale)
        tables = np.full((S, self.max_blocks), self.poison_block, dtype=np.int32)
        for i, seq in enumerate(self.seqs):
            tables[i, :len(seq.block_table)] = seq.block_table
        lens = np.array([seq.num_tokens for seq in self.seqs], dtype=np.int32)
        mapping = np.array(pairs, dtype=np.int32).reshape(-1, 2)
        return SamplingStep(self.step_index, mapping, np.array(slots, dtype=np.int32),
                            k_new, v_new, q, tables, lens)

    def unique_blocks(self) -> int:
        return self.num_blocks - self.bm.num_free


BEAM_SEARCH = DecodeConfig("beam_search", 5, 128, 32, 8, 128, 16, "bf16", 1.0, ("fixed", ()), 1000 + 64,
                           partition_size=-2)


class BeamSearchWorkload:
    """Beam search over a paged cache: every request's prompt is prefilled
    once and forked into `beams` beams that share its blocks. Each step first
    re-selects the beams (from the second step on): new beam j continues a
    seeded choice of current beam, so some beams end (their blocks are
    released) and others split (forks share every block). Then one token is
    appended per beam, with copy-on-write of a shared, partly filled last
    block. Stream 0 of the seed draws the beam choices (no lengths here)."""

    def __init__(self, prompt_len: int = 1000, num_requests: int = 32, beams: int = 4, steps: int = 64,
                 cfg: DecodeConfig = BEAM_SEARCH, poison: bool = True, values: bool = True):
        self.cfg = cfg
        self.prompt_len, self.num_requests, self.beams, self.steps = prompt_len, num_requests, beams, steps
        self.values = values
        seqs = np.random.SeedSequence(1000 + cfg.index).spawn(6)
        self.rng_beam = np.random.default_rng(seqs[0])
        rng_pool = np.random.default_rng(seqs[1])
        self.ss_q, self.ss_new = seqs[2], seqs[5]
        B = cfg.block_size
        # every beam distinct at the end bounds what is ever held at once
        per_beam = -(-(prompt_len + steps) // B)
        self.num_blocks = math.ceil(1.1 * num_requests * beams * per_beam)
        perm = rng_pool.permutation(self.num_blocks)
        self.bm = BlockManager(self.num_blocks, B, free_order=perm)
        self.max_blocks = per_beam
        Hkv, d = cfg.num_kv_heads, cfg.head_dim
        self.k_cache = self.v_cache = None
        if values:
            self.k_cache = random_stored(seqs[3], (self.num_blocks, Hkv, B, d), cfg.etype, cfg.value_scale)
            self.v_cache = random_stored(seqs[4], (self.num_blocks, Hkv, d, B), cfg.etype, cfg.value_scale)
        self.groups = []
        prompt_blocks = []
        for _ in range(num_requests):
            parent = self.bm.new_sequence()
            for _ in range(prompt_len):
                self.bm.append_token(parent)
            prompt_blocks.extend(parent.block_table)
            self.groups.append([parent] + [self.bm.fork(parent) for _ in range(beams - 1)])
        self.poison_block = int(self.bm.free[-1])
        if poison and values:
            pv = poison_value(cfg.etype)
            held = np.zeros(self.num_blocks, dtype=bool)
            held[prompt_blocks] = True
            self.k_cache[~held] = pv
            self.v_cache[~held] = pv
            tail = prompt_len % B
            if tail:
                for g in self.groups:
                    last = g[0].block_table[-1]
                    self.k_cache[last, :, tail:, :] = pv
                    set_v_tokens(self.v_cache, last, tail, pv)
        self.step_index = 0

    @property
    def num_seqs(self):
        return self.num_requests * self.beams

    def reselect(self) -> None:
        K = self.beams
        for r, cur in enumerate(self.groups):
            parents = np.sort(self.rng_beam.integers(0, K, size=K))
            new = [self.bm.fork(cur[int(pj)]) for pj in parents]
            for b in cur:
                self.bm.free_sequence(b)
            self.groups[r] = new

    def step(self) -> SamplingStep:
        if self.step_index >= self.steps:
            raise StopIteration
        if self.step_index > 0:
            self.reselect()
        self.step_index += 1
        cfg = self.cfg
        slots, pairs = [], []
        seqs = [b for g in self.groups for b in g]
        for seq in seqs:
            slot, copy = self.bm.append_token(seq)
            slots.append(slot)
            if copy is not None:
                pairs.append(copy)
        S, Hkv, d = self.num_seqs, cfg.num_kv_heads, cfg.head_dim
        q = k_new = v_new = None
        if self.values:
            q_ss = self.ss_q.spawn(1)[0]
            kn_ss, vn_ss = self.ss_new.spawn(1)[0].spawn(2)
            q = random_stored(q_ss, (S, cfg.num_heads, d), cfg.etype, cfg.value_scale)
            k_new = random_stored(kn_ss, (S, Hkv, d), cfg.etype, cfg.value_scale)
            v_new = random_stored(vn_ss, (S, Hkv, d), cfg.etype, cfg.value_scale)
        tables = np.full((S, self.max_blocks), self.poison_block, dtype=np.int32)
        for i, seq in enumerate(seqs):
            tables[i, :len(seq.block_table)] = seq.block_table
        lens = np.array([seq.num_tokens for seq in seqs], dtype=np.int32)
        mapping = np.array(pairs, dtype=np.int32).reshape(-1, 2)
        return SamplingStep(self.step_index, mapping, np.array(slots, dtype=np.int32),
                            k_new, v_new, q, tables, lens)

    def blocks_in_use(self) -> int:
        return self.num_blocks - self.bm.num_free


SHARED_PREFIX = DecodeConfig("shared_prefix", 6, 256, 32, 8, 128, 16, "bf16", 1.0, ("uniform", 16, 512),
                             1024 + 512, partition_size=-2)


def make_shared_prefix_workload(prefix_len: int = 1024, cfg: DecodeConfig = SHARED_PREFIX, poison: bool = True,
                                values: bool = True) -> DecodeWorkload:
    """One decode step of requests that all map the same prompt prefix (a
    shared system prompt): the prefix is prefilled once and its blocks are
    mapped into every request (forks, reference counts raised); each request
    then holds its own suffix of a drawn length, whose last token is the new
    one. The prefix stays reserved (its own reference is kept), so its last
    block is copy-on-write for every request ("PagedAttention 论文精读笔记"
    §6.3). A block-aligned prefix needs no copy. A prefix that ends inside a
    block makes each request copy that block at its first suffix token: the
    pools are then returned as they were before those copies (targets
    poisoned, the shared block valid up to the prefix's end), with the copy
    pairs and the suffix tokens that landed in the copies (new token
    excluded) to replay."""
    seqs = np.random.SeedSequence(1000 + cfg.index).spawn(6)
    rng_len, rng_pool = np.random.default_rng(seqs[0]), np.random.default_rng(seqs[1])
    suffix = draw_lengths(cfg, rng_len)
    B = cfg.block_size
    lens = (prefix_len + suffix).astype(np.int32)
    prefix_blocks = -(-prefix_len // B)
    own = -(-(lens.astype(np.int64) - (prefix_len // B) * B) // B)
    need = prefix_blocks + int(own.sum())
    num_blocks = math.ceil(1.1 * need)
    perm = rng_pool.permutation(num_blocks)
    bm = BlockManager(num_blocks, B, free_order=perm)
    root = bm.new_sequence()
    for _ in range(prefix_len):
        bm.append_token(root)
    max_blocks = -(-int(lens.max()) // B)
    poison_block = int(bm.free[-1])
    tables = np.full((cfg.num_seqs, max_blocks), poison_block, dtype=np.int32)
    slots = np.empty(cfg.num_seqs, dtype=np.int32)
    r = prefix_len % B
    pairs, pre_slots = [], []
    for s in range(cfg.num_seqs):
        seq = bm.fork(root)
        n_suf = int(suffix[s])
        for i in range(n_suf):
            slot, copy = bm.append_token(seq)
            if copy is not None:
                pairs.append(copy)
            if r and i < B - r and i < n_suf - 1:   # landed in the copy, before the new token
                pre_slots.append(slot)
        tables[s, :len(seq.block_table)] = seq.block_table
        slots[s] = slot
    if pairs and r == 0:
        raise AssertionError("a block-aligned prefix must not be copied")
    if r and len(pairs) != cfg.num_seqs:
        raise AssertionError("every request copies the reserved prefix's partial last block")
    copy_pairs = np.array(pairs, dtype=np.int32).reshape(-1, 2) if r else None
    pre = np.array(pre_slots, dtype=np.int32) if r else None
    # the reserved prefix's blocks are held too (its partial last block is
    # the copies' source, mapped by no request any more)
    used = np.array(sorted(set(tables[tables != poison_block].tolist()) | set(root.block_table)), dtype=np.int64)
    if not values:
        return DecodeWorkload(cfg, None, None, None, tables, lens, None, None, slots, num_blocks, poison_block, used,
                              copy_pairs, pre)
    Hkv, d = cfg.num_kv_heads, cfg.head_dim
    q = random_stored(seqs[2], (cfg.num_seqs, cfg.num_heads, d), cfg.etype, cfg.value_scale)
    k_cache = random_stored(seqs[3], (num_blocks, Hkv, B, d), cfg.etype, cfg.value_scale)
    v_cache = random_stored(seqs[4], (num_blocks, Hkv, d, B), cfg.etype, cfg.value_scale)
    kn_ss, vn_ss, pk_ss, pv_ss = seqs[5].spawn(4)
    k_new = random_stored(kn_ss, (cfg.num_seqs, Hkv, d), cfg.etype, cfg.value_scale)
    v_new = random_stored(vn_ss, (cfg.num_seqs, Hkv, d), cfg.etype, cfg.value_scale)
    pre_k = pre_v = None
    if r:
        pre_k = random_stored(pk_ss, (len(pre), Hkv, d), cfg.etype, cfg.value_scale)
        pre_v = random_stored(pv_ss, (len(pre), Hkv, d), cfg.etype, cfg.value_scale)
    if poison:
        pv = poison_value(cfg.etype)
        held = np.zeros(num_blocks, dtype=bool)
        held[used] = True
        k_cache[~held] = pv
        v_cache[~held] = pv
        for s in range(cfg.num_seqs):
            last = tables[s, (int(lens[s]) - 1) // B]
            off = (int(lens[s]) - 1) % B          # the new token's slot and the rest
            k_cache[last, :, off:, :] = pv
            set_v_tokens(v_cache, last, off, pv)
        if r:
            # before the copies: targets unwritten, the shared block valid up to the prefix's end
            k_cache[copy_pairs[:, 1]] = pv
            v_cache[copy_pairs[:, 1]] = pv
            src = int(copy_pairs[0, 0])
            k_cache[src, :, r:, :] = pv
            set_v_tokens(v_cache, src, r, pv)
    return DecodeWorkload(cfg, q, k_cache, v_cache, tables, lens, k_new, v_new, slots, num_blocks, poison_block, used,
                          copy_pairs, pre, pre_k, pre_v)


def make_forked_workload(cfg: DecodeConfig, groups, poison: bool = True) -> DecodeWorkload:
    """One decode step of sequences forked from shared prompts: `groups` is a
    list of (prompt_len, [own_len, ...]); the forks of a group are adjacent
    in the batch, map the prompt's full blocks by the same ids and hold their
    own tokens (at least one each, the new token among them) in blocks of
    their own. A prompt that ends inside a block gives every fork its own
    copy of that block (as copy-on-write leaves it), holding the prompt's
    tokens there. Ids come from a seeded permutation of the pool (10% spare,
    plus a poisoned padding block); values as in make_decode_workload."""
    seqs = np.random.SeedSequence(1000 + cfg.index).spawn(6)
    rng_pool = np.random.default_rng(seqs[1])
    B = cfg.block_size
    lens, layout = [], []
    need = 0
    for prompt_len, owns in groups:
        full = prompt_len // B
        need += full
        for own in owns:
            if own < 1:
                raise ValueError("every fork holds at least its new token")
            L = prompt_len + own
            need += -(-L // B) - full
            lens.append(L)
    num_blocks = math.ceil(1.1 * need) + 1
    perm = rng_pool.permutation(num_blocks).astype(np.int32)
    lens = np.array(lens, dtype=np.int32)
    S = len(lens)
    max_blocks = max(-(-cfg.max_len // B), int(-(-lens.max() // B)))
    poison_block = int(perm[need])
    tables = np.full((S, max_blocks), poison_block, dtype=np.int32)
    pos, s, copies = 0, 0, []
    for prompt_len, owns in groups:
        full = prompt_len // B
        shared = perm[pos:pos + full]
        pos += full
        src = None
        for own in owns:
            L = int(lens[s])
            n = -(-L // B)
            tables[s, :full] = shared
            tables[s, full:n] = perm[pos:pos + n - full]
            pos += n - full
            if prompt_len % B:
                if src is None:
                    src = int(tables[s, full])
                else:
                    copies.append((src, int(tables[s, full])))
            s += 1
    used = perm[:need]
    last_pos = lens.astype(np.int64) - 1
    slots = (tables[np.arange(S), last_pos // B].astype(np.int64) * B + last_pos % B).astype(np.int32)
    Hkv, d = cfg.num_kv_heads, cfg.head_dim
    q = random_stored(seqs[2], (S, cfg.num_heads, d), cfg.etype, cfg.value_scale)
    k_cache = random_stored(seqs[3], (num_blocks, Hkv, B, d), cfg.etype, cfg.value_scale)
    v_cache = random_stored(seqs[4], (num_blocks, Hkv, d, B), cfg.etype, cfg.value_scale)
    kn_ss, vn_ss = seqs[5].spawn(2)
    k_new = random_stored(kn_ss, (S, Hkv, d), cfg.etype, cfg.value_scale)
    v_new = random_stored(vn_ss, (S, Hkv, d), cfg.etype, cfg.value_scale)
    # the prompt's tokens in every fork's copy of its partial last block
    for a, b in copies:
        k_cache[b] = k_cache[a]
        v_cache[b] = v_cache[a]
    if poison:
        pv = poison_value(cfg.etype)
        k_cache[perm[need:]] = pv
        v_cache[perm[need:]] = pv
        for s in range(S):
            last = tables[s, int(last_pos[s]) // B]
            off = int(last_pos[s]) % B          # the new token's slot and the rest
            k_cache[last, :, off:, :] = pv
            set_v_tokens(v_cache, last, off, pv)
    cfg = dataclasses.replace(cfg, num_seqs=S)
    return DecodeWorkload(cfg, q, k_cache, v_cache, tables, lens, k_new, v_new, slots, num_blocks, poison_block, used)


# --------------------------------------------------------------------------
# Prompt phase: a batch of prompts whose K/V is in the pool.
# --------------------------------------------------------------------------

PREFILL = DecodeConfig("prefill", 7, 32, 32, 8, 128, 16, "bf16", 1.0, ("lognormal", 800.0, 1.0, 16, 8192), 8192)


@dataclass
class PrefillWorkload:
    """Prompt-phase inputs. The pool holds all context_lens[s] tokens of each
    sequence; its n_s queries, the context's last n_s tokens (n_s = L for a
    whole prompt), are packed in q rows q_start[s] .. q_start[s+1]-1."""
    cfg: DecodeConfig
    q: np.ndarray
    q_start: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    block_tables: np.ndarray
    context_lens: np.ndarray
    num_blocks: int
    poison_block: int
    used_blocks: np.ndarray

    @property
    def total_q(self) -> int:
        return int(self.q_start[-1])

    @property
    def queries(self) -> np.ndarray:
        return np.diff(self.q_start)

    def pairs(self) -> int:
        """(query, cached token) pairs a causal pass scores: query j of n at
        position L - n + j sees L - n + j + 1 tokens."""
        n = self.queries.astype(np.int64)
        L = self.context_lens.astype(np.int64)
        return int((n * (L - n) + n * (n + 1) // 2).sum())

    def flops(self) -> int:
        """QK and PV products: 2 * head_dim flops each per (pair, query head)."""
        return self.pairs() * self.cfg.num_heads * self.cfg.head_dim * 4

    def kv_bytes(self) -> int:
        c = self.cfg
        return int(self.context_lens.astype(np.int64).sum()) * c.num_kv_heads * c.head_dim * 2 * ELEMENT_BYTES[c.etype]


def make_prefill_workload(cfg: DecodeConfig = PREFILL, lengths=None, queries=None, poison: bool = True,
                          values: bool = True, contiguous: bool = False) -> PrefillWorkload:
    """Draw a prompt-phase batch: context lengths from the config's law (or
    given), `queries` per sequence (default: the whole context, 0 <= n <= L),
    blocks handed out in the seeded shuffled order (in order with
    contiguous=True). Unused blocks and the slots past each context are
    poisoned."""
    seqs = np.random.SeedSequence(1000 + cfg.index).spawn(5)
    rng_len, rng_pool = np.random.default_rng(seqs[0]), np.random.default_rng(seqs[1])
    lens = draw_lengths(cfg, rng_len) if lengths is None else np.asarray(lengths, dtype=np.int32)
    if lens.shape != (cfg.num_seqs,) or lens.min() < 1:
        raise ValueError("one positive length per sequence is required")
    n = lens.copy() if queries is None else np.asarray(queries, dtype=np.int32)
    if n.shape != lens.shape or n.min() < 0 or np.any(n > lens):
        raise ValueError("queries must satisfy 0 <= n <= L per sequence")
    q_start = np.concatenate([[0], np.cumsum(n.astype(np.int64))]).astype(np.int32)
    B = cfg.block_size
    nblk = -(-lens.astype(np.int64) // B)
    need = int(nblk.sum())
    num_blocks = cfg.pool_blocks if cfg.pool_blocks else math.ceil(1.1 * need)
    if num_blocks <= need:
        raise ValueError("pool too small to leave a spare block for poisoned padding")
    perm = np.arange(num_blocks, dtype=np.int32) if contiguous else rng_pool.permutation(num_blocks).astype(np.int32)
    max_blocks = max(-(-cfg.max_len // B), int(nblk.max()))
    poison_block = int(perm[need])
    tables = np.full((cfg.num_seqs, max_blocks), poison_block, dtype=np.int32)
    pos = 0
    for s in range(cfg.num_seqs):
        tables[s, :nblk[s]] = perm[pos:pos + nblk[s]]
        pos += int(nblk[s])
    used = perm[:need]
    if not values:
        return PrefillWorkload(cfg, None, q_start, None, None, tables, lens.copy(), num_blocks, poison_block, used)
    Hkv, d = cfg.num_kv_heads, cfg.head_dim
    q = random_stored(seqs[2], (int(q_start[-1]), cfg.num_heads, d), cfg.etype, cfg.value_scale)
    k_cache = random_stored(seqs[3], (num_blocks, Hkv, B, d), cfg.etype, cfg.value_scale)
    v_cache = random_stored(seqs[4], (num_blocks, Hkv, d, B), cfg.etype, cfg.value_scale)
    if poison:
        pv = poison_value(cfg.etype)
        k_cache[perm[need:]] = pv
        v_cache[perm[need:]] = pv
        for s in range(cfg.num_seqs):
            off = int(lens[s]) % B
            if off:
                last = tables[s, nblk[s] - 1]
                k_cache[last, :, off:, :] = pv
                set_v_tokens(v_cache, last, off, pv)
    return PrefillWorkload(cfg, q, q_start, k_cache, v_cache, tables, lens.copy(), num_blocks, poison_block, used)
