"""Host-side KV block manager: free pool, per-block reference counts, per-sequence
block tables, on-demand allocation, fork and copy-on-write.

It produces the integer inputs of the device calls (block tables, slot
mappings and copy lists); it never touches K/V values.

  * on-demand allocation: a physical block is taken from the free pool only
    when a token's logical block is not mapped yet ("paged-attention은 도대체
    뭘 최적화 하는 것일까", §6 and the §17 pseudocode `ensure_capacity`);
  * slot = physical_block * block_size + offset (same page, §14 and §17);
  * fork shares every block and raises its reference count; a write into a
    block whose count is above one first copies it to a fresh block, lowers
    the old count and writes the copy, while the last sharer writes in place
    ("PagedAttention 论文精读笔记", §6.1);
  * blocks return to the free pool when their count reaches zero (same page,
    §5.1 and §6.2);
  * swapping: an evicted group's blocks move to slots of a host swap space
    handed out by a CPU block allocator and come back into fresh GPU blocks
    when the group resumes, all or nothing per group (same page, §7.3-§7.4).
"""

from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field


class PoolExhausted(RuntimeError):
    """No free physical block is left (the serving layer would preempt)."""


@dataclass
class Sequence:
    block_table: list = field(default_factory=list)   # GPU blocks, or host slots while swapped out
    num_tokens: int = 0
    swapped: bool = False


class SwapSpace:
    """CPU block allocator: slots of a host swap space, each holding one
    block, with the number of sequence references the block had on the GPU
    (restored on swap-in)."""

    def __init__(self, num_slots: int):
        if num_slots < 1:
            raise ValueError("num_slots must be positive")
        self.num_slots = num_slots
        self.free = deque(range(num_slots))
        self.refs = [0] * num_slots

    @property
    def num_free(self) -> int:
        return len(self.free)


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        if num_blocks < 1 or block_size < 1:
            raise ValueError("num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of range(num_blocks)")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = deque(order)
        self.refcount = [0] * num_blocks

    # -- pool -------------------------------------------------------------
    def allocate(self) -> int:
        if not self.free:
            raise PoolExhausted("KV block pool exhausted")
        blk = self.free.popleft()
        self.refcount[blk] = 1
        return blk

    def release(self, blk: int) -> None:
        if self.refcount[blk] <= 0:
            raise ValueError(f"block {blk} released more often than referenced")
        self.refcount[blk] -= 1
        if self.refcount[blk] == 0:
            self.free.append(blk)

    @property
    def num_free(self) -> int:
        return len(self.free)

    # -- sequences ----------------------------------------------------------
    def new_sequence(self) -> Sequence:
        return Sequence()

    def append_token(self, seq: Sequence):
        """Reserve the slot of the sequence's next token.

        Returns (slot, copy) where copy is None or the (src, dst) pair that
        must be block-copied before the token's K/V is written.
        """
        t = seq.num_tokens
        logical = t // self.block_size
        copy = None
        if logical == len(seq.block_table):
            seq.block_table.append(self.allocate())
        else:
            blk = seq.block_table[logical]
            if self.refcount[blk] > 1:
                fresh = self.allocate()
                copy = (blk, fresh)
                self.refcount[blk] -= 1
                seq.block_table[logical] = fresh
        seq.num_tokens = t + 1
        slot = seq.block_table[logical] * self.block_size + t % self.block_size
        return slot, copy

    def fork(self, parent: Sequence) -> Sequence:
        for blk in parent.block_table:
            self.refcount[blk] += 1
        return Sequence(block_table=list(parent.block_table), num_tokens=parent.num_tokens)

    def free_sequence(self, seq: Sequence) -> None:
        for blk in seq.block_table:
            self.release(blk)
        seq.block_table = []
        seq.num_tokens = 0

    def slot_of(self, seq: Sequence, token_index: int) -> int:
        blk = seq.block_table[token_index // self.block_size]
        return blk * self.block_size + token_index % self.block_size

    # -- swapping -----------------------------------------------------------
    def swap_out(self, seqs, space: SwapSpace):
        """Evict a group of sequences: each distinct block the group maps goes
        to one host slot (in order of first appearance). The group must hold
        every reference to its blocks. Returns the (gpu block, host slot)
        pairs to copy out before the blocks are reused."""
        slot_of, pairs = {}, []
        refs = {}
        for seq in seqs:
            if seq.swapped:
                raise ValueError("sequence already swapped out")
            for blk in seq.block_table:
                refs[blk] = refs.get(blk, 0) + 1
        for blk, n in refs.items():
            if self.refcount[blk] != n:
                raise ValueError(f"block {blk} is also mapped outside the group")
        if len(refs) > space.num_free:
            raise PoolExhausted("swap space exhausted")
        for seq in seqs:
            for blk in seq.block_table:
                if blk not in slot_of:
                    slot = space.free.popleft()
                    space.refs[slot] = refs[blk]
                    slot_of[blk] = slot
                    pairs.append((blk, slot))
        for seq in seqs:
            for blk in seq.block_table:
                self.release(blk)
            seq.block_table = [slot_of[b] for b in seq.block_table]
            seq.swapped = True
        return pairs

    def swap_in(self, seqs, space: SwapSpace):
        """Resume a swapped-out group: every host slot it maps gets a fresh GPU
        block with the slot's reference count. Returns the (gpu block, host
        slot) pairs to copy in before the group runs again."""
        block_of, pairs = {}, []
        slots = []
        for seq in seqs:
            if not seq.swapped:
                raise ValueError("sequence is not swapped out")
            for slot in seq.block_table:
                if slot not in block_of:
                    block_of[slot] = None
                    slots.append(slot)
        if len(slots) > self.num_free:
            raise PoolExhausted("KV block pool exhausted")
        for slot in slots:
            blk = self.allocate()
            self.refcount[blk] = space.refs[slot]
            block_of[slot] = blk
            pairs.append((blk, slot))
        for slot in slots:
            space.refs[slot] = 0
            space.free.append(slot)
        for seq in seqs:
            seq.block_table = [block_of[s] for s in seq.block_table]
            seq.swapped = False
        return pairs
