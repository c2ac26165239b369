"""Host-side KV block manager: the CPU half of paged KV caching.

The pages describe the KV cache as fixed-size blocks carved out of one large
preallocated pool, handed out on demand and mapped per sequence by a block
table (runbyai "The core idea of PagedAttention", items 1-3; ai-hpc "2.1
Algorithm Principle"; architvora "Paged Attention" and "Just a python
process").  Bookkeeping runs on the CPU, and each step the engine packs the
tables into tensors for the GPU (architvora "Just a python process").

This module owns that bookkeeping:

* ``BlockPool``     -- free list plus per-block reference counts.  Shared
                       blocks (one copy of a common prompt, runbyai item 3;
                       ai-hpc "2.2 Advantages") carry refcount > 1 and go back
                       to the free list only when the last owner releases them.
* ``Sequence``      -- one sequence's logical-to-physical block list and token
                       count; ``append_slot`` allocates a block only when the
                       next token starts a new one (on-demand allocation).
* ``Sequence.fork`` / ``Sequence.append_slot_cow`` -- sharing a prompt between
                       forked sequences and the copy-on-write of a shared
                       block one of them writes into.
* ``swap_blocks``     -- the bookkeeping of moving a sequence's blocks to
                       another pool (host memory) and back.
* ``pack_block_tables`` / ``pack_context_lens`` -- pack the per-sequence
                       state into the int32 arrays the C-ABI consumes.
* ``tables_share_blocks`` -- whether a packed batch points several sequences
                       at one block, which selects the decode's cached-read
                       variant (the ``shared_blocks`` option).

A flat slot index is ``physical_block * block_size + offset_in_block``.
"""
from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field
from typing import Iterable, List, Optional, Sequence as Seq, Tuple

import numpy as np


class PoolExhausted(RuntimeError):
    """Raised when an allocation asks for more blocks than the pool has free.

    A serving engine would preempt a sequence here (architvora "Paged
    Attention": sequences can be preempted and moved to the CPU); this
    manager reports the condition and leaves the policy to the caller.
    """


class BlockPool:
    """Free list and reference counts over ``num_blocks`` physical blocks.

    ``order`` fixes the order in which free blocks are handed out; a seeded
    permutation reproduces "physical blocks drawn in random order".  Blocks
    released later are appended to the back of the free list (FIFO reuse).
    """

    def __init__(self, num_blocks: int, block_size: int = 16,
                 order: Optional[Iterable[int]] = None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        ids = np.arange(self.num_blocks, dtype=np.int64) if order is None \
            else np.asarray(list(order), dtype=np.int64)
        if ids.shape != (self.num_blocks,) or not np.array_equal(np.sort(ids), np.arange(self.num_blocks)):
            raise ValueError("order must be a permutation of range(num_blocks)")
        self._free = deque(int(i) for i in ids)  # allocate from the left, release to the right
        self.refcount = np.zeros(self.num_blocks, dtype=np.int32)

    @property
    def num_free(self) -> int:
        return len(self._free)

    def allocate(self, n: int = 1) -> List[int]:
        if n < 0:
            raise ValueError("n must be >= 0")
        if n > len(self._free):
            raise PoolExhausted(f"asked for {n} blocks, {len(self._free)} free of {self.num_blocks}")
        out = [self._free.popleft() for _ in range(n)]
        self.refcount[out] = 1
        return out

    def share(self, ids: Seq[int]) -> None:
        """Add one owner to each block in ``ids`` (prefix sharing)."""
        ids = list(ids)
        if any(self.refcount[i] <= 0 for i in ids):
            raise ValueError("cannot share a block that is not allocated")
        for i in ids:
            self.refcount[i] += 1

    def release(self, ids: Seq[int]) -> None:
        """Drop one owner from each block; blocks with no owner become free."""
        for i in ids:
            if self.refcount[i] <= 0:
                raise ValueError(f"block {i} released more times than allocated")
            self.refcount[i] -= 1
            if self.refcount[i] == 0:
                self._free.append(int(i))

    def free_ids(self) -> List[int]:
        return list(self._free)


@dataclass
class Sequence:
    """One sequence: its block list (logical block j -> ``blocks[j]``) and length."""

    seq_id: int
    blocks: List[int] = field(default_factory=list)
    num_tokens: int = 0

    def append_slot(self, pool: BlockPool) -> int:
        """Reserve the slot of the next token, allocating a block on demand."""
        bs = pool.block_size
        if self.num_tokens % bs == 0 and self.num_tokens // bs == len(self.blocks):
            self.blocks.extend(pool.allocate(1))
        pos = self.num_tokens
        self.num_tokens += 1
        return self.blocks[pos // bs] * bs + pos % bs

    def reserve(self, pool: BlockPool, n_tokens: int) -> np.ndarray:
        """Reserve ``n_tokens`` consecutive slots (a prompt); returns their flat slots."""
        bs = pool.block_size
        start = self.num_tokens
        need = blocks_needed(start + n_tokens, bs) - len(self.blocks)
        if need > 0:
            self.blocks.extend(pool.allocate(need))
        self.num_tokens += n_tokens
        pos = np.arange(start, start + n_tokens, dtype=np.int64)
        return np.asarray(self.blocks, dtype=np.int64)[pos // bs] * bs + pos % bs

    def slot_of(self, pos: int, block_size: int) -> int:
        if not 0 <= pos < self.num_tokens:
            raise IndexError(pos)
        return self.blocks[pos // block_size] * block_size + pos % block_size

    def release(self, pool: BlockPool) -> None:
        pool.release(self.blocks)
        self.blocks = []
        self.num_tokens = 0

    def fork(self, pool: BlockPool, seq_id: int) -> "Sequence":
        """A new sequence sharing every block of this one (parallel sampling,
        beam search: ai-hpc "2.2 Advantages", item 2)."""
        pool.share(self.blocks)
        return Sequence(seq_id, list(self.blocks), self.num_tokens)

    def append_slot_cow(self, pool: BlockPool) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Reserve the next token's slot, copy-on-write.

        If the token lands in a block that other sequences still own, this
        sequence first moves to a private copy of that block.  Returns the
        slot and the (source, destination) block copy that must run before
        the token is written, or None.
        """
        bs = pool.block_size
        copy = None
        j = self.num_tokens // bs
        if j < len(self.blocks) and pool.refcount[self.blocks[j]] > 1:
            old = self.blocks[j]
            new = pool.allocate(1)[0]
            pool.release([old])
            self.blocks[j] = new
            copy = (old, new)
        return self.append_slot(pool), copy


def swap_blocks(seq: Sequence, from_pool: BlockPool, to_pool: BlockPool) -> List[Tuple[int, int]]:
    """Move a sequence's blocks from one pool to another (device -> host to
    preempt it, host -> device to resume it: architvora "Paged Attention").

    Every block gets a fresh block in ``to_pool``; the sequence then refers
    to the new blocks, and drops its ownership of the old ones (a block other
    sequences still share stays where it is for them).  Returns the
    (old block, new block) pairs the block copy must run, in table order.
    """
    new = to_pool.allocate(len(seq.blocks))
    pairs = list(zip(seq.blocks, new))
    from_pool.release(seq.blocks)
    seq.blocks = list(new)
    return pairs


def blocks_needed(num_tokens: int, block_size: int) -> int:
    return -(-int(num_tokens) // int(block_size))


def pack_block_tables(seqs: Seq[Sequence], width: int, pad_block: int) -> np.ndarray:
    """Pack per-sequence block lists into an int32 ``[len(seqs), width]`` table.

    Entries past a sequence's last block are never read by the kernels; they
    are filled with ``pad_block`` (tests point it at a NaN-poisoned block).
    """
    bt = np.full((len(seqs), width), pad_block, dtype=np.int32)
    for i, s in enumerate(seqs):
        if len(s.blocks) > width:
            raise ValueError(f"sequence {s.seq_id} needs {len(s.blocks)} blocks > table width {width}")
        bt[i, :len(s.blocks)] = s.blocks
    return bt


def tables_share_blocks(block_tables: np.ndarray, context_lens: np.ndarray, block_size: int) -> bool:
    """True when some physical block appears in the used part of two tables
    (or twice in one), i.e. the decode will read it more than once."""
    bt = np.asarray(block_tables)
    used = [bt[i, :blocks_needed(max(int(L), 0), block_size)] for i, L in enumerate(np.asarray(context_lens))]
    ids = np.concatenate(used) if used else np.zeros(0, dtype=np.int32)
    return bool(np.unique(ids).size != ids.size)


def pack_context_lens(seqs: Seq[Sequence]) -> np.ndarray:
    return np.array([s.num_tokens for s in seqs], dtype=np.int32)


def check_unique_slots(slot_mapping: np.ndarray, num_blocks: int, block_size: int) -> None:
    """Host-side debug check: slots in range and no slot written twice.

    The device never validates slots (that would need a synchronisation); a
    duplicate slot would make the cache write racy.
    """
    s = np.asarray(slot_mapping, dtype=np.int64)
    s = s[s >= 0]
    if s.size and s.max() >= num_blocks * block_size:
        raise ValueError("slot out of range")
    if np.unique(s).size != s.size:
        raise ValueError("duplicate slot in slot_mapping")
