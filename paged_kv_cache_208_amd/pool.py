"""Host-side block-pool bookkeeping for paged KV caches.

The block manager sits on the host in the pages' designs and is not part of
the GPU data path; this module is the small allocator a caller of the library
uses to produce the three integer inputs the kernels consume: block tables,
context lengths and the slot of every new token.

Behaviour follows "Distributed LLM Inference Serving Platform":
  * section 2 and section 4: fixed 16-token physical blocks are handed out
    from a pool on demand and freed when a sequence ends;
  * section 7 (block manager): a free list, a reference count per block,
    allocation raising an out-of-memory error when the list is empty, free
    returning a block to the list when its count reaches zero, and sharing
    by incrementing the count;
  * section 11, Lab 1 worked solution (copy-on-write for parallel sampling):
    forking copies a table and bumps every block's count; a sequence that
    appends into a shared tail block clones it into a fresh block (copying
    the tokens already in it) and replaces the tail entry of its own table;
    the last holder of a block writes into it in place.  Full prefix blocks
    stay shared.
The page's simulation appends a cloned block to the table instead of
replacing the tail and can clone a full block; this module follows the
worked solution's semantics instead.

Also "Roadmap: vLLM-style serving features for TornadoVM batched decode",
Serving / scheduling: a shared prompt prefix is prefilled once into blocks
that every sequence's table references.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


class PoolExhausted(RuntimeError):
    """No free physical block is left in the pool."""


@dataclass
class _Block:
    ref: int = 0
    tokens: int = 0


@dataclass
class AppendResult:
    slot: int                    # flat slot = block * block_size + offset
    copy_from: int | None = None  # copy-on-write source block (or None)
    copy_to: int | None = None    # copy-on-write destination block
    copy_tokens: int = 0          # rows to copy from copy_from


@dataclass
class BlockPool:
    num_blocks: int
    block_size: int = 16
    _free: list = field(default_factory=list)
    _blocks: list = field(default_factory=list)
    tables: dict = field(default_factory=dict)
    lens: dict = field(default_factory=dict)

    def __post_init__(self):
        self._free = list(range(self.num_blocks))
        self._blocks = [_Block() for _ in range(self.num_blocks)]

    # -- block level ---------------------------------------------------------
    def available(self) -> int:
        return len(self._free)

    def refcount(self, blk: int) -> int:
        return self._blocks[blk].ref

    def token_count(self, blk: int) -> int:
        return self._blocks[blk].tokens

    def allocate(self) -> int:
        if not self._free:
            raise PoolExhausted("no free physical KV blocks left in the pool")
        blk = self._free.pop()
        self._blocks[blk] = _Block(ref=1, tokens=0)
        return blk

    def free_block(self, blk: int) -> None:
        b = self._blocks[blk]
        if b.ref <= 0:
            raise ValueError(f"block {blk} is not allocated")
        b.ref -= 1
        if b.ref == 0:
            b.tokens = 0
            self._free.append(blk)

    def share(self, blk: int) -> None:
        if self._blocks[blk].ref <= 0:
            raise ValueError(f"block {blk} is not allocated")
        self._blocks[blk].ref += 1

    # -- sequence level ------------------------------------------------------
    def add_sequence(self, sid, prefix_blocks=()) -> None:
        """New sequence, optionally starting on shared full prefix blocks."""
        if sid in self.tables:
            raise KeyError(f"sequence {sid!r} exists")
        for blk in prefix_blocks:
            if self._blocks[blk].tokens != self.block_size:
                raise ValueError("only full blocks can be shared as a prefix")
            self.share(blk)
        self.tables[sid] = list(prefix_blocks)
        self.lens[sid] = len(prefix_blocks) * self.block_size

    def append_slot(self, sid) -> AppendResult:
        """Reserve the slot for the sequence's next token."""
        table = self.tables[sid]
        L = self.lens[sid]
        if L % self.block_size == 0:
            blk = self.allocate()          # tail full (or no block yet)
            table.append(blk)
            res = AppendResult(slot=blk * self.block_size)
        else:
            tail = table[-1]
            tb = self._blocks[tail]
            if tb.ref > 1:                 # shared partial tail: copy on write
                tb.ref -= 1
                new = self.allocate()
                self._blocks[new].tokens = tb.tokens
                table[-1] = new
                res = AppendResult(slot=new * self.block_size + tb.tokens,
                                   copy_from=tail, copy_to=new, copy_tokens=tb.tokens)
            else:
                res = AppendResult(slot=tail * self.block_size + tb.tokens)
        blk = res.slot // self.block_size
        self._blocks[blk].tokens += 1
        self.lens[sid] = L + 1
        return res

    def fork(self, parent, children) -> None:
        """Children start with the parent's table; every block gains a ref."""
        for c in children:
            if c in self.tables:
                raise KeyError(f"sequence {c!r} exists")
            self.tables[c] = list(self.tables[parent])
            self.lens[c] = self.lens[parent]
            for blk in self.tables[parent]:
                self._blocks[blk].ref += 1

    def free_sequence(self, sid) -> None:
        for blk in self.tables.pop(sid):
            self.free_block(blk)
        self.lens.pop(sid)

    # -- kernel inputs -------------------------------------------------------
    def block_table_array(self, sids, max_blocks, pad_block) -> np.ndarray:
        out = np.full((len(sids), max_blocks), pad_block, dtype=np.int32)
        for i, s in enumerate(sids):
            t = self.tables[s]
            if len(t) > max_blocks:
                raise ValueError("table wider than max_blocks")
            out[i, :len(t)] = t
        return out

    def context_lens_array(self, sids) -> np.ndarray:
        return np.array([self.lens[s] for s in sids], dtype=np.int32)

    def shares_blocks(self, sids) -> bool:
        """True when some physical block is mapped by the tables of two or
        more of the sequences `sids` (a shared prefix, or forked sequences):
        the batch then reads that block several times in one decode call,
        which is when the caller passes the library's shared-blocks cache
        hint (PKV_KV_SHARED_BLOCKS)."""
        seen = set()
        for s in sids:
            for blk in set(self.tables[s]):
                if blk in seen:
                    return True
                seen.add(blk)
        return False
