"""CPU oracle for the paged KV cache: page allocation, token writes and
copy-on-write prefix sharing.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package.  The GPU library never
calls it, shares no code with it, and nothing here imports the GPU library.

Sources: [Different attention mechanisms, §5 Page Attention].
* Step 1: the KV cache is cut into fixed-size blocks (pages) that need not be
  contiguous in device memory.
* Step 2: every sequence keeps a page table mapping its logical blocks to
  physical blocks.
* Step 3: when a token arrives, a physical block is taken for it on demand and
  only the page table changes; nothing already cached moves.
* Advantages: requests with a common prefix point their page tables at the
  same physical blocks, shared copy-on-write.

Readings where the pages are silent (each is listed in the design notes):
* a block holds 16 consecutive tokens of every K/V head of a sequence;
* a new block is taken only when the sequence's last block is full (or it
  has none);
* the lowest-numbered free block is taken first, and a new sequence gets the
  lowest free id (any choice is correct; a fixed one makes results unique);
* fork: the child starts with a copy of the parent's page table; each block
  in it is referenced once more;
* copy-on-write: a token may only be written into a block that no other
  sequence references; a sequence about to write into a shared block (its
  partly filled last block) first takes a new block, has the old block's
  contents copied into it and repoints its table entry;
* release: each block of the sequence is referenced once less; a block no
  table references is free again;
* a reservation either succeeds completely or changes nothing; an invalid
  request (unknown id, negative count, a table growing past its width) is
  refused before free blocks are counted.

Two levels, each checkable on its own:
* ``LogicalKV`` is the definition a paged cache must reproduce: each live
  sequence is the list of its tokens in order, a fork copies the parent's
  list.
* ``PagePool`` is the allocator: block ids, reference counts, page tables.
  ``scatter_tokens`` / ``copy_blocks`` / ``gather`` move rows through a
  numpy page array, so a test can check that pages read back through the
  tables equal ``LogicalKV``.
"""
from __future__ import annotations

import copy

import numpy as np

BLOCK = 16


class OutOfBlocks(Exception):
    """Not enough free blocks (or free sequence ids) for a request."""


class InvalidRequest(Exception):
    """Unknown sequence id, negative count, or a table growing past its width."""


class LogicalKV:
    """The definition: each sequence is the ordered list of its token rows."""

    def __init__(self):
        self.seqs: dict[int, list] = {}

    def new(self, sid: int):
        self.seqs[sid] = []

    def fork(self, parent: int, child: int):
        self.seqs[child] = list(self.seqs[parent])

    def append(self, sid: int, rows):
        self.seqs[sid].extend(rows)

    def release(self, sid: int):
        del self.seqs[sid]


class PagePool:
    """Physical blocks with reference counts and per-sequence page tables."""

    def __init__(self, num_blocks: int, max_seqs: int, max_blocks_per_seq: int):
        self.num_blocks = num_blocks
        self.max_seqs = max_seqs
        self.max_blocks = max_blocks_per_seq
        self.refs = [0] * num_blocks
        self.tables: dict[int, list[int]] = {}
        self.lens: dict[int, int] = {}

    # -- helpers -----------------------------------------------------------
    def free_blocks(self) -> int:
        return sum(1 for r in self.refs if r == 0)

    def _take_block(self) -> int:
        for b in range(self.num_blocks):          # lowest free block first
            if self.refs[b] == 0:
                self.refs[b] = 1
                return b
        raise OutOfBlocks()

    def _check(self, sid: int):
        if sid not in self.tables:
            raise InvalidRequest(f"unknown sequence {sid}")

    # -- sequences -----------------------------------------------------------
    def new_seq(self) -> int:
        for sid in range(self.max_seqs):          # lowest free id
            if sid not in self.tables:
                self.tables[sid] = []
                self.lens[sid] = 0
                return sid
        raise OutOfBlocks()

    def fork(self, parent: int) -> int:
        self._check(parent)
        child = self.new_seq()
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.refs[b] += 1
        return child

    def release(self, sid: int):
        self._check(sid)
        for b in self.tables.pop(sid):
            self.refs[b] -= 1
        del self.lens[sid]

    # -- token slots ---------------------------------------------------------
    def _write_slot(self, sid: int) -> tuple[int, tuple | None]:
        """Slot for the next token of sid; the copy it needs first, if any."""
        table, pos = self.tables[sid], self.lens[sid]
        copied = None
        if pos % BLOCK == 0:                      # last block full (or none): take a new one
            table.append(self._take_block())
        elif self.refs[table[-1]] > 1:            # shared: copy before writing
            old = table[-1]
            new = self._take_block()
            self.refs[old] -= 1
            table[-1] = new
            copied = (old, new)
        self.lens[sid] = pos + 1
        return table[pos // BLOCK] * BLOCK + pos % BLOCK, copied

    def reserve(self, seqs, counts):
        """Slots for counts[i] new tokens of seqs[i], in order, and the block
        copies (src, dst) to perform before writing them.  All or nothing."""
        # An invalid request is refused before capacity is looked at.
        grow: dict[int, int] = {}
        for sid, c in zip(seqs, counts):
            self._check(sid)
            if c < 0:
                raise InvalidRequest("negative count")
            grow[sid] = grow.get(sid, 0) + c
        for sid, c in grow.items():
            if -(-(self.lens[sid] + c) // BLOCK) > self.max_blocks:
                raise InvalidRequest("page table full")
        saved = (copy.deepcopy(self.tables), dict(self.lens), list(self.refs))
        try:
            slots, copies = [], []
            for sid, c in zip(seqs, counts):
                for _ in range(c):
                    s, cp = self._write_slot(sid)
                    slots.append(s)
                    if cp is not None:
                        copies.append(cp)
            return slots, copies
        except OutOfBlocks:
            self.tables, self.lens, self.refs = saved
            raise

    def block_table(self, seqs, max_blocks: int):
        table = np.full((len(seqs), max_blocks), -1, dtype=np.int32)
        lens = np.zeros(len(seqs), dtype=np.int32)
        for i, sid in enumerate(seqs):
            self._check(sid)
            t = self.tables[sid]
            if len(t) > max_blocks:
                raise InvalidRequest("table wider than max_blocks")
            table[i, :len(t)] = t
            lens[i] = self.lens[sid]
        return table, lens


# -- moving rows through a page array [num_blocks, Hkv, 16, d] ---------------

def scatter_tokens(pages: np.ndarray, slots, rows: np.ndarray):
    """pages[s // 16, :, s % 16, :] = rows[i] for s = slots[i] (rows [n, Hkv, d])."""
    for i, s in enumerate(slots):
        pages[s // BLOCK, :, s % BLOCK, :] = rows[i]


def copy_blocks(pages: np.ndarray, copies):
    for src, dst in copies:
        pages[dst] = pages[src]


def gather(pages: np.ndarray, table_row, length: int) -> np.ndarray:
    """The logical rows [length, Hkv, d] of one sequence, read through its table."""
    out = np.empty((length,) + (pages.shape[1], pages.shape[3]), dtype=pages.dtype)
    for t in range(length):
        out[t] = pages[table_row[t // BLOCK], :, t % BLOCK, :]
    return out
