"""Plain model of the KV-cache block manager (TEST INFRASTRUCTURE ONLY).

Only ``tests/`` may import this module.  It is the block manager written out in
the simplest way -- Python lists and dicts, one operation at a time -- and
shares no code with the library's C++ manager.

What it models, and where the pages define it:

* A block holds ``block_size`` tokens and a reference count; a sequence's block
  table lists its physical blocks in logical order, so token t of a sequence
  lives in slot ``table[t // block_size] * block_size + t % block_size`` --
  page "Nano-vLLM-Ascend", section 2.1 (``Block`` with ``ref_count``,
  ``BlockTable`` mapping logical positions to physical blocks; a 1000-token
  sequence of 16-token blocks takes ``ceil(1000/16) = 63`` blocks).
* Blocks are shared between sequences (prefix sharing for long contexts, page
  "vLLM-Ascend ...", section 4); a shared block is copied before one sharer
  writes into it (copy on write), and a block whose count reaches zero is free
  again.  A pool in which every sequence has been freed is entirely free: the
  reference-count check the pages give for memory leaks (page
  "Nano-vLLM-Ascend", section 4.2, problem 3).

The allocation policy is part of the model so that results can be compared
exactly: free blocks form a stack that first hands out 0, 1, 2, ...; a freed
block is pushed and is the next one handed out.
"""
from __future__ import annotations


class NoBlocks(Exception):
    """The pool has too few free blocks (the C ABI's PA_ERR_NO_BLOCKS)."""


class BlockManagerModel:
    def __init__(self, num_blocks: int, block_size: int):
        assert num_blocks >= 1 and block_size >= 1
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = list(range(num_blocks - 1, -1, -1))   # top of the stack is the end
        self.refs = [0] * num_blocks
        self.tables: dict[int, list[int]] = {}
        self.tokens: dict[int, int] = {}
        self.copies: list[tuple[int, int]] = []

    # -- helpers ----------------------------------------------------------
    def _blocks_for(self, n: int) -> int:
        return -(-n // self.block_size)

    def _take(self) -> int:
        b = self.free.pop()
        self.refs[b] = 1
        return b

    def _release(self, b: int) -> None:
        self.refs[b] -= 1
        if self.refs[b] == 0:
            self.free.append(b)

    def slot(self, seq: int, t: int) -> int:
        return self.tables[seq][t // self.block_size] * self.block_size + t % self.block_size

    # -- operations -------------------------------------------------------
    def add(self, seq: int, n: int) -> list[int]:
        if seq in self.tables or n < 0:
            raise ValueError("bad add")
        if self._blocks_for(n) > len(self.free):
            raise NoBlocks
        self.tables[seq] = [self._take() for _ in range(self._blocks_for(n))]
        self.tokens[seq] = n
        return [self.slot(seq, t) for t in range(n)]

    def fork(self, parent: int, child: int, n: int) -> None:
        if parent not in self.tables or child in self.tables or not 0 <= n <= self.tokens[parent]:
            raise ValueError("bad fork")
        shared = self.tables[parent][:self._blocks_for(n)]
        for b in shared:
            self.refs[b] += 1
        self.tables[child] = list(shared)
        self.tokens[child] = n

    def append(self, seq: int, n: int) -> list[int]:
        if seq not in self.tables or n < 0:
            raise ValueError("bad append")
        table, have = self.tables[seq], self.tokens[seq]
        partial_shared = have % self.block_size != 0 and self.refs[table[-1]] > 1
        need = self._blocks_for(have + n) - len(table) + (1 if partial_shared and n > 0 else 0)
        if need > len(self.free):
            raise NoBlocks
        if n == 0:
            return []
        if partial_shared:                      # copy on write
            old = table[-1]
            new = self._take()
            self._release(old)
            table[-1] = new
            self.copies.append((old, new))
        slots = []
        for t in range(have, have + n):
            if t // self.block_size == len(table):
                table.append(self._take())
            slots.append(self.slot(seq, t))
        self.tokens[seq] = have + n
        return slots

    def free_seq(self, seq: int) -> None:
        if seq not in self.tables:
            raise ValueError("bad free")
        for b in self.tables.pop(seq):
            self._release(b)
        del self.tokens[seq]

    def take_copies(self, capacity: int) -> list[tuple[int, int]]:
        out, self.copies = self.copies[:capacity], self.copies[capacity:]
        return out

    # -- checks -----------------------------------------------------------
    def check_invariants(self) -> None:
        """Counts equal table references; free blocks are exactly the zero-count ones."""
        refs = [0] * self.num_blocks
        for table in self.tables.values():
            for b in table:
                refs[b] += 1
        assert refs == self.refs
        assert sorted(self.free) == [b for b in range(self.num_blocks) if self.refs[b] == 0]
        assert len(set(self.free)) == len(self.free)
        for seq, table in self.tables.items():
            assert len(table) == self._blocks_for(self.tokens[seq])
