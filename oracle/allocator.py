"""Step-by-step model of the block manager (host side).

TEST INFRASTRUCTURE ONLY (see the package docstring).  Pinned by
tests/test_oracle_allocator.py.

Semantics, from the pages:

* free blocks sit in a queue; allocation takes from the front and freed
  blocks go to the back ([vllm] §4.1, FreeKVCacheBlockQueue popleft/append).
  The initial queue order is an input (the seeded ``free_order``).
* a sequence needs ceil(tokens / block_size) blocks; a new block is taken
  when the last one is full ([k4i] #the-block-manager allocate/append_slot;
  [tut] §3.3.2).
* sharing increments a block's reference count; freeing decrements it and
  returns the block to the queue at zero ([atb] reference-count section;
  [k4i] #the-block-manager free).
* writing into a block whose count is above one copies it first
  (copy-on-write): take a free block, copy the shared block into it,
  decrement the old block's count, repoint the table, then write; with a
  count of one the write goes in place ([k4i] #cow steps 1-5; [atb]
  copy-on-write section).

* prefix cache ([k4i] #prefix-caching; [vllm] §4.2-4.3): a full block is
  known by the chain (parent block's key, its token ids, an extra key); a
  new prompt reuses the cached blocks of its full blocks from the left up to
  the first miss (count + 1), takes fresh blocks for the rest and registers
  the keys of the fresh full blocks.  Reading taken where the pages differ:
  a block whose count drops to zero keeps its key and goes to the back of
  the queue (so the queue's remove-from-the-middle serves hits on it and its
  front-first hand-out is the least-recently-freed eviction of §4.1); the
  key is dropped when the queue hands the block out for new content.  The
  chain here is the exact nested tuple, so this model has no hash
  collisions.

Allocation is all-or-nothing: when the queue holds fewer blocks than an
append needs, ``OutOfBlocks`` is raised and no state changes.
"""
from __future__ import annotations

from collections import deque
from typing import Dict, List, Tuple


class OutOfBlocks(RuntimeError):
    pass


class BlockManagerModel:
    def __init__(self, num_blocks: int, block_size: int, free_order):
        self.block_size = int(block_size)
        self.num_blocks = int(num_blocks)
        order = [int(b) for b in free_order]
        assert sorted(order) == list(range(num_blocks)), "free_order must permute the pool"
        self.free = deque(order)
        self.ref = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}
        self._next = 0
        self.cache: Dict[tuple, int] = {}       # chain key -> block
        self.block_key: Dict[int, tuple] = {}   # cached block -> its chain key

    # ---------------------------------------------------------------- seqs
    def add_seq(self) -> int:
        sid = self._next
        self._next += 1
        self.tables[sid] = []
        self.lens[sid] = 0
        return sid

    def _take(self) -> int:
        b = self.free.popleft()
        assert self.ref[b] == 0
        self.ref[b] = 1
        key = self.block_key.pop(b, None)  # new content: the cached key goes
        if key is not None and self.cache.get(key) == b:
            del self.cache[key]
        return b

    def add_seq_cached(self, tokens, extra: int = 0) -> Tuple[int, int]:
        """New sequence holding the prompt ``tokens`` with the prefix cache.

        Returns (sequence id, tokens covered by reused blocks)."""
        bs = self.block_size
        tokens = [int(t) for t in tokens]
        nfull, nblocks = len(tokens) // bs, -(-len(tokens) // bs)
        keys, hits, parent = [], [], None
        for i in range(nfull):
            key = (parent, tuple(tokens[i * bs:(i + 1) * bs]), int(extra))
            keys.append(key)
            if len(hits) == i and key in self.cache:
                hits.append(self.cache[key])
            parent = key
        revived = sum(1 for b in hits if self.ref[b] == 0)
        if nblocks - len(hits) + revived > len(self.free):
            raise OutOfBlocks(f"prompt of {len(tokens)}: free {len(self.free)}")
        sid = self.add_seq()
        tab = self.tables[sid]
        for b in hits:
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1
            tab.append(b)
        for i in range(len(hits), nblocks):
            b = self._take()
            tab.append(b)
            if i < nfull:
                old = self.cache.get(keys[i])
                if old is not None and old != b:
                    self.block_key.pop(old, None)
                self.cache[keys[i]] = b
                self.block_key[b] = keys[i]
        self.lens[sid] = len(tokens)
        return sid, len(hits) * bs

    def blocks_needed(self, sid: int, n: int) -> int:
        """Free blocks an append of n tokens consumes (new blocks + copy-on-write)."""
        bs, L, tab = self.block_size, self.lens[sid], self.tables[sid]
        need = -(-(L + n) // bs) - len(tab)
        if n > 0 and L % bs != 0 and self.ref[tab[-1]] > 1:
            need += 1
        return need

    def append(self, sid: int, n: int) -> Tuple[List[int], List[Tuple[int, int]]]:
        """Append n tokens to sequence sid.

        Returns (slots, cow) where slots[i] = block * block_size + offset of
        the token at position len + i ([vllm] §3.2) and cow lists the
        (source, destination) block copies the caller must perform before
        writing the new tokens.
        """
        if self.blocks_needed(sid, n) > len(self.free):
            raise OutOfBlocks(f"seq {sid}: need {self.blocks_needed(sid, n)}, free {len(self.free)}")
        bs, tab = self.block_size, self.tables[sid]
        slots, cow = [], []
        for p in range(self.lens[sid], self.lens[sid] + n):
            lb = p // bs
            if lb == len(tab):
                tab.append(self._take())
            elif self.ref[tab[lb]] > 1:
                old = tab[lb]
                new = self._take()
                self.ref[old] -= 1
                tab[lb] = new
                cow.append((old, new))
            slots.append(tab[lb] * bs + p % bs)
        self.lens[sid] += n
        return slots, cow

    def fork(self, parent: int) -> int:
        """New sequence sharing every block of ``parent`` (counts + 1)."""
        child = self.add_seq()
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1
        return child

    def free_seq(self, sid: int) -> None:
        for b in self.tables.pop(sid):
            self.ref[b] -= 1
            assert self.ref[b] >= 0
            if self.ref[b] == 0:
                self.free.append(b)
        del self.lens[sid]

    # ------------------------------------------------------------- queries
    def block_table(self, sid: int) -> List[int]:
        return list(self.tables[sid])

    def num_free(self) -> int:
        return len(self.free)

    def num_cached(self) -> int:
        return len(self.cache)
