"""Plain block manager and block copy (test infrastructure only).

The bookkeeping of a paged KV cache, written from the pages:

* page "PagedAttention by hand", section "Why divide memory into physical
  blocks?": every block has the same size, the free list is a stack of
  interchangeable ids, and a sequence takes a new block only when its last
  one is full;
* same page, section "Memory Sharing (Copy-on-Write)": a reference count per
  physical block (how many sequences use it); candidates forked from one
  prompt share its blocks; before a sequence writes into a block whose count
  is above 1 it takes a fresh block, copies the shared block's contents into
  it, lowers the shared block's count by one and writes into the copy.

Where the pages leave a choice open the same policy as the library's pool is
taken (a specification, not shared code): the free stack first pops block 0,
then 1, 2, ...; a released sequence pushes its freed blocks in table order;
sequence ids count up from 0.

Only the tests, the smoke check and the benchmark's CPU baseline use this.
"""
from __future__ import annotations

import copy


class OutOfBlocks(Exception):
    pass


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        """free_order: the order in which the fresh stack hands blocks out
        (default 0, 1, 2, ...)."""
        assert num_blocks > 0 and block_size > 0
        self.B = block_size
        self.NB = num_blocks
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        assert sorted(order) == list(range(num_blocks))
        self.free = order[::-1]                         # top of stack = end
        self.refcount = [0] * num_blocks
        self.tables = {}     # seq id -> list of physical blocks
        self.lengths = {}    # seq id -> tokens
        self.next_id = 0

    # -- sequences ---------------------------------------------------------
    def create(self) -> int:
        sid = self.next_id
        self.next_id += 1
        self.tables[sid] = []
        self.lengths[sid] = 0
        return sid

    def fork(self, parent: int) -> int:
        child = self.create()
        self.tables[child] = list(self.tables[parent])
        self.lengths[child] = self.lengths[parent]
        for b in self.tables[child]:
            self.refcount[b] += 1
        return child

    def release(self, sid: int) -> None:
        for b in self.tables.pop(sid):
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free.append(b)
        del self.lengths[sid]

    # -- writes ------------------------------------------------------------
    def _blocks_needed(self, sid: int, n: int) -> int:
        """Fresh blocks that appending n tokens takes (copy included)."""
        if n == 0:
            return 0
        L, table = self.lengths[sid], self.tables[sid]
        room = len(table) * self.B - L              # free slots in the last block
        new = max(0, -(-(n - room) // self.B))      # ceil((n - room) / B)
        cow = 1 if room > 0 and self.refcount[table[-1]] > 1 else 0
        return new + cow

    def append(self, sid: int, n: int = 1):
        """Reserve slots for n new tokens.  Returns (slots, copy) where copy is
        (shared block, fresh block) or None."""
        if self._blocks_needed(sid, n) > len(self.free):
            raise OutOfBlocks
        table = self.tables[sid]
        copy = None
        slots = []
        for _ in range(n):
            pos = self.lengths[sid]
            j, off = divmod(pos, self.B)
            if j == len(table):                         # last block full: on demand
                b = self.free.pop()
                self.refcount[b] = 1
                table.append(b)
            elif self.refcount[table[j]] > 1:           # shared: copy on write
                shared = table[j]
                fresh = self.free.pop()
                self.refcount[fresh] = 1
                self.refcount[shared] -= 1
                table[j] = fresh
                copy = (shared, fresh)
            slots.append(table[j] * self.B + off)
            self.lengths[sid] = pos + 1
        return slots, copy

    def append_batch(self, sids):
        """One new token for each sequence in order; all or nothing (tried on
        a copy of the state, kept only if every sequence got its slot)."""
        if len(set(sids)) != len(sids):
            raise KeyError("repeated sequence id")
        trial = copy.deepcopy(self)
        slots, pairs = [], []
        for s in sids:
            sl, cp = trial.append(s, 1)          # raises OutOfBlocks: self untouched
            slots += sl
            if cp:
                pairs.append(cp)
        self.__dict__.update(trial.__dict__)
        return slots, pairs

    # -- views -------------------------------------------------------------
    def table(self, sid: int):
        return list(self.tables[sid])

    def export(self, sids, max_blocks: int, pad: int = 0):
        tables = [self.tables[s] + [pad] * (max_blocks - len(self.tables[s])) for s in sids]
        return tables, [self.lengths[s] for s in sids]


def copy_blocks(key_cache, value_cache, pairs):
    """Copy whole blocks src -> dst in both caches (host copies returned).

    Pairs whose ids fall outside the pool, or with src == dst, are skipped;
    the remaining dst blocks must be distinct and must not be another pair's
    src (each copy then reads an unchanged block)."""
    kc = key_cache.detach().to("cpu").clone()
    vc = value_cache.detach().to("cpu").clone()
    NB = kc.shape[0]
    live = [(int(s), int(d)) for s, d in pairs if 0 <= s < NB and 0 <= d < NB and s != d]
    dsts = [d for _, d in live]
    assert len(set(dsts)) == len(dsts), "two copies into one block"
    assert not set(dsts) & {s for s, _ in live}, "a copy target is also a copy source"
    src_k, src_v = key_cache.detach().to("cpu"), value_cache.detach().to("cpu")
    for s, d in live:
        kc[d] = src_k[s]
        vc[d] = src_v[s]
    return kc, vc
