"""Reference model of the GDN prefix-state cache's bookkeeping. TEST INFRASTRUCTURE ONLY: the tests use it
to check the library's host-side cache (gdn_pcache_*); nothing in the product imports it.

What it models, as the "qev_fast/statecache.py" page's StateCache describes the cache (its lookup, chunk
ends, row bookkeeping and LRU eviction), restated as rules:

  * a checkpoint is the recurrent state (fp32 state + conv tail) of one sequence after its first `pos`
    tokens, made while some earlier row ran; the attention K / V that the page also keeps belongs to
    other layers and is left out;
  * a row of n tokens whose state should cover p_state tokens can only checkpoint P = min(p_state, n)
    tokens, rounded down to a multiple of `align` (p); rows with p < min_prefix bypass the cache;
  * a checkpoint serves a new row when its pos is no longer than the prefix the new row (its first p
    tokens) has in common with the row that made it; the row starts from the deepest such checkpoint
    (among equally deep ones, the one made first), or from zero;
  * the row then stops, and saves a checkpoint, at every multiple of `stride` strictly between the
    start and p, at P - tail rounded down, and at p itself (each only if it lies past the start),
    with extra stops so that no stretch is longer than max_chunk;
  * capacity counts checkpoints (all have the same size; the page counts bytes); using a checkpoint
    makes it the most recently used one, new checkpoints are the most recent, and the least recently
    used ones go while there are too many.

Checkpoints are numbered in the order they are made so that another implementation can be compared
with this one number for number. A row whose checkpoints have all been evicted is forgotten.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class _Checkpoint:
    num: int      # order of creation
    pos: int      # tokens the saved state covers
    owner: int    # key of the row (token ids) that made it


def common_prefix(a: np.ndarray, b: np.ndarray) -> int:
    """Length of the longest common prefix of two id arrays."""
    m = min(len(a), len(b))
    same = a[:m] == b[:m]
    if same.all():
        return m
    return int(np.argmin(same))  # first position where they differ


class PrefixCacheModel:
    def __init__(self, capacity: int, stride: int = 2048, tail: int = 16, align: int = 64, max_chunk: int = 2048,
                 min_prefix: int = 256):
        if max_chunk <= 0:
            raise ValueError("max_chunk must be positive")
        self.capacity, self.stride, self.tail, self.align = capacity, stride, tail, align
        self.max_chunk, self.min_prefix = max_chunk, min_prefix
        self.lru: list[_Checkpoint] = []        # live checkpoints, least recently used first
        self.owners: dict[int, np.ndarray] = {}  # row key -> the token ids it checkpointed
        self.next_num = 0
        self.next_owner = 0
        self.stats = dict(rows=0, hits=0, partial=0, cold=0, plain=0, tokens_reused=0, tokens_computed=0,
                          ckpts_made=0, evicted=0, rows_kept=0)

    def round_down(self, x: int) -> int:
        if not self.align:
            return x
        return (x // self.align) * self.align

    def deepest(self, prefix: np.ndarray):
        """The live checkpoint a row with this checkpointable prefix starts from, or None."""
        shared = {}   # owner -> common prefix length with this row, computed once per owner
        best = None
        for ck in sorted(self.lru, key=lambda c: c.num):
            if ck.owner not in shared:
                shared[ck.owner] = common_prefix(self.owners[ck.owner], prefix)
            if ck.pos <= shared[ck.owner] and (best is None or ck.pos > best.pos):
                best = ck
        return best

    def chunk_ends(self, start: int, state_len: int) -> list[int]:
        """The stops of a row that resumes at `start` and should checkpoint `state_len` tokens."""
        end = self.round_down(state_len)
        stops = set()
        if self.stride:
            k = (start // self.stride + 1) * self.stride
            while k < end:
                stops.add(k)
                k += self.stride
        if self.tail:
            before_tail = self.round_down(state_len - self.tail)
            if before_tail > start:
                stops.add(before_tail)
        if end > start:
            stops.add(end)
        ends, prev = [], start
        for stop in sorted(stops):
            extra = (stop - prev - 1) // self.max_chunk  # stretches longer than max_chunk are cut
            ends.extend(prev + self.max_chunk * i for i in range(1, extra + 1))
            ends.append(stop)
            prev = stop
        return ends

    def _evict(self):
        while len(self.lru) > self.capacity:
            gone = self.lru.pop(0)
            self.stats["evicted"] += 1
            if not any(c.owner == gone.owner for c in self.lru):
                del self.owners[gone.owner]

    def row(self, ids, p_state):
        """Plan and book one row -> (restored checkpoint number or -1, c0, p, chunk ends, the new
        checkpoints' numbers, with -1 for those evicted at once)."""
        ids = np.asarray(ids, dtype=np.int64)
        n = len(ids)
        state_len = min(p_state, n)
        p = self.round_down(state_len)
        if p < self.min_prefix:
            self.stats["plain"] += 1
            self.stats["tokens_computed"] += n
            return -1, 0, p, [], []
        prefix = ids[:p]
        start_ck = self.deepest(prefix)
        c0 = start_ck.pos if start_ck is not None else 0
        self.stats["rows"] += 1
        if c0 == p:
            self.stats["hits"] += 1
        elif c0 > 0:
            self.stats["partial"] += 1
        else:
            self.stats["cold"] += 1
        self.stats["tokens_reused"] += c0
        self.stats["tokens_computed"] += n - c0
        if start_ck is not None:  # a use: most recently used now
            self.lru.remove(start_ck)
            self.lru.append(start_ck)
        ends = self.chunk_ends(c0, state_len) if c0 < p else []
        made = []
        if ends:
            owner = self.next_owner
            self.next_owner += 1
            self.owners[owner] = prefix.copy()
            for pos in ends:
                ck = _Checkpoint(self.next_num, pos, owner)
                self.next_num += 1
                self.lru.append(ck)
                made.append(ck.num)
                self.stats["ckpts_made"] += 1
        self._evict()
        self.stats["rows_kept"] = len(self.owners)
        live = {c.num for c in self.lru}
        return (start_ck.num if start_ck is not None else -1), c0, p, ends, [m if m in live else -1 for m in made]

    def alive(self):
        return sorted(c.num for c in self.lru)

    def rows_remembered(self) -> int:
        return len(self.owners)
