"""Bookkeeping of the GDN prefix-state cache, written plainly from the "qev_fast/statecache.py" page
(StateCache: _lookup, _bounds, _row, _done, _touch, _evict). TEST INFRASTRUCTURE ONLY.

Only the recurrent part is modelled: a checkpoint is the fp32 state and conv tail after its first
`pos` tokens; the attention K / V the page also keeps is not part of this layer. Capacity is counted
in checkpoints (every checkpoint has the same size), where the page counts bytes. Checkpoints are
numbered in the order they are made, so that another implementation can be compared with this one.
"""
from __future__ import annotations

from collections import OrderedDict

import numpy as np


class PrefixCacheModel:
    def __init__(self, capacity: int, stride: int = 2048, tail: int = 16, align: int = 64, max_chunk: int = 2048,
                 min_prefix: int = 256):
        self.capacity, self.stride, self.tail, self.align = capacity, stride, tail, align
        self.max_chunk, self.min_prefix = max_chunk, min_prefix
        self.groups = []              # [ids, [checkpoint numbers]] in creation order
        self.ckpts = OrderedDict()    # number -> (group index, pos); least recently used first
        self.made = 0
        self.stats = dict(rows=0, hits=0, partial=0, cold=0, plain=0, tokens_reused=0, tokens_computed=0,
                          ckpts_made=0, evicted=0)

    def _down(self, x):
        return x - x % self.align if self.align else x

    def _lookup(self, x):
        """Checkpoints usable by a row whose checkpointable prefix is x: pos <= the prefix it shares with the
        row that made them."""
        out = []
        for gi, (ids, nums) in enumerate(self.groups):
            m = min(len(ids), len(x))
            if m == 0 or ids[0] != x[0]:
                continue
            ne = np.flatnonzero(ids[:m] != x[:m])
            lcp = int(ne[0]) if len(ne) else m
            out += [c for c in nums if c in self.ckpts and self.ckpts[c][1] <= lcp]
        return out

    def _bounds(self, c, p):
        """Chunk ends from c for a state of p tokens: multiples of stride, p - tail and p (rounded down to
        align), no chunk longer than max_chunk."""
        e = self._down(p)
        b = {k for k in range(self.stride, e, self.stride) if k > c} if self.stride else set()
        if self.tail and self._down(p - self.tail) > c:
            b.add(self._down(p - self.tail))
        if e > c:
            b.add(e)
        out, s = [], c
        for x in sorted(b):
            while x - s > self.max_chunk:
                s += self.max_chunk
                out.append(s)
            out.append(x)
            s = x
        return out

    def row(self, ids, p_state):
        """Plan and book one row -> (restored checkpoint number or -1, c0, p, bounds, new checkpoint numbers
        that survive the row's eviction, or -1 for those evicted at once)."""
        ids = np.asarray(ids, dtype=np.int64)
        n = len(ids)
        p = self._down(min(p_state, n))
        if p < self.min_prefix:
            self.stats["plain"] += 1
            self.stats["tokens_computed"] += n
            return -1, 0, p, [], []
        x = ids[:p]
        cands = self._lookup(x)
        best = None
        for c in cands:  # the first of the deepest
            if best is None or self.ckpts[c][1] > self.ckpts[best][1]:
                best = c
        c0 = self.ckpts[best][1] if best is not None else 0
        self.stats["rows"] += 1
        self.stats["hits" if c0 == p else ("partial" if c0 > 0 else "cold")] += 1
        bounds = self._bounds(c0, min(p_state, n)) if c0 < p else []  # the page passes the unrounded length
        self.stats["tokens_reused"] += c0
        self.stats["tokens_computed"] += n - c0
        if best is not None:
            self.ckpts.move_to_end(best)
        new = []
        if bounds:
            self.groups.append([x.copy(), []])
            gi = len(self.groups) - 1
            for b in bounds:
                num = self.made
                self.made += 1
                self.groups[gi][1].append(num)
                self.ckpts[num] = (gi, b)
                new.append(num)
                self.stats["ckpts_made"] += 1
        while len(self.ckpts) > self.capacity:
            self.ckpts.popitem(last=False)
            self.stats["evicted"] += 1
        return (best if best is not None else -1), c0, p, bounds, [c if c in self.ckpts else -1 for c in new]

    def alive(self):
        return sorted(self.ckpts)
