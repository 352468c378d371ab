"""Deterministic simulator of one sequence's heterogeneous KV cache (one layer).

TEST INFRASTRUCTURE ONLY (see the package docstring).

[P3] section 9 ("Heterogeneous KV Cache"): a request carries the exact recent window, the
compressed entries (one per m tokens: m = 4 for CSA, m' = 128 for HCA) and the
uncompressed tail of an incomplete block; block lifecycle rules create an entry whenever a
block completes, keep the last W tokens exact, and must keep tails consistent when a
request starts from a cached prefix.  The page proposes a CPU simulator of the memory
accounting and update rules; this is that simulator, written against the rules, with
values carried along so that a device implementation can be compared with it.

Reading for the device layout it models: the raw tokens live in a ring of R rows,
R = m * ceil((W + m - 1) / m) (room for the window and a tail, a whole number of blocks),
stored twice (slot p mod R and p mod R + R) so that any R consecutive positions are
contiguous rows.  Blocks are pooled with `oracle.pool` semantics.
"""
import numpy as np

from .csahca import pool


def ring_rows(W, m):
    """Rows R of the raw ring for window W and block size m."""
    return m * (-(-(W + m - 1) // m))


class KVSim:
    """State after every append: n tokens, n // m entries, a tail of n % m tokens, and
    the ring contents.  `append` returns the indices of the entries it created."""

    def __init__(self, c, m, W):
        self.c, self.m, self.W = c, m, W
        self.R = ring_rows(W, m)
        self.n = 0
        self.entries = np.zeros((0, c))
        self.ring_pos = np.full(2 * self.R, -1, dtype=np.int64)  # position held by each row
        self.ring_x = np.zeros((2 * self.R, c))
        self.ring_z = np.zeros((2 * self.R, c))
        self._raw_x = []   # every token appended (kept only to pool blocks here)
        self._raw_z = []

    def append(self, X, Z):
        X = np.asarray(X, dtype=np.float64).reshape(-1, self.c)
        Z = np.asarray(Z, dtype=np.float64).reshape(-1, self.c)
        n0 = self.n
        for j in range(X.shape[0]):
            p = n0 + j
            for slot in (p % self.R, p % self.R + self.R):
                self.ring_pos[slot] = p
                self.ring_x[slot] = X[j]
                self.ring_z[slot] = Z[j]
        self._raw_x.append(X)
        self._raw_z.append(Z)
        self.n = n0 + X.shape[0]
        first, last = n0 // self.m, self.n // self.m
        if last > first:
            allx, allz = np.vstack(self._raw_x), np.vstack(self._raw_z)
            lo, hi = first * self.m, last * self.m
            self.entries = np.vstack([self.entries, pool(allx[lo:hi], allz[lo:hi], self.m)])
        return list(range(first, last))

    def tail(self):
        """Positions of the uncompressed tail (tokens of the incomplete block)."""
        return list(range(self.n - self.n % self.m, self.n))

    def window_rows(self, L=None):
        """(first row, first position) of the last L tokens (default W) in the ring."""
        L = self.W if L is None else L
        L = min(L, self.n)
        p0 = self.n - L
        return p0 % self.R, p0

    def memory_bytes(self, elem_bytes):
        """Bytes one sequence holds for this layer: entries plus the doubled ring of values
        and gate logits."""
        return (self.entries.shape[0] * self.c + 2 * (2 * self.R) * self.c) * elem_bytes

    def fork(self, P):
        """A new request that shares this one's first P tokens (a prefix hit): the
        entries of the complete blocks before P and the ring rows of positions
        P - R .. P - 1 are carried over; the tail is P mod m tokens."""
        if P > self.n:
            raise ValueError("prefix longer than the request")
        s = KVSim(self.c, self.m, self.W)
        s.n = P
        s.entries = self.entries[:P // self.m].copy()
        allx, allz = np.vstack(self._raw_x), np.vstack(self._raw_z)
        s._raw_x, s._raw_z = [allx[:P]], [allz[:P]]
        for p in range(max(0, P - self.R), P):
            for slot in (p % self.R, p % self.R + self.R):
                s.ring_pos[slot] = p
                s.ring_x[slot] = allx[p]
                s.ring_z[slot] = allz[p]
        return s
