"""Pins of the KV-cache lifecycle simulator (oracle/kvcache.py) against the rules of the
heterogeneous cache ([P3] section 9) and the pages' entry counts."""
import numpy as np

from oracle import kvcache as K
from oracle import pool
from tests.conftest import read_golden


def _chunks(rng, total, sizes):
    out, left = [], total
    while left > 0:
        s = int(min(left, sizes[rng.integers(len(sizes))]))
        out.append(s)
        left -= s
    return out


def test_counts_match_the_pages():
    """n = 10^6 tokens (the pages' budget example, window 128): the stored compressed
    entries plus the window are the printed counts; the tails are n mod m."""
    g = read_golden("budget_counts.txt")
    n, W = g["n"], 128
    rng = np.random.default_rng(0)
    for m, stored in ((4, g["csa_stored"]), (128, g["hca_stored"])):
        s = K.KVSim(1, m, W)
        for k in _chunks(rng, n, [1, 3, 4, 127, 128, 1000, 65536, 250000]):
            s.append(np.zeros((k, 1)), np.zeros((k, 1)))
        assert s.n == n
        assert s.entries.shape[0] + W == stored
        assert len(s.tail()) == n % m


def test_ring_size_window_and_tail():
    for W, m in ((128, 4), (128, 128), (0, 4), (5, 3), (128, 1)):
        R = K.ring_rows(W, m)
        assert R % m == 0 and R >= W + m - 1 and R - m < W + m - 1  # the smallest such
    rng = np.random.default_rng(1)
    s = K.KVSim(2, 4, 16)
    pos = 0
    for k in _chunks(rng, 200, [1, 2, 3, 5, 19, 40]):
        made = s.append(rng.normal(size=(k, 2)), rng.normal(size=(k, 2)))
        assert made == list(range(pos // 4, (pos + k) // 4))  # entries as blocks complete
        pos += k
        r0, p0 = s.window_rows()
        L = min(16, pos)
        assert p0 == pos - L
        np.testing.assert_array_equal(s.ring_pos[r0:r0 + L], np.arange(pos - L, pos))  # contiguous
        t = s.tail()
        assert t == list(range(pos - pos % 4, pos))
        for p in t:  # the tail is still in the ring
            assert p in s.ring_pos


def test_appends_equal_one_pass_and_fork_continues():
    rng = np.random.default_rng(2)
    n, c = 700, 3
    X, Z = rng.normal(size=(n, c)), rng.normal(size=(n, c)) * 2
    for m in (4, 128):
        s = K.KVSim(c, m, 128)
        at = 0
        cuts = _chunks(rng, n, [1, 2, 7, 64, 129, 300])
        for k in cuts:
            s.append(X[at:at + k], Z[at:at + k])
            at += k
        np.testing.assert_allclose(s.entries, pool(X, Z, m), rtol=0, atol=1e-15)
        # a prefix hit at P: the fork carries the complete blocks and the ring rows, and
        # appending the rest gives the same cache
        for P in (0, 1, 130, 257, 512, n):
            f = s.fork(P)
            assert f.entries.shape[0] == P // m and f.tail() == list(range(P - P % m, P))
            f.append(X[P:], Z[P:])
            np.testing.assert_allclose(f.entries, s.entries, atol=1e-15)
            keep = f.ring_pos >= max(0, n - f.R)
            np.testing.assert_array_equal(f.ring_pos[keep], s.ring_pos[keep])
            np.testing.assert_array_equal(f.ring_x[keep], s.ring_x[keep])


def test_memory_accounting():
    """Per sequence and layer: entries plus the doubled ring (values and gate logits)."""
    s = K.KVSim(512, 4, 128)
    s.n = 1 << 20
    s.entries = np.zeros(((1 << 20) // 4, 512))
    R = K.ring_rows(128, 4)
    assert s.memory_bytes(2) == (262144 * 512 + 4 * R * 512) * 2
