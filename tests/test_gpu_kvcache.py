"""GPU parity of the KV-cache lifecycle (csahca_kv_append / csahca_kv_fork) against the
CPU simulator oracle.kvcache.KVSim, on identical input bytes.

After every append: each ring row that holds one of the last R positions equals that
token bit for bit (both halves of the doubled ring); the entries made equal the
simulator's within the pooling tolerance (fp32 max |d| <= 1e-5; bf16 |d| <= one bf16 ulp
of the fp64 value + 2^-16 * sum_j S_j |x_j|).  A fork continues exactly as the request
it was cut from would have; attention reading its window from the ring returns the bits
of attention reading a dense copy of the window.
"""
import numpy as np
import pytest
import torch

import compressed_attention_compress_amd as lib
import oracle
from oracle import kvcache as K
from synthgen.configs import BF16, F32
from synthgen.host import encode
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    H.require_gpu()


def bf16_ulp(x):
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


class DevCache:
    """Device rings and entries of B sequences, appended through the C ABI."""

    def __init__(self, B, c, m, W, dtype, n_max):
        self.B, self.c, self.m, self.W, self.dtype = B, c, m, W, dtype
        self.R = lib.csahca_kv_ring_rows(W, m)
        self.NE = max(n_max // m, 1)
        self.rx = H.empty((B, 2 * self.R, c), dtype).zero_()
        self.rz = H.empty((B, 2 * self.R, c), dtype).zero_()
        self.ent = H.empty((B, self.NE, c), dtype).zero_()
        self.n = 0

    def append(self, dX, dZ, lo, k, P=None):
        """Append tokens lo .. lo+k-1 of device [B, total, c] arrays (strided view)."""
        B, total, c = dX.shape
        lib.csahca_kv_append(self.rx, self.rz, self.ent, dX[:, lo:], dZ[:, lo:], P, B, self.n, k, c,
                             self.m, self.W, self.dtype, total * c, 2 * self.R * c, self.NE * c)
        self.n += k

    def fork(self):
        d = DevCache(self.B, self.c, self.m, self.W, self.dtype, self.NE * self.m)
        lib.csahca_kv_fork(d.rx, d.rz, d.ent, self.rx, self.rz, self.ent, self.B, self.n // self.m,
                           self.c, self.m, self.W, self.dtype, 2 * self.R * self.c, self.NE * self.c)
        d.n = self.n
        return d


def check_ring(dev, sim, codes_x, codes_z, b):
    """Every row holding one of the last R positions equals that token's codes."""
    rx = H.to_host_codes(dev.rx, dev.dtype)[b]
    rz = H.to_host_codes(dev.rz, dev.dtype)[b]
    live = np.nonzero(sim.ring_pos >= max(0, sim.n - sim.R))[0]
    assert len(live) == 2 * min(sim.n, sim.R)
    pos = sim.ring_pos[live]
    np.testing.assert_array_equal(rx[live], codes_x[b, pos])
    np.testing.assert_array_equal(rz[live], codes_z[b, pos])
    r0, p0 = sim.window_rows(sim.R)
    L = sim.n - p0
    np.testing.assert_array_equal(rx[r0:r0 + L], codes_x[b, p0:sim.n])  # contiguous window


def check_entries(dev, sim, X, Z, b, lo, hi):
    got = oracle.decode(H.to_host_codes(dev.ent, dev.dtype)[b, lo:hi], dev.dtype)
    ref = sim.entries[lo:hi]
    assert got.shape == ref.shape
    if dev.dtype == F32:
        assert np.max(np.abs(got - ref), initial=0.0) <= 1e-5
    else:
        m = dev.m
        cond = oracle.pool(np.abs(X[b, lo * m:hi * m]), Z[b, lo * m:hi * m], m)
        bad = np.abs(got - ref) > bf16_ulp(ref) + 2.0 ** -16 * cond
        assert not bad.any(), f"seq {b}: {bad.sum()} pooled values outside tolerance"


def make_tokens(rng, B, n, c, dtype):
    cx = encode(rng.standard_normal((B, n, c), dtype=np.float32) * 0.1, dtype)
    cz = encode(rng.standard_normal((B, n, c), dtype=np.float32), dtype)
    return cx, cz, oracle.decode(cx, dtype), oracle.decode(cz, dtype)


CASES = [
    (BF16, 4, 128, [1, 1, 2, 3, 4, 5, 7, 130, 1, 1, 1, 300, 3, 1, 64, 133]),
    (BF16, 128, 128, [1, 100, 27, 1, 300, 128, 5, 700, 1, 255]),
    (F32, 4, 16, [3, 1, 1, 1, 17, 40, 2, 9, 1, 1, 1, 1]),
    (F32, 3, 5, [2, 2, 2, 1, 10, 4, 1, 1, 30]),   # m not a power of two, R = 9
    (BF16, 4, 0, [1, 2, 3, 9, 4, 1]),              # no window: the ring holds one block
    (F32, 1, 8, [1, 5, 1, 20]),                    # every token is an entry
]


@pytest.mark.parametrize("dtype,m,W,chunks", CASES)
def test_append_lifecycle(dtype, m, W, chunks):
    print(f"[kv append dtype={dtype} m={m} W={W} chunks={chunks}]", flush=True)
    rng = np.random.default_rng(1000 * m + W + len(chunks))
    B, c = 2, (512 if dtype == BF16 else 64)
    total = sum(chunks)
    cx, cz, X, Z = make_tokens(rng, B, total, c, dtype)
    dX, dZ = H.to_dev(cx), H.to_dev(cz)
    dev = DevCache(B, c, m, W, dtype, total)
    sims = [K.KVSim(c, m, W) for _ in range(B)]
    lo = 0
    for k in chunks:
        dev.append(dX, dZ, lo, k)
        torch.cuda.synchronize()
        for b in range(B):
            made = sims[b].append(X[b, lo:lo + k], Z[b, lo:lo + k])
            check_ring(dev, sims[b], cx, cz, b)
            if made:
                check_entries(dev, sims[b], X, Z, b, made[0], made[-1] + 1)
        lo += k
    for b in range(B):
        check_entries(dev, sims[b], X, Z, b, 0, total // m)


def test_append_with_position_bias():
    rng = np.random.default_rng(5)
    B, c, m, W = 2, 512, 4, 128
    chunks = [3, 2, 1, 8, 131, 2]
    total = sum(chunks)
    cx, cz, X, Z = make_tokens(rng, B, total, c, BF16)
    P = rng.standard_normal((m, c)).astype(np.float32)
    dX, dZ, dP = H.to_dev(cx), H.to_dev(cz), H.to_dev(P)
    dev = DevCache(B, c, m, W, BF16, total)
    lo = 0
    for k in chunks:
        dev.append(dX, dZ, lo, k, P=dP)
        lo += k
    torch.cuda.synchronize()
    got = oracle.decode(H.to_host_codes(dev.ent, BF16), BF16)
    for b in range(B):
        ref = oracle.pool(X[b], Z[b], m, P)
        cond = oracle.pool(np.abs(X[b]), Z[b], m, P)
        bad = np.abs(got[b, :total // m] - ref) > bf16_ulp(ref) + 2.0 ** -16 * cond
        assert not bad.any()


@pytest.mark.parametrize("m,P", [(4, 4 * 50 + 3), (128, 128 * 3 + 77), (4, 4 * 80)])
def test_fork_continues_like_the_prefix_owner(m, P):
    """Fork at the source's length P, then give source and fork different continuations:
    each matches its own simulator, and the fork's bits equal those of a request that
    appended prefix + continuation itself in the same chunks."""
    print(f"[kv fork m={m} P={P}]", flush=True)
    rng = np.random.default_rng(m + P)
    B, c, W = 2, 512, 128
    pre = [P // 3, 1, P - P // 3 - 1]
    cont = [1, 2, m, 3 * m + 1, 1, 200]
    nc = sum(cont)
    cx, cz, X, Z = make_tokens(rng, B, P + 2 * nc, c, BF16)
    # sequence A = prefix + continuation a (tokens P .. P+nc-1),
    # sequence B = prefix + continuation b (tokens P+nc .. P+2nc-1)
    ib = np.r_[np.arange(P), np.arange(P + nc, P + 2 * nc)]
    cxb, czb, Xb, Zb = cx[:, ib], cz[:, ib], X[:, ib], Z[:, ib]
    dX, dZ = H.to_dev(cx), H.to_dev(cz)
    dXb, dZb = H.to_dev(cxb), H.to_dev(czb)
    src = DevCache(B, c, m, W, BF16, P + nc)
    lo = 0
    for k in pre:
        src.append(dX, dZ, lo, k)
        lo += k
    fk = src.fork()
    fresh = DevCache(B, c, m, W, BF16, P + nc)
    lo = 0
    for k in pre:
        fresh.append(dXb, dZb, lo, k)
        lo += k
    for k in cont:
        src.append(dX, dZ, lo, k)
        fk.append(dXb, dZb, lo, k)
        fresh.append(dXb, dZb, lo, k)
        lo += k
    torch.cuda.synchronize()
    NE = (P + nc) // m
    assert torch.equal(fk.ent[:, :NE], fresh.ent[:, :NE])
    assert torch.equal(fk.rx, fresh.rx) and torch.equal(fk.rz, fresh.rz)
    for b in range(B):
        sa = K.KVSim(c, m, W)
        sa.append(X[b, :P], Z[b, :P])
        sb = sa.fork(P)
        sa.append(X[b, P:P + nc], Z[b, P:P + nc])
        sb.append(Xb[b, P:], Zb[b, P:])
        check_entries(src, sa, X, Z, b, 0, NE)
        check_entries(fk, sb, Xb, Zb, b, 0, NE)
        check_ring(src, sa, cx, cz, b)
        check_ring(fk, sb, cxb, czb, b)


@pytest.mark.parametrize("m", [4, 128])
def test_attend_reads_window_from_ring(m):
    """hca_attend over the cache's entries with the window taken straight from the ring
    (win_kv = ring, L = 2R, win_pos = R * floor(max(0, n - R) / R)) returns the bits of the
    same call on a dense copy of the window, over decode steps that move the window across
    the ring's wrap, and for a chunk of R - W + 1 queries."""
    print(f"[kv attend from ring m={m}]", flush=True)
    rng = np.random.default_rng(77 + m)
    B, c, W, n_h = 2, 512, 128, 64
    R = lib.csahca_kv_ring_rows(W, m)
    steps = [1] * 6 + [R - W + 1] + [1] * 3
    n0 = 2 * R + 5
    total = n0 + sum(steps)
    cx, cz, _, _ = make_tokens(rng, B, total, c, BF16)
    dX, dZ = H.to_dev(cx), H.to_dev(cz)
    dev = DevCache(B, c, m, W, BF16, total)
    dev.append(dX, dZ, 0, n0)
    lo = n0
    scale = 1.0 / np.sqrt(c)
    for k in steps:
        dev.append(dX, dZ, lo, k)
        lo += k
        n = dev.n
        Tq = k
        Q = H.to_dev(encode(rng.standard_normal((B, Tq, n_h, c), dtype=np.float32), BF16))
        q_pos = torch.full((B,), n - Tq, dtype=torch.int32, device=H.DEV)
        C = dev.ent[:, :n // m].contiguous()
        wp_ring = R * (max(0, n - R) // R)
        o_r, l_r = H.run_hca_attend(Q, C, dev.rx, torch.full((B,), wp_ring, dtype=torch.int32, device=H.DEV),
                                    q_pos, m, W, BF16, scale=scale)
        wp = max(0, n - Tq - W + 1)
        dense = dX[:, wp:n].contiguous()
        o_d, l_d = H.run_hca_attend(Q, C, dense, torch.full((B,), wp, dtype=torch.int32, device=H.DEV),
                                    q_pos, m, W, BF16, scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(o_r, o_d), f"n={n} Tq={Tq}"
        assert torch.equal(l_r, l_d), f"n={n} Tq={Tq}"


def test_append_far_into_a_long_sequence():
    """A sequence first given 2^20 + 3 tokens in one chunk (a prefill), then decode
    appends: ring slots and entry indices at million-token positions."""
    print("[kv append far positions]", flush=True)
    rng = np.random.default_rng(12)
    B, c, m, W = 1, 64, 4, 128
    n0 = (1 << 20) + 3
    chunks = [n0, 1, 1, 2, 5, 130]
    total = sum(chunks)
    cx = rng.standard_normal((B, total, c), dtype=np.float32) * 0.1
    cz = rng.standard_normal((B, total, c), dtype=np.float32)
    dX, dZ = H.to_dev(cx), H.to_dev(cz)
    dev = DevCache(B, c, m, W, F32, total)
    sim = K.KVSim(c, m, W)
    X, Z = cx.astype(np.float64), cz.astype(np.float64)
    lo = 0
    for k in chunks:
        dev.append(dX, dZ, lo, k)
        torch.cuda.synchronize()
        made = sim.append(X[0, lo:lo + k], Z[0, lo:lo + k])
        check_ring(dev, sim, cx, cz, 0)
        if made:  # the last few entries made (the first chunk makes 2^18 of them)
            check_entries(dev, sim, X, Z, 0, max(made[0], made[-1] - 7), made[-1] + 1)
        lo += k
