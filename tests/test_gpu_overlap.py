"""GPU parity of the overlapped two-stream CSA pooling (csa_compress_overlap) against the
CPU oracle, on identical input bytes.

Tolerance as for single-stream pooling: fp32 max |d| <= 1e-5; bf16 |d| <= one bf16 ulp of
the fp64 value + 2^-16 * sum_j S_j |x_j| over the entry's 2m raw values.
"""
import numpy as np
import pytest
import torch

import oracle
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


def check_overlap(h, dtype, m, prev, got_dev, P=None, entries=None):
    """h: host codes (Xa, Za, Xb, Zb), each [B, n, c].  entries: the entry indices to
    compare (all when None)."""
    got = oracle.decode(H.to_host_codes(got_dev, dtype), dtype)
    Xa, Za, Xb, Zb = (oracle.decode(a, dtype) for a in h)
    B, n, _ = Xa.shape
    for b in range(B):
        if entries is None:
            ref = oracle.pool_overlap(Xa[b], Za[b], Xb[b], Zb[b], m, P, prev)
            cond = oracle.pool_overlap(np.abs(Xa[b]), Za[b], np.abs(Xb[b]), Zb[b], m, P, prev)
            g = got[b]
        else:
            # entry e reads blocks e+prev-1 and e+prev: cut those 2m tokens (an append)
            ref, cond, g = [], [], []
            for e in entries:
                i = e + prev
                lo = max(0, i - 1) * m
                sl = slice(lo, (i + 1) * m)
                pv = 1 if i >= 1 else 0
                ref.append(oracle.pool_overlap(Xa[b, sl], Za[b, sl], Xb[b, sl], Zb[b, sl], m, P, pv)[-1])
                cond.append(oracle.pool_overlap(np.abs(Xa[b, sl]), Za[b, sl], np.abs(Xb[b, sl]), Zb[b, sl],
                                                m, P, pv)[-1])
                g.append(got[b, e])
            ref, cond, g = np.array(ref), np.array(cond), np.array(g)
        assert g.shape == ref.shape
        if dtype == F32:
            assert np.max(np.abs(g - ref), initial=0.0) <= 1e-5
        else:
            bad = np.abs(g - ref) > bf16_ulp(ref) + 2.0 ** -16 * cond
            assert not bad.any(), f"seq {b}: {bad.sum()} pooled values outside tolerance"


def inputs(rng, B, n, c, dtype):
    X = lambda: encode(rng.standard_normal((B, n, c), dtype=np.float32) * 0.1, dtype)
    Zg = lambda: encode(rng.standard_normal((B, n, c), dtype=np.float32), dtype)
    return X(), Zg(), X(), Zg()


@pytest.mark.parametrize("dtype,m,B,n,prev", [
    (BF16, 4, 2, 4 * 300 + 3, 0),    # many blocks, ragged tail
    (BF16, 4, 4, 8, 1),              # a decode append: blocks i-1 and i, one entry each
    (BF16, 4, 3, 4 * 5 + 1, 1),
    (BF16, 16, 2, 16 * 400, 0),      # many blocks, 8-token chunks
    (BF16, 128, 2, 128 * 5 + 7, 0),  # few blocks of many tokens (split over sub-ranges)
    (BF16, 128, 1, 256, 1),
    (F32, 4, 1, 4096, 0),
    (F32, 1, 1, 40, 0),
    (BF16, 3, 1, 3 * 50 + 2, 1),
])
def test_overlap_pool_parity(dtype, m, B, n, prev):
    print(f"[overlap pool dtype={dtype} m={m} B={B} n={n} prev={prev}]", flush=True)
    rng = np.random.default_rng(m * 1000 + n)
    c = 512 if dtype == BF16 else 64
    h = inputs(rng, B, n, c, dtype)
    P = rng.standard_normal((2 * m, c)).astype(np.float32)
    d = [H.to_dev(a) for a in h]
    for bias in (None, P):
        out = H.run_pool_overlap(*d, m, prev, dtype, P=None if bias is None else H.to_dev(bias))
        torch.cuda.synchronize()
        check_overlap(h, dtype, m, prev, out, P=bias)


def test_overlap_stream_b_gated_off_equals_single_stream():
    """With stream b's logits at the lowest finite bf16 its weights are exactly 0, and the
    kernel returns csa_compress's bits for stream a."""
    rng = np.random.default_rng(3)
    B, n, c, m = 2, 4 * 200, 512, 4
    Xa, Za, Xb, _ = inputs(rng, B, n, c, BF16)
    Zb = np.full((B, n, c), 0xFF7F, dtype=np.uint16)  # -3.39e38
    d = [H.to_dev(a) for a in (Xa, Za, Xb, Zb)]
    ov = H.run_pool_overlap(*d, m, 0, BF16)
    single = H.run_pool(d[0], d[1], m, BF16)
    torch.cuda.synchronize()
    assert torch.equal(ov, single)


def test_overlap_full_sequence_sampled():
    """One 131072-token sequence (the 128K decode shape), every entry computed, sampled
    entries checked against the oracle on the blocks they read."""
    print("[overlap pool full sequence]", flush=True)
    rng = np.random.default_rng(17)
    B, n, c, m = 1, 131072, 512, 4
    h = inputs(rng, B, n, c, BF16)
    d = [H.to_dev(a) for a in h]
    out = H.run_pool_overlap(*d, m, 0, BF16)
    torch.cuda.synchronize()
    N = n // m
    entries = sorted({0, 1, N - 1} | {int(x) for x in rng.integers(0, N, 64)})
    check_overlap(h, BF16, m, 0, out, entries=entries)
