"""GPU parity of RMSNorm + partial RoPE (csahca_norm_rope, csahca_compress_norm_rope,
csa_compress_overlap_norm_rope) against the CPU oracle, on identical input bytes.

Tolerances (per element; S = |a| + |b| over the normalised pair the element belongs to,
or |a| alone outside the rotated channels):
- rows:    bf16 |d| <= ulp_bf16(ref) + 2^-16 S;  fp32 |d| <= 2^-20 S;
- pooling: the pooling bound carried through the norm and the rotation, i.e. bf16
  |d| <= ulp_bf16(ref) + 2^-16 (|g_a| K_a + |g_b| K_b) / rms + 2^-18 S with K the
  pooling condition sum_j S_j |x_j| of the pair's channels; fp32 drops the ulp term and
  uses 2^-20 S.
Angles are formed in double on both sides, so positions up to 2^21 are covered.
"""
import numpy as np
import pytest
import torch

import compressed_attention_compress_amd as lib
import oracle
from synthgen.configs import BF16, F32
from synthgen.host import encode
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

EPS, THETA = 1e-6, 10000.0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    H.require_gpu()


def bf16_ulp(x):
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def pair_sum(a, d):
    """|a| plus, on the last d channels, the magnitude of the pair partner."""
    s = np.abs(a).copy()
    c = a.shape[-1]
    if d:
        t = np.abs(a[..., c - d:])
        partner = t.reshape(*t.shape[:-1], d // 2, 2)[..., ::-1].reshape(t.shape)
        s[..., c - d:] += partner
    return s


def rows_tol(ref_norm, ref, d, dtype):
    S = pair_sum(ref_norm, d)
    if dtype == F32:
        return 2.0 ** -20 * S + 1e-30
    return bf16_ulp(ref) + 2.0 ** -16 * S


@pytest.mark.parametrize("dtype,c,d,H_,T,norm,gain,inplace", [
    (BF16, 512, 64, 4, 5, 1, True, False),
    (BF16, 512, 64, 1, 37, 1, False, True),
    (BF16, 512, 0, 2, 3, 1, True, False),     # norm only
    (BF16, 512, 512, 2, 3, 0, False, False),  # RoPE only, every channel rotated
    (F32, 64, 16, 8, 9, 1, True, False),
    (F32, 64, 8, 1, 300, 1, True, True),
    (F32, 8, 8, 3, 4, 1, True, False),        # one lane per row
    (F32, 64, 64, 1, 3, 1, False, False),     # more pairs than lanes per row (the per-lane path)
])
def test_norm_rope_rows(dtype, c, d, H_, T, norm, gain, inplace):
    print(f"[norm_rope rows dtype={dtype} c={c} d={d} H={H_} T={T} norm={norm}]", flush=True)
    rng = np.random.default_rng(c + d + T)
    B = 3
    x = encode(rng.standard_normal((B, T, H_, c), dtype=np.float32) * 0.7, dtype)
    g = rng.uniform(0.5, 1.5, size=c).astype(np.float32) if gain else None
    pos = np.array([0, 1 << 20, (1 << 30) + 123457], dtype=np.int32)  # up to 2^30
    pstride = 3
    dx = H.to_dev(x)
    dy = dx if inplace else torch.empty_like(dx)
    lib.csahca_norm_rope(dx, dy, None if g is None else H.to_dev(g), H.to_dev(pos), B, T, H_, c,
                         pstride, d, EPS, THETA, norm, dtype)
    torch.cuda.synchronize()
    got = oracle.decode(H.to_host_codes(dy, dtype), dtype)
    X = oracle.decode(x, dtype)
    p = pos[:, None, None] + pstride * np.arange(T)[None, :, None]
    p = np.broadcast_to(p, (B, T, H_))
    xn = oracle.rmsnorm(X, g, EPS) if norm else X
    ref = oracle.rope_tail(xn, p, d, THETA)
    bad = np.abs(got - ref) > rows_tol(xn, ref, d, dtype)
    assert not bad.any(), f"{bad.sum()} of {bad.size} outside tolerance, max |d| {np.abs(got - ref).max()}"


def pooled_reference(X, Z, m, P, g, d, entry0, ov=None, prev=0):
    """Oracle entries and their tolerance for one sequence."""
    if ov is None:
        pooled = oracle.pool(X, Z, m, P)
        cond = oracle.pool(np.abs(X), Z, m, P)
    else:
        Xb, Zb = ov
        pooled = oracle.pool_overlap(X, Z, Xb, Zb, m, P, prev)
        cond = oracle.pool_overlap(np.abs(X), Z, np.abs(Xb), Zb, m, P, prev)
    pos = oracle.entry_positions(m, entry0, pooled.shape[0])
    xn = oracle.rmsnorm(pooled, g, EPS)
    ref = oracle.rope_tail(xn, pos, d, THETA)
    rms = np.sqrt((pooled ** 2).mean(axis=-1, keepdims=True) + EPS)
    gg = np.ones(X.shape[1]) if g is None else np.abs(g)
    return ref, xn, pair_sum(gg * cond, d) / rms


def check_pooled(got, ref, xn, kcond, d, dtype):
    S = pair_sum(xn, d)
    if dtype == F32:  # the same float32 arithmetic, rounded once to float32
        tol = 2.0 ** -16 * kcond + 2.0 ** -20 * S
    else:
        tol = bf16_ulp(ref) + 2.0 ** -16 * kcond + 2.0 ** -18 * S
    bad = np.abs(got - ref) > tol
    assert not bad.any(), f"{bad.sum()} of {bad.size} outside tolerance, max |d| {np.abs(got - ref).max()}"


@pytest.mark.parametrize("dtype,m,B,n,bias,entry0", [
    (BF16, 4, 2, 4 * 700 + 3, True, 0),      # many blocks (one lane group per entry)
    (BF16, 4, 2, 4 * 50, False, 262000),     # far positions
    (BF16, 128, 2, 128 * 3 + 5, True, 7),    # few blocks of many tokens (workgroup merge)
    (BF16, 128, 4, 128, False, 8191),        # a decode append
    (F32, 4, 1, 4 * 300, True, 0),
    (F32, 16, 2, 16 * 20 + 3, False, 5),     # few blocks at c = 64 (8 lanes per slice group)
])
def test_pool_norm_rope(dtype, m, B, n, bias, entry0):
    print(f"[pool norm_rope dtype={dtype} m={m} B={B} n={n} entry0={entry0}]", flush=True)
    rng = np.random.default_rng(m * 100 + n)
    c = 512 if dtype == BF16 else 64
    d = 64 if dtype == BF16 else 16
    X = encode(rng.standard_normal((B, n, c), dtype=np.float32) * 0.1, dtype)
    Z = encode(rng.standard_normal((B, n, c), dtype=np.float32), dtype)
    P = rng.standard_normal((m, c)).astype(np.float32) if bias else None
    g = rng.uniform(0.5, 1.5, size=c).astype(np.float32)
    N = n // m
    out = H.empty((B, N, c), dtype)
    lib.csahca_compress_norm_rope(H.to_dev(X), H.to_dev(Z), None if P is None else H.to_dev(P),
                                  H.to_dev(g), out, B, n, c, m, entry0, d, EPS, THETA, dtype,
                                  n * c, N * c)
    torch.cuda.synchronize()
    got = oracle.decode(H.to_host_codes(out, dtype), dtype)
    Xd, Zd = oracle.decode(X, dtype), oracle.decode(Z, dtype)
    for b in range(B):
        ref, xn, kc = pooled_reference(Xd[b], Zd[b], m, P, g, d, entry0)
        check_pooled(got[b], ref, xn, kc, d, dtype)


@pytest.mark.parametrize("m", [4, 128])
def test_pool_norm_rope_append_equals_whole_pass(m):
    """An append of the last block (entry0 = its index) writes the bits the whole pass wrote
    for that entry."""
    rng = np.random.default_rng(m)
    B, c, N = 2, 512, 8
    n = N * m
    X = H.to_dev(encode(rng.standard_normal((B, n, c), dtype=np.float32) * 0.1, BF16))
    Z = H.to_dev(encode(rng.standard_normal((B, n, c), dtype=np.float32), BF16))
    g = H.to_dev(rng.uniform(0.5, 1.5, size=c).astype(np.float32))
    whole = H.empty((B, N, c), BF16)
    lib.csahca_compress_norm_rope(X, Z, None, g, whole, B, n, c, m, 0, 64, EPS, THETA, BF16, n * c, N * c)
    app = H.empty((B, N, c), BF16).zero_()
    for e in range(N):
        lib.csahca_compress_norm_rope(X[:, e * m:], Z[:, e * m:], None, g, app[:, e:], B, m, c, m, e, 64,
                                      EPS, THETA, BF16, n * c, N * c)
    torch.cuda.synchronize()
    # m = 4: both take the one-lane-group-per-entry kernel; m = 128: both the workgroup
    # merge with the same sub-ranges
    assert torch.equal(app, whole)


@pytest.mark.parametrize("m,B,n,prev", [(4, 2, 4 * 300 + 1, 0), (4, 3, 8, 1), (16, 2, 16 * 6, 1)])
def test_overlap_pool_norm_rope(m, B, n, prev):
    print(f"[overlap pool norm_rope m={m} B={B} n={n} prev={prev}]", flush=True)
    rng = np.random.default_rng(m + n + prev)
    c, d = 512, 64
    arrs = [encode(rng.standard_normal((B, n, c), dtype=np.float32) * (0.1 if k % 2 == 0 else 1.0), BF16)
            for k in range(4)]
    P = rng.standard_normal((2 * m, c)).astype(np.float32)
    g = rng.uniform(0.5, 1.5, size=c).astype(np.float32)
    N = n // m - prev
    entry0 = 40
    out = H.empty((B, N, c), BF16)
    lib.csa_compress_overlap_norm_rope(*[H.to_dev(a) for a in arrs], H.to_dev(P), H.to_dev(g), out, B, n,
                                       c, m, prev, entry0, d, EPS, THETA, BF16, n * c, N * c)
    torch.cuda.synchronize()
    got = oracle.decode(H.to_host_codes(out, BF16), BF16)
    Xa, Za, Xb, Zb = (oracle.decode(a, BF16) for a in arrs)
    for b in range(B):
        ref, xn, kc = pooled_reference(Xa[b], Za[b], m, P, g, d, entry0,
                                       ov=(Xb[b], Zb[b]), prev=prev)
        check_pooled(got[b], ref, xn, kc, d, BF16)


def test_chain_attention_over_normalised_rotated_rows():
    """Everything on the GPU (entries pooled with the norm and rotation fused, queries and
    window rows through csahca_norm_rope, then hca_attend), checked stage by stage as the
    rest of the suite is: the normalised, rotated entries, window rows and queries the GPU
    stored against the oracle at the row and pooling tolerances, then the attention over
    exactly those stored bf16 rows at 2e-2 x RMS(O_ref) plus the output's own bf16
    rounding (half an ulp of O_ref; see below).  The oracle-all-the-way error
    (fp64 rows, no bf16 storage) is printed beside it: when a head's softmax is peaked its
    output is close to one row, so it inherits that row's bf16 rounding (2^-9 |v|)."""
    rng = np.random.default_rng(31)
    B, c, m, W, n_h, d = 2, 512, 4, 32, 16, 64
    n = 4 * 96 + 2                                 # decode at position n - 1
    X = encode(rng.standard_normal((B, n, c), dtype=np.float32), BF16)
    Z = encode(rng.standard_normal((B, n, c), dtype=np.float32), BF16)
    Q = encode(rng.standard_normal((B, 1, n_h, c), dtype=np.float32), BF16)
    gk = rng.uniform(0.5, 1.5, size=c).astype(np.float32)
    gq = rng.uniform(0.5, 1.5, size=c).astype(np.float32)
    N = n // m
    dX, dZ = H.to_dev(X), H.to_dev(Z)
    C = H.empty((B, N, c), BF16)
    lib.csahca_compress_norm_rope(dX, dZ, None, H.to_dev(gk), C, B, n, c, m, 0, d, EPS, THETA, BF16,
                                  n * c, N * c)
    wp = n - W
    win = H.empty((B, W, c), BF16)
    win_pos = torch.full((B,), wp, dtype=torch.int32, device=H.DEV)
    # the window read straight out of the [B, n, c] raw array (batch stride n * c)
    lib.csahca_norm_rope(dX[:, wp:], win, H.to_dev(gk), win_pos, B, W, 1, c, 1, d, EPS, THETA, 1, BF16,
                         x_bstride=n * c, y_bstride=W * c)
    q_pos = torch.full((B,), n - 1, dtype=torch.int32, device=H.DEV)
    dQ = H.to_dev(Q)
    lib.csahca_norm_rope(dQ, dQ, H.to_dev(gq), q_pos, B, 1, n_h, c, 1, d, EPS, THETA, 1, BF16)
    out, _ = H.run_hca_attend(dQ, C, win, win_pos, q_pos, m, W, BF16, scale=1.0 / np.sqrt(c))
    torch.cuda.synchronize()
    got = oracle.decode(H.to_host_codes(out, BF16), BF16)
    Cg = oracle.decode(H.to_host_codes(C, BF16), BF16)
    Wg = oracle.decode(H.to_host_codes(win, BF16), BF16)
    Qg = oracle.decode(H.to_host_codes(dQ, BF16), BF16)
    Xd, Zd, Qd = oracle.decode(X, BF16), oracle.decode(Z, BF16), oracle.decode(Q, BF16)
    for b in range(B):
        # stage 1: the stored normalised, rotated rows against the oracle
        Cr, xn, kc = pooled_reference(Xd[b], Zd[b], m, None, gk, d, 0)
        check_pooled(Cg[b], Cr, xn, kc, d, BF16)
        wn = oracle.rmsnorm(Xd[b, wp:], gk, EPS)
        Wr = oracle.rope_tail(wn, np.arange(wp, n), d, THETA)
        assert not (np.abs(Wg[b] - Wr) > rows_tol(wn, Wr, d, BF16)).any(), "window rows"
        qn = oracle.rmsnorm(Qd[b, 0], gq, EPS)
        qr = oracle.rope_tail(qn, np.full(n_h, n - 1), d, THETA)
        assert not (np.abs(Qg[b, 0] - qr) > rows_tol(qn, qr, d, BF16)).any(), "queries"
        # stage 2: attention over the rows the GPU consumed.  The bound is 2e-2 x RMS(O_ref)
        # plus the half-ulp rounding of the stored bf16 output: here the output's largest
        # value (1.58 in sequence 0) is 8.9x its RMS, so that rounding alone (2^-8 = 0.0039)
        # is 1.10x of 2e-2 x RMS (0.0035) and no bf16 output could meet the bare bound.
        ref, _ = oracle.attend(Qg[b, 0], oracle.hca_rows(Cg[b], m, Wg[b], wp, n - 1, W), 1.0 / np.sqrt(c))
        err = np.abs(got[b, 0] - ref)
        rms_tol = 2e-2 * np.sqrt((ref ** 2).mean())
        excess = err - 0.5 * bf16_ulp(ref)       # what is left after the output's own rounding
        # oracle all the way, for the record
        full, _ = oracle.attend(qr, oracle.hca_rows(Cr, m, Wr, wp, n - 1, W), 1.0 / np.sqrt(c))
        print(f"chain seq {b}: max |d| = {err.max():.3g} ({err.max() / rms_tol:.3f} of 2e-2 x RMS), "
              f"beyond the output's half-ulp {excess.max() / rms_tol:.3f} of 2e-2 x RMS; "
              f"against fp64 rows throughout {np.abs(got[b, 0] - full).max():.3g}", flush=True)
        assert excess.max() <= rms_tol, err.max()
