"""csahca_compress_pair against the two separate calls (csa_compress, hca_compress): the
entries must be the same bits, in the fused launch (one side with few entries of many
tokens) and in the fallback of two launches, and the separate calls are checked against
the oracle.  Tolerance against the oracle as for pooling: fp32 max |d| <= 1e-5; bf16
|d| <= one bf16 ulp of the fp64 value + 2^-16 * sum_j S_j |x_j|.
"""
import zlib

import numpy as np
import pytest
import torch

import compressed_attention_compress_amd as lib
import oracle
from synthgen.configs import BF16, F32
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    H.require_gpu()


def _side(g, B, n, c, dt, pad=0):
    """X, Z [B, n + pad, c] (pad: extra rows, so the batch stride exceeds n * c)."""
    tdt = torch.bfloat16 if dt == BF16 else torch.float32
    X = (torch.randn((B, n + pad, c), generator=g, device="cuda") / 8).to(tdt)
    Z = torch.randn((B, n + pad, c), generator=g, device="cuda").to(tdt)
    return X, Z


def _codes(t, dt):
    """Host storage codes of a device tensor (bf16 as its 16-bit patterns)."""
    return H.to_host_codes(t.contiguous().view(torch.int16) if dt == BF16 else t, dt)


def _check_oracle(X, Z, out, m, dt):
    got = oracle.decode(_codes(out, dt), dt)
    x = oracle.decode(_codes(X, dt), dt)
    z = oracle.decode(_codes(Z, dt), dt)
    n = X.shape[1] // m * m
    for b in range(X.shape[0]):
        ref = oracle.pool(x[b, :n], z[b, :n], m)
        if dt == F32:
            assert np.max(np.abs(got[b] - ref)) <= 1e-5
        else:
            cond = oracle.pool(np.abs(x[b, :n]), z[b, :n], m)
            ax = np.maximum(np.abs(ref), 2.0 ** -126)
            ulp = 2.0 ** (np.floor(np.log2(ax)) - 7)
            assert np.all(np.abs(got[b] - ref) <= ulp + 2.0 ** -16 * cond)


CASES = {
    # name: (B, c, (n_a, m_a), (n_b, m_b), dtype, pad)
    "decode_pair": (4, 512, (4, 4), (128, 128), BF16, 0),          # fused
    "decode_pair_swapped": (4, 512, (128, 128), (4, 4), BF16, 0),  # fused, sides swapped
    "chunk_pair": (1, 512, (8192, 4), (8192, 128), BF16, 0),       # fused, many CSA entries
    "ragged_strides": (3, 512, (4 * 37 + 3, 4), (128 * 2 + 5, 128), BF16, 24),
    "both_many": (2, 512, (4 * 4096, 4), (128 * 600, 128), BF16, 0),  # two launches
    "hca_side_empty": (2, 512, (4 * 9, 4), (100, 128), BF16, 0),      # side b emits nothing
    "fp32_small_c": (2, 64, (4 * 5, 4), (128 * 3, 128), F32, 0),      # fused, 8 slices
}


@pytest.mark.parametrize("name", list(CASES))
def test_pair_equals_separate_calls(name):
    B, c, (n_a, m_a), (n_b, m_b), dt, pad = CASES[name]
    print(f"[pool pair {name}]", flush=True)
    g = torch.Generator(device="cuda").manual_seed(zlib.crc32(name.encode()) % 1000)
    Xa, Za = _side(g, B, n_a, c, dt, pad)
    Xb, Zb = _side(g, B, n_b, c, dt, pad)
    ibs_a, ibs_b = (n_a + pad) * c, (n_b + pad) * c
    Na, Nb = n_a // m_a, n_b // m_b
    tdt = Xa.dtype
    sep_a = torch.full((B, max(Na, 1) + 1, c), 7, dtype=tdt, device="cuda")
    sep_b = torch.full((B, max(Nb, 1) + 1, c), 7, dtype=tdt, device="cuda")
    pair_a, pair_b = sep_a.clone(), sep_b.clone()
    obs_a, obs_b = sep_a.shape[1] * c, sep_b.shape[1] * c
    lib.csa_compress(Xa, Za, None, sep_a, B, n_a, c, m_a, dt, ibs_a, obs_a)
    lib.hca_compress(Xb, Zb, None, sep_b, B, n_b, c, m_b, dt, ibs_b, obs_b)
    lib.csahca_compress_pair(Xa, Za, pair_a, n_a, m_a, ibs_a, obs_a, Xb, Zb, pair_b, n_b, m_b, ibs_b,
                             obs_b, B, c, dt)
    torch.cuda.synchronize()
    assert torch.equal(pair_a.view(torch.int16 if dt == BF16 else torch.int32),
                       sep_a.view(torch.int16 if dt == BF16 else torch.int32))
    assert torch.equal(pair_b.view(torch.int16 if dt == BF16 else torch.int32),
                       sep_b.view(torch.int16 if dt == BF16 else torch.int32))
    # rows past the entries are untouched
    assert bool((pair_a[:, Na:] == 7).all()) and bool((pair_b[:, Nb:] == 7).all())
    if B * n_a * c <= 1 << 21:  # the oracle on the smaller cases
        if Na:
            _check_oracle(Xa[:, :n_a], Za[:, :n_a], pair_a[:, :Na], m_a, dt)
        if Nb:
            _check_oracle(Xb[:, :n_b], Zb[:, :n_b], pair_b[:, :Nb], m_b, dt)


def test_pair_in_a_graph_replays():
    """The decode pair inside a HIP graph, replayed with new inputs between replays."""
    B, c, dt = 4, 512, BF16
    g = torch.Generator(device="cuda").manual_seed(5)
    Xa, Za = _side(g, B, 4, c, dt)
    Xb, Zb = _side(g, B, 128, c, dt)
    oa = torch.zeros((B, 1, c), dtype=Xa.dtype, device="cuda")
    ob = torch.zeros((B, 1, c), dtype=Xa.dtype, device="cuda")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        lib.csahca_compress_pair(Xa, Za, oa, 4, 4, 4 * c, c, Xb, Zb, ob, 128, 128, 128 * c, c, B, c, dt,
                                 stream=s)
    for rep in range(3):
        Xa.copy_(_side(g, B, 4, c, dt)[0])
        Zb.copy_(_side(g, B, 128, c, dt)[1])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ra = torch.empty_like(oa)
        rb = torch.empty_like(ob)
        lib.csa_compress(Xa, Za, None, ra, B, 4, c, 4, dt, 4 * c, c)
        lib.hca_compress(Xb, Zb, None, rb, B, 128, c, 128, dt, 128 * c, c)
        torch.cuda.synchronize()
        assert torch.equal(oa.view(torch.int16), ra.view(torch.int16)), rep
        assert torch.equal(ob.view(torch.int16), rb.view(torch.int16)), rep


NR_CASES = ["decode_pair", "decode_pair_swapped", "chunk_pair", "ragged_strides", "hca_side_empty",
            "fp32_small_c"]


@pytest.mark.parametrize("name", NR_CASES)
def test_pair_norm_rope_equals_separate_calls(name):
    """csahca_compress_pair_norm_rope against two csahca_compress_norm_rope calls (same
    bits), each side with its own gain and first entry; the decode pair also against the
    oracle (pooling, RMSNorm, RoPE at position m * entry)."""
    from tests.test_gpu_normrope import check_pooled, pooled_reference

    B, c, (n_a, m_a), (n_b, m_b), dt, pad = CASES[name]
    print(f"[pool pair norm_rope {name}]", flush=True)
    g = torch.Generator(device="cuda").manual_seed(zlib.crc32(name.encode()) % 1000 + 1)
    Xa, Za = _side(g, B, n_a, c, dt, pad)
    Xb, Zb = _side(g, B, n_b, c, dt, pad)
    ga = torch.rand((c,), generator=g, device="cuda") + 0.5
    gb = torch.rand((c,), generator=g, device="cuda") + 0.5
    e0a, e0b = 1000, 7
    d, eps, theta = min(64, c), 1e-6, 10000.0
    ibs_a, ibs_b = (n_a + pad) * c, (n_b + pad) * c
    Na, Nb = n_a // m_a, n_b // m_b
    tdt = Xa.dtype
    sep_a = torch.full((B, max(Na, 1) + 1, c), 7, dtype=tdt, device="cuda")
    sep_b = torch.full((B, max(Nb, 1) + 1, c), 7, dtype=tdt, device="cuda")
    pair_a, pair_b = sep_a.clone(), sep_b.clone()
    obs_a, obs_b = sep_a.shape[1] * c, sep_b.shape[1] * c
    lib.csahca_compress_norm_rope(Xa, Za, None, ga, sep_a, B, n_a, c, m_a, e0a, d, eps, theta, dt, ibs_a,
                                  obs_a)
    lib.csahca_compress_norm_rope(Xb, Zb, None, gb, sep_b, B, n_b, c, m_b, e0b, d, eps, theta, dt, ibs_b,
                                  obs_b)
    lib.csahca_compress_pair_norm_rope(Xa, Za, ga, pair_a, n_a, m_a, e0a, ibs_a, obs_a, Xb, Zb, gb, pair_b,
                                       n_b, m_b, e0b, ibs_b, obs_b, B, c, d, eps, theta, dt)
    torch.cuda.synchronize()
    iv = torch.int16 if dt == BF16 else torch.int32
    assert torch.equal(pair_a.view(iv), sep_a.view(iv))
    assert torch.equal(pair_b.view(iv), sep_b.view(iv))
    assert bool((pair_a[:, Na:] == 7).all()) and bool((pair_b[:, Nb:] == 7).all())
    if name == "decode_pair":
        for X, Z, out, m, gg, e0, N in ((Xa, Za, pair_a, m_a, ga, e0a, Na), (Xb, Zb, pair_b, m_b, gb, e0b, Nb)):
            x = oracle.decode(_codes(X, dt), dt)
            z = oracle.decode(_codes(Z, dt), dt)
            got = oracle.decode(_codes(out, dt), dt)
            for b in range(B):
                ref, xn, kc = pooled_reference(x[b, :N * m], z[b, :N * m], m, None, gg.cpu().numpy(), d, e0)
                check_pooled(got[b, :N], ref, xn, kc, d, dt)


@pytest.mark.parametrize("name,T,sides", [("decode_pair", 1, "ab"), ("decode_pair_swapped", 3, "ab"),
                                          ("ragged_strides", 2, "ab"), ("hca_side_empty", 1, "ab"),
                                          ("decode_pair", 1, "a"), ("hca_side_empty", 2, "b"),
                                          ("fp32_small_c", 2, "ab")])
def test_pair_norm_rope_rows_equals_separate_calls(name, T, sides):
    """csahca_compress_pair_norm_rope_rows against csahca_compress_pair_norm_rope and
    csahca_norm_rope calls on the rows (same bits): the window rows of the sides named in
    `sides` (the other side's row pointers NULL), each with its side's gain and its own
    positions, in one launch (decode shapes, one side without entries) and after the
    fallback launches (float32); rows past T, and a side without rows, are left alone."""
    B, c, (n_a, m_a), (n_b, m_b), dt, pad = CASES[name]
    print(f"[pool pair norm_rope rows {name} T={T}]", flush=True)
    g = torch.Generator(device="cuda").manual_seed(zlib.crc32(name.encode()) % 1000 + 2)
    Xa, Za = _side(g, B, n_a, c, dt, pad)
    Xb, Zb = _side(g, B, n_b, c, dt, pad)
    ga = torch.rand((c,), generator=g, device="cuda") + 0.5
    gb = torch.rand((c,), generator=g, device="cuda") + 0.5
    e0a, e0b = 1000, 7
    d, eps, theta = min(64, c), 1e-6, 10000.0
    ibs_a, ibs_b = (n_a + pad) * c, (n_b + pad) * c
    Na, Nb = n_a // m_a, n_b // m_b
    tdt = Xa.dtype
    sep_a = torch.full((B, max(Na, 1) + 1, c), 7, dtype=tdt, device="cuda")
    sep_b = torch.full((B, max(Nb, 1) + 1, c), 7, dtype=tdt, device="cuda")
    pair_a, pair_b = sep_a.clone(), sep_b.clone()
    obs_a, obs_b = sep_a.shape[1] * c, sep_b.shape[1] * c
    # rows: the last T raw tokens of each side into a window buffer of T + 5 rows per
    # sequence (strided), at positions from a device array
    LW = T + 5
    xa_rows, xb_rows = Xa[:, n_a + pad - T:], Xb[:, n_b + pad - T:]
    ya_sep = torch.full((B, LW, c), 3, dtype=tdt, device="cuda")
    yb_sep = ya_sep.clone()
    ya_pair, yb_pair = ya_sep.clone(), yb_sep.clone()
    pos_a = torch.arange(B, dtype=torch.int32, device="cuda") * 1000003 + n_a - T
    pos_b = torch.arange(B, dtype=torch.int32, device="cuda") * 7919 + n_b - T
    lib.csahca_compress_pair_norm_rope(Xa, Za, ga, sep_a, n_a, m_a, e0a, ibs_a, obs_a, Xb, Zb, gb, sep_b,
                                       n_b, m_b, e0b, ibs_b, obs_b, B, c, d, eps, theta, dt)
    if "a" in sides:
        lib.csahca_norm_rope(xa_rows, ya_sep[:, 2:], ga, pos_a, B, T, 1, c, 1, d, eps, theta, 1, dt,
                             x_bstride=ibs_a, y_bstride=LW * c)
    if "b" in sides:
        lib.csahca_norm_rope(xb_rows, yb_sep[:, 2:], gb, pos_b, B, T, 1, c, 1, d, eps, theta, 1, dt,
                             x_bstride=ibs_b, y_bstride=LW * c)
    ra = (xa_rows, ya_pair[:, 2:]) if "a" in sides else (None, None)
    rb = (xb_rows, yb_pair[:, 2:]) if "b" in sides else (None, None)
    lib.csahca_compress_pair_norm_rope_rows(Xa, Za, ga, pair_a, n_a, m_a, e0a, ibs_a, obs_a, Xb, Zb, gb,
                                            pair_b, n_b, m_b, e0b, ibs_b, obs_b, B, c, d, eps, theta, dt,
                                            T, *ra, pos_a, ibs_a, LW * c, *rb, pos_b, ibs_b, LW * c)
    torch.cuda.synchronize()
    iv = torch.int16 if dt == BF16 else torch.int32
    assert torch.equal(pair_a.view(iv), sep_a.view(iv))
    assert torch.equal(pair_b.view(iv), sep_b.view(iv))
    assert torch.equal(ya_pair.view(iv), ya_sep.view(iv))
    assert torch.equal(yb_pair.view(iv), yb_sep.view(iv))
    assert bool((ya_pair[:, :2] == 3).all()) and bool((ya_pair[:, 2 + T:] == 3).all())
