"""lightning_index_topk_csa_compress: the indexer with a CSA pooling enqueued beside it.
Its results are those of lightning_index_topk followed by csa_compress on the same
inputs, bit for bit: the top-k list, its scores, all scores and every pooled entry (and
nothing written past the pooled entries).  Cases:

- decode with chunk lists and a bfloat16 block (the pooling runs in extra workgroups of
  the selection launch), one block and many blocks, batch strides wider than the rows;
- a pooling that emits nothing (fewer tokens than a block): the output is untouched;
- float32 entries, and a prefill shape (no chunk lists): the pooling's own launch.
"""
import numpy as np
import pytest
import torch

import compressed_attention_compress_amd as lib
from synthgen.configs import BF16, F32, FP8
from synthgen.host import encode
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    H.require_gpu()


def inputs(seed, B, Tq, N_c, n_tok, c, dtype, n_ih=64, pad=0):
    rng = np.random.default_rng(seed)
    qc = encode(rng.standard_normal((B, Tq, n_ih, 128), dtype=np.float32), FP8)
    w = rng.random((B, Tq, n_ih), dtype=np.float32)
    kc = encode(rng.standard_normal((B, N_c, 128), dtype=np.float32), FP8)
    # the last query sits at the end of the cache (decode), earlier ones a token apart
    q_pos = np.array([[4 * N_c - Tq + t for t in range(Tq)] for _ in range(B)], dtype=np.int32)
    rows = n_tok + pad
    X = rng.standard_normal((B, rows, c), dtype=np.float32)
    Z = rng.standard_normal((B, rows, c), dtype=np.float32) * 2.0
    if dtype == BF16:
        X, Z = encode(X, BF16), encode(Z, BF16)
    return qc, w, kc, q_pos, X, Z


def call(fused, qc, w, kc, q_pos, k, X, Z, n_tok, m, dtype, out_rows):
    B, Tq, n_ih, c_I = qc.shape
    N_c = kc.shape[1]
    c = X.shape[2]
    ws_bytes = lib.lightning_index_topk_workspace_size(B, Tq, n_ih, N_c, k)
    ws = torch.full((ws_bytes,), 0xA5, dtype=torch.uint8, device=H.DEV)
    idx = torch.full((B, Tq, k), -7, dtype=torch.int32, device=H.DEV)
    sc = torch.full((B, Tq, k), float("nan"), dtype=torch.float32, device=H.DEV)
    alls = torch.full((B, Tq, N_c), float("nan"), dtype=torch.float32, device=H.DEV)
    out = H.empty((B, out_rows, c), dtype)
    out.view(torch.uint8).fill_(0x5A)  # sentinel: rows past the pooled entries stay so
    dq, dw, dk, dp, dX, dZ = (H.to_dev(a) for a in (qc, w, kc, q_pos, X, Z))
    in_bs, out_bs = X.shape[1] * c, out_rows * c
    if fused:
        lib.lightning_index_topk_csa_compress(dq, dw, dk, FP8, dp, m, B, Tq, n_ih, c_I, N_c, k, idx, sc, alls,
                                              ws, ws_bytes, dX, dZ, out, n_tok, c, dtype, in_bs, out_bs)
    else:
        lib.lightning_index_topk(dq, dw, dk, FP8, dp, m, B, Tq, n_ih, c_I, N_c, k, idx, sc, alls, ws, ws_bytes)
        lib.csa_compress(dX, dZ, None, out, B, n_tok, c, m, dtype, in_bs, out_bs)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (idx, sc, alls)] + [out.view(torch.uint8).cpu().numpy()]


@pytest.mark.parametrize("B,Tq,N_c,k,n_tok,c,dtype,pad,out_rows", [
    (4, 1, 32768, 1024, 4, 512, BF16, 0, 1),        # a decode step's one new block
    (2, 1, 8192, 512, 4 * 37 + 3, 512, BF16, 5, 40),  # many blocks, a ragged tail, wide strides
    (3, 1, 6000, 512, 4, 128, BF16, 0, 2),          # a narrow entry, one spare output row
    (2, 1, 4096, 512, 3, 512, BF16, 0, 1),          # fewer tokens than a block: nothing pooled
    (2, 1, 8192, 512, 8, 512, F32, 0, 2),           # float32 entries: the pooling's own launch
    (2, 3, 4096, 512, 8, 512, BF16, 0, 2),          # several queries: no chunk lists
])
def test_matches_the_two_calls(B, Tq, N_c, k, n_tok, c, dtype, pad, out_rows):
    print(f"[index+pool B={B} Tq={Tq} N_c={N_c} k={k} n={n_tok} c={c} dtype={dtype}]", flush=True)
    args = inputs(500 + B * Tq + n_tok, B, Tq, N_c, n_tok, c, dtype, pad=pad)
    a = call(True, *args[:4], k, *args[4:], n_tok, 4, dtype, out_rows)
    b = call(False, *args[:4], k, *args[4:], n_tok, 4, dtype, out_rows)
    for name, x, y in zip(("top-k", "top-k scores", "all scores", "entries"), a, b):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), name
    N = n_tok // 4
    assert np.all(a[3].reshape(B, out_rows, -1)[:, N:] == 0x5A)  # nothing past the entries
    assert N == 0 or not np.all(a[3].reshape(B, out_rows, -1)[:, :N] == 0x5A)


def call_nr(fused, qc, w, kc, q_pos, k, X, Z, n_tok, m, out_rows, gamma, entry0, T, with_rows):
    """The same with the norm and the step's window rows (the last T tokens of X, at
    positions row_pos[b] + t, into a window buffer of L rows)."""
    B, Tq, n_ih, c_I = qc.shape
    N_c = kc.shape[1]
    c = X.shape[2]
    L = T + 3
    ws_bytes = lib.lightning_index_topk_workspace_size(B, Tq, n_ih, N_c, k)
    ws = torch.full((ws_bytes,), 0xA5, dtype=torch.uint8, device=H.DEV)
    idx = torch.full((B, Tq, k), -7, dtype=torch.int32, device=H.DEV)
    sc = torch.full((B, Tq, k), float("nan"), dtype=torch.float32, device=H.DEV)
    alls = torch.full((B, Tq, N_c), float("nan"), dtype=torch.float32, device=H.DEV)
    out = H.empty((B, out_rows, c), BF16)
    out.view(torch.uint8).fill_(0x5A)
    win = H.empty((B, L, c), BF16)
    win.view(torch.uint8).fill_(0x3C)
    dq, dw, dk, dp, dX, dZ = (H.to_dev(a) for a in (qc, w, kc, q_pos, X, Z))
    g = None if gamma is None else H.to_dev(gamma)
    rpos = torch.arange(B, dtype=torch.int32, device=H.DEV) * 1000 + 77
    in_bs, out_bs = X.shape[1] * c, out_rows * c
    rx, ry = (dX[:, n_tok - T:], win[:, L - T:]) if with_rows else (None, None)
    D, EPS, THETA = 64, 1e-6, 10000.0
    if fused:
        lib.lightning_index_topk_csa_compress_norm_rope_rows(
            dq, dw, dk, FP8, dp, m, B, Tq, n_ih, c_I, N_c, k, idx, sc, alls, ws, ws_bytes, dX, dZ, g, out, n_tok, c,
            entry0, D, EPS, THETA, BF16, in_bs, out_bs, T, rx, ry, rpos, in_bs, L * c)
    else:
        lib.lightning_index_topk(dq, dw, dk, FP8, dp, m, B, Tq, n_ih, c_I, N_c, k, idx, sc, alls, ws, ws_bytes)
        lib.csahca_compress_pair_norm_rope_rows(dX, dZ, g, out, n_tok, m, entry0, in_bs, out_bs,
                                                None, None, None, None, 0, 128, 0, c, c,
                                                B, c, D, EPS, THETA, BF16, T, rx, ry, rpos, in_bs, L * c,
                                                None, None, None, c, c)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (idx, sc, alls)] + [out.view(torch.uint8).cpu().numpy(),
                                                          win.view(torch.uint8).cpu().numpy()]


@pytest.mark.parametrize("B,Tq,N_c,k,n_tok,out_rows,entry0,T,rows,unit", [
    (4, 1, 32768, 1024, 4, 1, 262143, 1, True, False),   # a decode step: one block and its row
    (2, 1, 8192, 512, 4 * 9 + 2, 10, 5, 2, True, True),  # several blocks, two rows, unit gain
    (2, 1, 8192, 512, 4, 1, 100, 1, False, False),       # the pooling alone
    (3, 1, 6000, 512, 3, 1, 0, 1, True, False),          # the row alone: no block completed
    (2, 3, 4096, 512, 8, 2, 7, 3, True, False),          # several queries: launches of their own
])
def test_norm_rope_rows_match_the_calls(B, Tq, N_c, k, n_tok, out_rows, entry0, T, rows, unit):
    print(f"[index+pool+norm B={B} Tq={Tq} N_c={N_c} n={n_tok} T={T} rows={rows}]", flush=True)
    c = 512
    args = inputs(700 + B * Tq + n_tok, B, Tq, N_c, n_tok, c, BF16)
    gamma = None if unit else (np.random.default_rng(5).random(c, dtype=np.float32) + 0.5)
    a = call_nr(True, *args[:4], k, *args[4:], n_tok, 4, out_rows, gamma, entry0, T, rows)
    b = call_nr(False, *args[:4], k, *args[4:], n_tok, 4, out_rows, gamma, entry0, T, rows)
    for name, x, y in zip(("top-k", "top-k scores", "all scores", "entries", "window rows"), a, b):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), name
    N = n_tok // 4
    assert np.all(a[3].reshape(B, out_rows, -1)[:, N:] == 0x5A)
    win = a[4].reshape(B, T + 3, -1)
    assert np.all(win[:, :3] == 0x3C)  # rows before the step's are untouched
    assert np.all(win[:, 3:] == 0x3C) != rows
