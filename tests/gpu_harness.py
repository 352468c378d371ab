"""Helpers shared by the GPU tests: upload seeded inputs, call the library through the
C ABI binding, download results.  Nothing here computes any part of the method."""
import math

import numpy as np
import torch

import compressed_attention_compress_amd as lib
from synthgen.configs import BF16, F32, FP8, MXFP4

DEV = "cuda"


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    lib.load()


def to_dev(arr):
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).to(DEV)
    if arr.dtype == np.uint8:
        return torch.from_numpy(arr).to(DEV)
    if arr.dtype == np.float32:
        return torch.from_numpy(arr).to(DEV)
    if arr.dtype == np.int32:
        return torch.from_numpy(arr).to(DEV)
    raise TypeError(arr.dtype)


def to_host_codes(t, dtype):
    a = t.detach().cpu().numpy()
    if dtype == BF16:
        return a.view(np.uint16)
    return a


def empty(shape, dtype):
    tdt = {F32: torch.float32, BF16: torch.int16, FP8: torch.uint8}[dtype]
    return torch.empty(shape, dtype=tdt, device=DEV)


def run_pool(X, Z, m, dtype, P=None, fn=lib.csa_compress):
    """X, Z device [B, n, c] -> device [B, n//m, c]."""
    B, n, c = X.shape
    out = empty((B, n // m, c), dtype)
    fn(X, Z, P, out, B, n, c, m, dtype, n * c, (n // m) * c)
    return out


def run_pool_overlap(Xa, Za, Xb, Zb, m, prev, dtype, P=None):
    """Overlapped two-stream pooling: device [B, n, c] x 4 -> device [B, n//m - prev, c]."""
    B, n, c = Xa.shape
    N = max(n // m - prev, 0)
    out = empty((B, N, c), dtype)
    lib.csa_compress_overlap(Xa, Za, Xb, Zb, P, out, B, n, c, m, prev, dtype, n * c, max(N, 1) * c)
    return out


def key_buffer(prob):
    """The indexer-key argument: the key codes, or for MX FP4 all packed rows followed by
    all scales in one device buffer."""
    KI = prob["KI"]
    if "KI_scales" not in prob:
        return KI if torch.is_tensor(KI) else to_dev(KI)
    rows, sc = KI, prob["KI_scales"]
    if not torch.is_tensor(rows):
        rows, sc = to_dev(rows), to_dev(sc)
    return torch.cat([rows.reshape(-1), sc.reshape(-1)])


def run_index(qI, w, KI, q_pos, m, k, idx_dtype, split=False, N_c=None):
    B, Tq, n_ih, c_I = qI.shape
    N_c = KI.shape[1] if N_c is None else N_c
    ws_bytes = lib.lightning_index_topk_workspace_size(B, Tq, n_ih, N_c, k)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    idx = torch.empty((B, Tq, k), dtype=torch.int32, device=DEV)
    sc = torch.empty((B, Tq, k), dtype=torch.float32, device=DEV)
    alls = torch.full((B, Tq, N_c), float("nan"), dtype=torch.float32, device=DEV)
    if split:
        lib.lightning_index_score(qI, w, KI, idx_dtype, q_pos, m, B, Tq, n_ih, c_I, N_c, k, alls,
                                  ws, ws_bytes)
        lib.lightning_index_select(alls, q_pos, m, B, Tq, N_c, k, idx, sc, ws, ws_bytes)
    else:
        lib.lightning_index_topk(qI, w, KI, idx_dtype, q_pos, m, B, Tq, n_ih, c_I, N_c, k, idx,
                                 sc, alls, ws, ws_bytes)
    return idx, sc, alls


def run_csa_attend(Q, C, topk, win, win_pos, q_pos, W, dtype, scale=None, lse=True, sink=None,
                   nrq=None):
    """nrq: (q_gamma device or None, d_rope, eps, theta) to normalise and rotate the queries
    inside the call (csa_attend_ex), else None."""
    B, Tq, n_h, c = Q.shape
    N_c = C.shape[1]
    k = topk.shape[2]
    L = win.shape[1]
    scale = 1.0 / math.sqrt(c) if scale is None else scale
    ws_bytes = lib.csa_attend_workspace_size(B, Tq, n_h, c, k, W)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=DEV)
    out = empty((B, Tq, n_h, c), dtype)
    l = torch.empty((B, Tq, n_h), dtype=torch.float32, device=DEV) if lse else None
    if nrq is not None:
        lib.csa_attend_ex(Q, C, topk, win, win_pos, q_pos, B, Tq, n_h, c, N_c, k, L, W, scale, sink,
                          nrq[0], 1, *nrq[1:], dtype, out, l, ws, ws_bytes)
    elif sink is None:
        lib.csa_attend(Q, C, topk, win, win_pos, q_pos, B, Tq, n_h, c, N_c, k, L, W, scale, dtype,
                       out, l, ws, ws_bytes)
    else:
        lib.csa_attend_sink(Q, C, topk, win, win_pos, q_pos, B, Tq, n_h, c, N_c, k, L, W, scale, sink,
                            dtype, out, l, ws, ws_bytes)
    return out, l


def run_hca_attend(Q, C, win, win_pos, q_pos, m, W, dtype, scale=None, lse=True, sink=None,
                   nrq=None):
    B, Tq, n_h, c = Q.shape
    N_h = C.shape[1]
    L = win.shape[1]
    scale = 1.0 / math.sqrt(c) if scale is None else scale
    ws_bytes = lib.hca_attend_workspace_size(B, Tq, n_h, c, N_h, W)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=DEV)
    out = empty((B, Tq, n_h, c), dtype)
    l = torch.empty((B, Tq, n_h), dtype=torch.float32, device=DEV) if lse else None
    if nrq is not None:
        lib.hca_attend_ex(Q, C, win, win_pos, q_pos, m, B, Tq, n_h, c, N_h, L, W, scale, sink, nrq[0],
                          1, *nrq[1:], dtype, out, l, ws, ws_bytes)
    elif sink is None:
        lib.hca_attend(Q, C, win, win_pos, q_pos, m, B, Tq, n_h, c, N_h, L, W, scale, dtype, out, l,
                       ws, ws_bytes)
    else:
        lib.hca_attend_sink(Q, C, win, win_pos, q_pos, m, B, Tq, n_h, c, N_h, L, W, scale, sink, dtype,
                            out, l, ws, ws_bytes)
    return out, l
