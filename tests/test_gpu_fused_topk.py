"""The decode top-k selection from chunk lists (lightning_index_topk, decode, c_I = 128:
every scoring workgroup lists its chunk's best entries, the selection kernel selects from
their union): bit-exact against oracle.topk of the GPU's own scores, on score
distributions chosen to drive each of its paths, which the workspace's last words record:

- random keys: every chunk's list holds its share of the top k (the lists path);
- a few far outliers over a tight cluster: the chunk cut needs a second histogram pass;
- the best entries clustered inside one chunk, or scores rising with the index: a chunk
  holds more of the top k than it lists, so the selection goes through the group maxima;
- heavy ties (few distinct key rows), zero head weights, no usable entry, k >= V;
- one workspace reused across calls of different shapes.
Scores are also checked against the oracle at 1e-3 relative.
"""
import math

import numpy as np
import pytest
import torch

import compressed_attention_compress_amd as lib
import oracle
from synthgen.configs import FP8, MXFP4
from synthgen.host import encode
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    H.require_gpu()


LISTS, GROUPS, ALL = 1, 2, 3  # how a query's selection went (the workspace's last words)


def run(qI, w, KI, q_pos, m, k, ws=None):
    """qI [B,1,n_ih,128] fp8 codes, w [B,1,n_ih] f32, KI [B,N_c,128] fp8 codes (host).
    Returns the top-k list, its scores, all scores and each query's selection path."""
    B, Tq, n_ih, c_I = qI.shape
    N_c = KI.shape[1]
    ws_bytes = lib.lightning_index_topk_workspace_size(B, Tq, n_ih, N_c, k)
    if ws is None:
        ws = torch.full((ws_bytes,), 0xA5, dtype=torch.uint8, device=H.DEV)  # no initial contents needed
    assert ws.numel() >= ws_bytes
    idx = torch.full((B, Tq, k), -7, dtype=torch.int32, device=H.DEV)
    sc = torch.full((B, Tq, k), float("nan"), dtype=torch.float32, device=H.DEV)
    alls = torch.full((B, Tq, N_c), float("nan"), dtype=torch.float32, device=H.DEV)
    lib.lightning_index_topk(H.to_dev(qI), H.to_dev(w), H.to_dev(KI), FP8, H.to_dev(q_pos), m, B, Tq,
                             n_ih, c_I, N_c, k, idx, sc, alls, ws, ws.numel())
    torch.cuda.synchronize()
    nq = B * Tq
    path_off = ws_bytes - (-(-nq * 4 // 256) * 256)
    path = ws[path_off:path_off + 4 * nq].view(torch.int32).cpu().numpy()
    return idx.cpu().numpy(), sc.cpu().numpy(), alls.cpu().numpy(), path


def check(qI, w, KI, q_pos, m, k, got, label, path=None):
    idx, sc, alls, paths = got
    print(f"{label}: selection paths {paths.tolist()}", flush=True)
    if path is not None:
        assert np.array_equal(paths, np.broadcast_to(path, paths.shape)), f"{label}: paths {paths}"
    q = oracle.decode(qI, FP8)
    K = oracle.decode(KI, FP8)
    B = qI.shape[0]
    for b in range(B):
        V = oracle.visible(int(q_pos[b]), m, K.shape[1])
        g = alls[b, 0, :V].astype(np.float64)
        if V:
            ref = oracle.index_scores(q[b, 0], w[b, 0], K[b], V)
            rms = math.sqrt(float(np.mean(ref * ref)))
            assert np.all(np.abs(g - ref) <= 1e-3 * np.abs(ref) + 1e-6 * rms), f"{label}: scores b={b}"
        want = oracle.topk(g, k)
        assert np.array_equal(idx[b, 0], want), f"{label}: top-k b={b}"
        keff = min(k, V)
        assert np.array_equal(sc[b, 0, :keff], alls[b, 0, want[:keff]]), f"{label}: top-k scores b={b}"
        assert np.all(np.isneginf(sc[b, 0, keff:])), f"{label}: padding b={b}"


def draw(seed, B, N_c, n_ih=64):
    rng = np.random.default_rng(seed)
    qI = rng.standard_normal((B, 1, n_ih, 128), dtype=np.float32)
    w = rng.random((B, 1, n_ih), dtype=np.float32)
    KI = rng.standard_normal((B, N_c, 128), dtype=np.float32)
    return rng, qI, w, KI


def aligned(qI, w):
    """Per sequence, the head-weighted query direction, with norm sqrt(128)."""
    u = (w[:, 0, :, None] * qI[:, 0]).sum(1)
    return u * (np.sqrt(128) / np.linalg.norm(u, axis=1, keepdims=True))


def decode_pos(B, N_c, m=4):
    return np.full(B, N_c * m - 1, dtype=np.int32)


@pytest.mark.parametrize("B,N_c,k", [(4, 262144 // 8, 1024), (32, 4096, 512), (3, 20000, 1024), (2, 1000, 64),
                                     (1, 70000, 1024)])
def test_random_keys(B, N_c, k):
    print(f"[fused random B={B} N_c={N_c} k={k}]", flush=True)
    _, qI, w, KI = draw(100 + B, B, N_c)
    qc, kc = encode(qI, FP8), encode(KI, FP8)
    q_pos = decode_pos(B, N_c)
    check(qc, w, kc, q_pos, 4, k, run(qc, w, kc, q_pos, 4, k), "random", path=LISTS)


def test_outliers_over_a_tight_cluster():
    """Every key is the query direction plus a little noise in a few dims: the scores
    bunch together, and a handful of far outliers widen the first histogram's range, so
    the cut needs a second pass (and possibly a third) inside one bin."""
    B, N_c, k = 2, 16384, 512
    rng, qI, w, KI = draw(7, B, N_c)
    u = aligned(qI, w)
    KI = np.repeat(u[:, None, :], N_c, axis=1)
    KI[:, :, :8] += rng.standard_normal((B, N_c, 8), dtype=np.float32) * 0.5
    out = rng.choice(N_c, size=(B, 6), replace=False)
    for b in range(B):
        KI[b, out[b]] = 6.0 * u[b]
    qc, kc = encode(qI, FP8), encode(KI, FP8)
    q_pos = decode_pos(B, N_c)
    check(qc, w, kc, q_pos, 4, k, run(qc, w, kc, q_pos, 4, k), "cluster")


@pytest.mark.parametrize("where", ["one_chunk", "rising"])
def test_best_entries_clustered(where):
    """More of the top k inside one chunk than a chunk lists (or scores rising with the
    index, all of the top k in the last chunks): the exact selection from all scores."""
    B, N_c, k = 2, 32768, 512
    rng, qI, w, KI = draw(11, B, N_c)
    u = aligned(qI, w)
    if where == "one_chunk":
        for b in range(B):
            lo = 5000 + 3000 * b
            KI[b, lo:lo + 400] = u[b] + 0.1 * rng.standard_normal((400, 128), dtype=np.float32)
    else:
        # scale of the query direction rising with the index (fp8 keeps about 16 levels per
        # octave, so long runs tie; ties go to the lower index)
        lvl = np.linspace(0.05, 4.0, N_c, dtype=np.float32)
        KI = lvl[None, :, None] * u[:, None, :]
    qc, kc = encode(qI, FP8), encode(KI, FP8)
    q_pos = decode_pos(B, N_c)
    check(qc, w, kc, q_pos, 4, k, run(qc, w, kc, q_pos, 4, k), where, path=GROUPS)


def test_heavy_ties_and_zero_weights():
    B, N_c, k = 2, 12000, 1024
    rng, qI, w, KI = draw(13, B, N_c)
    rows = rng.standard_normal((B, 5, 128), dtype=np.float32)
    KI = rows[np.arange(B)[:, None], rng.integers(0, 5, size=(B, N_c))]   # five distinct keys
    qc, kc = encode(qI, FP8), encode(KI, FP8)
    q_pos = decode_pos(B, N_c)
    check(qc, w, kc, q_pos, 4, k, run(qc, w, kc, q_pos, 4, k), "ties")
    w0 = np.zeros_like(w)
    got = run(qc, w0, kc, q_pos, 4, k)
    check(qc, w0, kc, q_pos, 4, k, got, "zero weights", path=GROUPS)  # all scores equal
    assert np.array_equal(got[0][:, 0], np.broadcast_to(np.arange(k), (B, k)))


def test_visible_counts_at_the_edges():
    """Per sequence: no usable entry, fewer usable entries than k (all selected), exactly
    k, and a chunk boundary inside the usable range."""
    B, N_c, k = 4, 6000, 512
    _, qI, w, KI = draw(17, B, N_c)
    qc, kc = encode(qI, FP8), encode(KI, FP8)
    q_pos = np.array([2, 4 * 300 + 1, 4 * 512 - 1, 4 * 2049 + 3], dtype=np.int32)  # V = 0, 300, 512, 2050
    check(qc, w, kc, q_pos, 4, k, run(qc, w, kc, q_pos, 4, k), "edges", path=np.array([ALL, ALL, ALL, LISTS]))


def test_one_workspace_across_shapes():
    """One workspace (never cleared) serves calls of different shapes in turn."""
    shapes = [(4, 30000, 1024), (2, 1000, 64), (8, 8192, 512), (4, 30000, 1024)]
    need = max(lib.lightning_index_topk_workspace_size(B, 1, 64, N_c, k) for B, N_c, k in shapes)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device=H.DEV)  # stale contents
    for i, (B, N_c, k) in enumerate(shapes):
        _, qI, w, KI = draw(200 + i, B, N_c)
        qc, kc = encode(qI, FP8), encode(KI, FP8)
        q_pos = decode_pos(B, N_c)
        check(qc, w, kc, q_pos, 4, k, run(qc, w, kc, q_pos, 4, k, ws=ws), f"shape {i}", path=LISTS)


def test_split_calls_use_the_lists_too():
    """lightning_index_score + lightning_index_select at decode: the scoring launch writes
    and marks the chunk lists, the selection takes them (path LISTS) and the result is the
    fused call's, bit for bit.  A second selection over the same scoring output finds the
    mark consumed and selects through the group maxima: same result again."""
    B, N_c, k = 4, 30000, 1024
    _, qI, w, KI = draw(300, B, N_c)
    qc, kc = encode(qI, FP8), encode(KI, FP8)
    q_pos = decode_pos(B, N_c)
    fused = run(qc, w, kc, q_pos, 4, k)
    ws_bytes = lib.lightning_index_topk_workspace_size(B, 1, 64, N_c, k)
    ws = torch.full((ws_bytes,), 0xA5, dtype=torch.uint8, device=H.DEV)
    scores = torch.empty((B, 1, N_c), dtype=torch.float32, device=H.DEV)
    dq, dw, dk, dp = H.to_dev(qc), H.to_dev(w), H.to_dev(kc), H.to_dev(q_pos)
    lib.lightning_index_score(dq, dw, dk, FP8, dp, 4, B, 1, 64, 128, N_c, k, scores, ws, ws_bytes)
    path_off = ws_bytes - (-(-B * 4 // 256) * 256)
    for want_path in (LISTS, GROUPS):
        idx = torch.full((B, 1, k), -7, dtype=torch.int32, device=H.DEV)
        sc = torch.full((B, 1, k), float("nan"), dtype=torch.float32, device=H.DEV)
        lib.lightning_index_select(scores, dp, 4, B, 1, N_c, k, idx, sc, ws, ws_bytes)
        torch.cuda.synchronize()
        paths = ws[path_off:path_off + 4 * B].view(torch.int32).cpu().numpy()
        print(f"split selection paths {paths.tolist()}", flush=True)
        assert np.all(paths == want_path)
        assert np.array_equal(idx.cpu().numpy(), fused[0])
        assert np.array_equal(sc.cpu().numpy(), fused[1])
        assert np.array_equal(scores.cpu().numpy(), fused[2])


def test_fused_call_in_a_graph_replays():
    """lightning_index_topk captured in a HIP graph (the scoring launch marks each query's
    lists ready, the selection takes them): replayed three times with new keys copied in
    between, each replay equal to the eager call on the same inputs, bit for bit."""
    B, N_c, k = 4, 30000, 1024
    rng, qI, w, KI = draw(400, B, N_c)
    qc, kc = encode(qI, FP8), encode(KI, FP8)
    q_pos = decode_pos(B, N_c)
    dq, dw, dk, dp = H.to_dev(qc), H.to_dev(w), H.to_dev(kc), H.to_dev(q_pos)
    ws_bytes = lib.lightning_index_topk_workspace_size(B, 1, 64, N_c, k)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=H.DEV)
    idx = torch.empty((B, 1, k), dtype=torch.int32, device=H.DEV)
    sc = torch.empty((B, 1, k), dtype=torch.float32, device=H.DEV)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        lib.lightning_index_topk(dq, dw, dk, FP8, dp, 4, B, 1, 64, 128, N_c, k, idx, sc, None, ws, ws_bytes,
                                 stream=s)
    path_off = ws_bytes - (-(-B * 4 // 256) * 256)
    for rep in range(3):
        KI2 = rng.standard_normal((B, N_c, 128), dtype=np.float32)
        dk.copy_(H.to_dev(encode(KI2, FP8)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_i, got_s = idx.clone(), sc.clone()
        paths = ws[path_off:path_off + 4 * B].view(torch.int32).cpu().numpy()
        assert np.all(paths == LISTS), (rep, paths)
        lib.lightning_index_topk(dq, dw, dk, FP8, dp, 4, B, 1, 64, 128, N_c, k, idx, sc, None, ws, ws_bytes)
        torch.cuda.synchronize()
        assert torch.equal(got_i, idx) and torch.equal(got_s, sc), rep
