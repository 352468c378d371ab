"""The top-k selection of a prefill chunk (lightning_index_topk with Tq > 1: no chunk lists,
the selection goes through the group maxima): bit-exact against oracle.topk of the GPU's
own scores, for every query of the chunk, on score distributions and shapes chosen to
drive each selection kernel and path:

- one wave per query (k <= 512, at most 5120 groups; 16, 48 or 80 group maxima per lane):
  random keys (the candidates fit in LDS); scores rising with the index (every entry of
  the selected groups is a candidate, more than LDS holds, so every count re-reads the
  scores); heavy ties; zero head weights; queries with no usable entry, fewer than k,
  and no more groups than k (every group taken);
- one workgroup per query with 8 keys per thread (k <= 512, up to 8192 groups) and with 16
  (k > 512 or more groups).
Scores of sampled queries are also checked against the oracle at 1e-3 relative.
"""
import math

import numpy as np
import pytest
import torch

import compressed_attention_compress_amd as lib
import oracle
from synthgen.configs import FP8
from synthgen.host import encode
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    H.require_gpu()


def run(qc, w, kc, q_pos, m, k):
    B, Tq, n_ih, c_I = qc.shape
    N_c = kc.shape[1]
    ws_bytes = lib.lightning_index_topk_workspace_size(B, Tq, n_ih, N_c, k)
    ws = torch.full((ws_bytes,), 0xA5, dtype=torch.uint8, device=H.DEV)
    idx = torch.full((B, Tq, k), -7, dtype=torch.int32, device=H.DEV)
    sc = torch.full((B, Tq, k), float("nan"), dtype=torch.float32, device=H.DEV)
    alls = torch.full((B, Tq, N_c), float("nan"), dtype=torch.float32, device=H.DEV)
    lib.lightning_index_topk(H.to_dev(qc), H.to_dev(w), H.to_dev(kc), FP8, H.to_dev(q_pos), m, B, Tq,
                             n_ih, c_I, N_c, k, idx, sc, alls, ws, ws.numel())
    torch.cuda.synchronize()
    return idx.cpu().numpy(), sc.cpu().numpy(), alls.cpu().numpy()


def check(qc, w, kc, q_pos, m, k, got, label, n_score_checks=2):
    idx, sc, alls = got
    B, Tq = qc.shape[:2]
    N_c = kc.shape[1]
    q = oracle.decode(qc, FP8)
    K = oracle.decode(kc, FP8)
    rng = np.random.default_rng(0)
    for b in range(B):
        for t in rng.choice(Tq, size=min(n_score_checks, Tq), replace=False):
            V = oracle.visible(int(q_pos[b]) + int(t), m, N_c)
            if V:
                ref = oracle.index_scores(q[b, t], w[b, t], K[b], V)
                rms = math.sqrt(float(np.mean(ref * ref)))
                g = alls[b, t, :V].astype(np.float64)
                assert np.all(np.abs(g - ref) <= 1e-3 * np.abs(ref) + 1e-6 * rms), f"{label}: scores {b},{t}"
        for t in range(Tq):
            V = oracle.visible(int(q_pos[b]) + t, m, N_c)
            want = oracle.topk(alls[b, t, :V].astype(np.float64), k)
            assert np.array_equal(idx[b, t], want), f"{label}: top-k b={b} t={t} V={V}"
            keff = min(k, V)
            assert np.array_equal(sc[b, t, :keff], alls[b, t, want[:keff]]), f"{label}: scores b={b} t={t}"
            assert np.all(np.isneginf(sc[b, t, keff:])), f"{label}: padding b={b} t={t}"


def draw(seed, B, Tq, N_c, n_ih=64):
    rng = np.random.default_rng(seed)
    qI = rng.standard_normal((B, Tq, n_ih, 128), dtype=np.float32)
    w = rng.random((B, Tq, n_ih), dtype=np.float32)
    KI = rng.standard_normal((B, N_c, 128), dtype=np.float32)
    return rng, qI, w, KI


def chunk_end_pos(B, Tq, N_c, m=4):
    """Chunk positions whose last query sees every entry."""
    return np.full(B, N_c * m - Tq, dtype=np.int32)


@pytest.mark.parametrize("B,Tq,N_c,k", [
    (2, 24, 12000, 512),     # wave kernel, 16 maxima per lane
    (1, 40, 67584, 512),     # wave kernel, 80 per lane (the 256K context + 8K chunk's shape)
    (2, 16, 30000, 256),     # 48 per lane
    (1, 16, 100000, 512),    # 6250 groups: workgroup kernel, 8 keys per thread
    (1, 12, 40000, 1024),    # k > 512: workgroup kernel, 16 keys per thread
    (1, 8, 200000, 512),     # 12500 groups: 16 keys per thread
])
def test_random_keys(B, Tq, N_c, k):
    print(f"[prefill random B={B} Tq={Tq} N_c={N_c} k={k}]", flush=True)
    _, qI, w, KI = draw(500 + Tq, B, Tq, N_c)
    qc, kc = encode(qI, FP8), encode(KI, FP8)
    q_pos = chunk_end_pos(B, Tq, N_c)
    check(qc, w, kc, q_pos, 4, k, run(qc, w, kc, q_pos, 4, k), "random")


@pytest.mark.parametrize("N_c,k", [(32768, 512), (12000, 256), (70000, 512), (100000, 512), (40000, 1024)])
def test_scores_rising_with_the_index(N_c, k):
    """Every entry of the selected groups scores at least the k-th group maximum: more
    candidates than LDS holds (one wave per query), and long runs of ties from the fp8
    levels (ties go to the lower index)."""
    print(f"[prefill rising N_c={N_c} k={k}]", flush=True)
    B, Tq = 1, 8
    rng, qI, w, _ = draw(600, B, Tq, N_c)
    u = (w[:, 0, :, None] * qI[:, 0]).sum(1)
    u *= np.sqrt(128) / np.linalg.norm(u, axis=1, keepdims=True)
    # every query of the chunk shares the first query's weighted direction
    qI[:] = qI[:, :1]
    w[:] = w[:, :1]
    lvl = np.linspace(0.05, 4.0, N_c, dtype=np.float32)
    KI = lvl[None, :, None] * u[:, None, :]
    qc, kc = encode(qI, FP8), encode(KI, FP8)
    q_pos = chunk_end_pos(B, Tq, N_c)
    check(qc, w, kc, q_pos, 4, k, run(qc, w, kc, q_pos, 4, k), "rising")


@pytest.mark.parametrize("N_c,k", [(30000, 512), (12000, 1024)])
def test_heavy_ties_and_zero_weights(N_c, k):
    print(f"[prefill ties N_c={N_c} k={k}]", flush=True)
    B, Tq = 2, 8
    rng, qI, w, _ = draw(700, B, Tq, N_c)
    rows = rng.standard_normal((B, 5, 128), dtype=np.float32)
    KI = rows[np.arange(B)[:, None], rng.integers(0, 5, size=(B, N_c))]   # five distinct keys
    qc, kc = encode(qI, FP8), encode(KI, FP8)
    q_pos = chunk_end_pos(B, Tq, N_c)
    check(qc, w, kc, q_pos, 4, k, run(qc, w, kc, q_pos, 4, k), "ties")
    w0 = np.zeros_like(w)
    got = run(qc, w0, kc, q_pos, 4, k)
    check(qc, w0, kc, q_pos, 4, k, got, "zero weights")
    assert np.array_equal(got[0], np.broadcast_to(np.arange(k), (B, Tq, k)))


def test_chunk_from_the_start():
    """A chunk from position 0: its queries see no entry, fewer than k, exactly k, no more
    groups than k (every group taken), then more."""
    B, Tq, N_c, k, m = 1, 192, 48, 16, 4   # V = 0 .. 48 over the chunk
    _, qI, w, KI = draw(800, B, Tq, N_c)
    qc, kc = encode(qI, FP8), encode(KI, FP8)
    q_pos = np.zeros(B, dtype=np.int32)
    check(qc, w, kc, q_pos, m, k, run(qc, w, kc, q_pos, m, k), "from 0", n_score_checks=4)
    # and a longer context seen from a chunk in its middle: V from 4000 to 4000 + Tq/4
    B, Tq, N_c, k = 2, 64, 9000, 512
    _, qI, w, KI = draw(801, B, Tq, N_c)
    qc, kc = encode(qI, FP8), encode(KI, FP8)
    q_pos = np.array([4 * 4000, 4 * 8000 + 2], dtype=np.int32)
    check(qc, w, kc, q_pos, m, k, run(qc, w, kc, q_pos, m, k), "middle")
