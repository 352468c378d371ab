"""GPU parity: every stage of the HIP path against the CPU oracle on identical input bytes.

Stages are compared on the bytes the GPU consumed (staged comparison): attention uses
the GPU-written compressed cache and the GPU's top-k list, the top-k check uses the
GPU's own fp32 scores.  Tolerances:
  pooling    fp32: max |d| <= 1e-5; bf16: |d| <= one bf16 ulp of the fp64 value
             + 2^-16 * sum_j S_j |x_j| (fp32 rounding of the weighted sum)
  indexer    |d| <= 1e-3 * max(|ref|, RMS of the query's scores)
  top-k      bit-exact index lists (ascending, -1 padded) given the GPU scores
  attention  fp32: max |d| <= 1e-5; bf16: max |d| <= 2e-2 * RMS of the call's output, or
             for a query with few rows the bf16 rounding bound 2^-7 (|O| + sum_r p_r |v_r|)
"""
import math

import numpy as np
import pytest
import torch

import oracle
from synthgen.configs import BF16, CONFIGS, F32, FP8, MXFP4
from synthgen.host import make_problem
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    H.require_gpu()


def bf16_ulp(x):
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def check_pool(Xc, Zc, dtype, m, gpu_out, P=None):
    B = Xc.shape[0]
    got = oracle.decode(H.to_host_codes(gpu_out, dtype), dtype)
    for b in range(B):
        ref = oracle.pool(oracle.decode(Xc[b], dtype), oracle.decode(Zc[b], dtype), m, P)
        if dtype == F32:
            assert np.max(np.abs(got[b] - ref), initial=0.0) <= 1e-5
        else:
            # one bf16 ulp of the exact value, plus the fp32 rounding of the weighted sum
            # (its condition: sum_j S_j |x_j|), which matters only under cancellation
            cond = oracle.pool(np.abs(oracle.decode(Xc[b], dtype)), oracle.decode(Zc[b], dtype), m, P)
            bad = np.abs(got[b] - ref) > bf16_ulp(ref) + 2.0 ** -16 * cond
            assert not bad.any(), f"seq {b}: {bad.sum()} pooled values outside tolerance"


def decode_keys(prob):
    """Indexer queries and keys as fp64, from the bytes the GPU consumed."""
    cfg = prob["cfg"]
    if cfg.idx_dtype == MXFP4:
        return oracle.decode(prob["qI"], FP8), oracle.decode_mxfp4(prob["KI"], prob["KI_scales"])
    return oracle.decode(prob["qI"], cfg.idx_dtype), oracle.decode(prob["KI"], cfg.idx_dtype)


def check_index(prob, q_pos, k, idx, sc, alls):
    cfg = prob["cfg"]
    qI, KI = decode_keys(prob)
    w = prob["w"]
    idx = idx.cpu().numpy()
    sc = sc.cpu().numpy()
    alls = alls.cpu().numpy()
    B, Tq = qI.shape[:2]
    N_c = KI.shape[1]
    for b in range(B):
        for t in range(Tq):
            p = int(q_pos[b]) + t
            V = oracle.visible(p, cfg.m, N_c)
            ref = oracle.index_scores(qI[b, t], w[b, t], KI[b], V)
            g = alls[b, t, :V].astype(np.float64)
            if V:
                rms = math.sqrt(float(np.mean(ref * ref)))
                tol = 1e-3 * np.maximum(np.abs(ref), rms)
                assert np.all(np.abs(g - ref) <= tol), f"scores b={b} t={t}"
            want = oracle.topk(g, k)
            assert np.array_equal(idx[b, t], want), f"top-k b={b} t={t}"
            keff = min(k, V)
            assert np.array_equal(sc[b, t, :keff], alls[b, t, want[:keff]])
            assert np.all(np.isneginf(sc[b, t, keff:]))


def check_attend(Qc, dtype, rows_fn, gpu_out, gpu_lse, scale, sink=None):
    """rows_fn(b, t) -> fp64 row set for that query (from the GPU-consumed bytes)."""
    Q = oracle.decode(Qc, dtype)
    B, Tq = Q.shape[:2]
    got = oracle.decode(H.to_host_codes(gpu_out, dtype), dtype)
    lse = gpu_lse.cpu().numpy().astype(np.float64)
    ref = np.zeros_like(got)
    ref_abs = np.zeros_like(got)
    ref_lse = np.zeros(lse.shape)
    for b in range(B):
        for t in range(Tq):
            rows = rows_fn(b, t)
            ref[b, t], ref_lse[b, t] = oracle.attend(Q[b, t], rows, scale, sink)
            if dtype != F32 and rows.shape[0]:
                # the same softmax weights applied to |rows|: scale of the bf16 rounding of P
                wts = np.exp(scale * Q[b, t] @ rows.T - ref_lse[b, t][:, None])
                ref_abs[b, t] = wts @ np.abs(rows)
    err = np.abs(got - ref)
    if dtype == F32:
        assert err.max() <= 1e-5, f"attention max |d| = {err.max()}"
        assert np.max(np.abs(lse - ref_lse)) <= 1e-5
    else:
        rms = math.sqrt(float(np.mean(ref * ref)))
        # 2e-2 x output RMS; for queries with only a few rows (the first tokens of a
        # sequence) the bf16 rounding of P and O bounds the error by 2^-8 (|O| + sum p|v|)
        tol = np.maximum(2e-2 * rms, 2.0 ** -7 * (np.abs(ref) + ref_abs))
        assert np.all(err <= tol), f"attention max |d| = {err.max()}, RMS = {rms}"
        assert np.max(np.abs(lse - ref_lse)) <= 1e-3
    return float(err.max())


# ---------------------------------------------------------------------------------------
# cases
# ---------------------------------------------------------------------------------------
def small_cases():
    c1 = CONFIGS[1]
    c2 = CONFIGS[2]
    c3 = CONFIGS[3]
    c4 = CONFIGS[4]
    c5 = CONFIGS[5]
    return {
        "cfg1_tiny_fp32": c1,
        "hca_h64_ragged": c2.scaled(B=2, n=128 * 21 + 50, seed=21),
        "hca_h128": c5.scaled(kind="hca_decode", B=1, n=128 * 40 + 3, seed=22, plants=0),
        "csa_h64_k512": c3.scaled(B=2, n=4 * 900 + 2, seed=23),
        "csa_h128_k1024": c5.scaled(kind="csa_decode", B=1, n=4 * 2600 + 1, seed=24),
        "csa_k_ge_visible": c3.scaled(B=2, n=4 * 100, seed=25, plants=4),
        "prefill_small": c4.scaled(n=4096, Tq=200, seed=26),
        "prefill_from_zero": c4.scaled(n=0, Tq=40, seed=27, k=8),
        # an odd chunk: the last workgroup of two-query HCA prefill has one query only
        "prefill_odd_tq": c4.scaled(n=4096 + 5, Tq=41, seed=32),
        "pair_h128": c5.scaled(B=2, n=4 * 3000, seed=28, plants=16),
        # MX FP4 indexer keys (FP8 queries)
        "csa_fp4_h64_k512": c3.scaled(B=2, n=4 * 900 + 2, seed=29, idx_dtype=MXFP4),
        "pair_fp4_h128": c5.scaled(B=2, n=4 * 3000 + 1, seed=30, plants=16, idx_dtype=MXFP4),
        "prefill_fp4": c4.scaled(n=4096, Tq=200, seed=31, idx_dtype=MXFP4),
    }


CASES = small_cases()


def run_chain(cfg, split_index=False, W=None, sink=None):
    """Run every stage on the GPU and check each against the oracle; return outputs.
    sink: optional [n_h] float32 attention sink for both attention calls."""
    prob = make_problem(cfg)
    W = cfg.W if W is None else W
    B, c, dt = cfg.B, cfg.c, cfg.dtype
    n_total = prob["n_total"]
    Tq = prob["Tq"]
    q_pos_h = prob["q_pos"]
    q_pos = H.to_dev(q_pos_h)
    scale = 1.0 / math.sqrt(c)
    results = {}
    for layer in ("csa", "hca"):
        if f"X_{layer}" not in prob:
            continue
        m = cfg.m if layer == "csa" else cfg.m_hca
        Xh, Zh = prob[f"X_{layer}"], prob[f"Z_{layer}"]
        X, Z = H.to_dev(Xh), H.to_dev(Zh)
        fn = H.lib.csa_compress if layer == "csa" else H.lib.hca_compress
        C = H.run_pool(X, Z, m, dt, fn=fn)
        check_pool(Xh, Zh, dt, m, C)
        Ch = oracle.decode(H.to_host_codes(C, dt), dt)
        Xd = oracle.decode(Xh, dt)
        win_pos = H.to_dev(np.zeros(B, np.int32))
        Q = H.to_dev(prob[f"Q_{layer}"])
        if layer == "csa":
            if C.shape[1] == 0:
                continue
            qI, w, KI = H.to_dev(prob["qI"]), H.to_dev(prob["w"]), H.key_buffer(prob)
            idx, sc, alls = H.run_index(qI, w, KI, q_pos, m, cfg.k, cfg.idx_dtype, split=split_index,
                                        N_c=prob["KI"].shape[1])
            check_index(prob, q_pos_h, cfg.k, idx, sc, alls)
            idx_h = idx.cpu().numpy()
            out, lse = H.run_csa_attend(Q, C, idx, X, win_pos, q_pos, W, dt,
                                        sink=None if sink is None else H.to_dev(sink))
            rows = lambda b, t: oracle.csa_rows(Ch[b], idx_h[b, t], Xd[b], 0, int(q_pos_h[b]) + t, W)
            results["csa_idx"] = idx_h
            if "plant_positions" in prob:
                rec = np.mean([np.isin(prob["plant_positions"][b], idx_h[b, 0]).mean() for b in range(B)])
                results["planted_recall"] = rec
        else:
            if C.shape[1] == 0:
                continue
            out, lse = H.run_hca_attend(Q, C, X, win_pos, q_pos, m, W, dt,
                                        sink=None if sink is None else H.to_dev(sink))
            rows = lambda b, t: oracle.hca_rows(Ch[b], m, Xd[b], 0, int(q_pos_h[b]) + t, W)
        check_attend(prob[f"Q_{layer}"], dt, rows, out, lse, scale, sink)
        results[f"{layer}_out"] = out.cpu().numpy()
        results[f"{layer}_lse"] = lse.cpu().numpy()
        results[f"{layer}_C"] = C.cpu().numpy()
    return results


@pytest.mark.parametrize("name", list(CASES))
def test_chain_parity(name):
    print(f"[case {name}]", flush=True)
    res = run_chain(CASES[name])
    if "planted_recall" in res:
        print(f"planted recall {res['planted_recall']:.3f}")


@pytest.mark.parametrize("name", ["cfg1_tiny_fp32", "hca_h64_ragged", "csa_h128_k1024",
                                  "prefill_small", "prefill_from_zero", "prefill_odd_tq",
                                  "pair_h128"])
def test_attention_sink(name):
    """csa_attend_sink / hca_attend_sink against the oracle's sink: per-head logits of
    both signs, one dominating the rows and one at -inf (no effect)."""
    print(f"[sink {name}]", flush=True)
    cfg = CASES[name]
    rng = np.random.default_rng(41)
    sink = (rng.standard_normal(cfg.n_h) * 3).astype(np.float32)
    sink[0] = 30.0
    sink[-1] = -np.inf
    run_chain(cfg, sink=sink)


def test_sink_of_minus_inf_changes_no_bit():
    cfg = CASES["pair_h128"]
    a = run_chain(cfg)
    b = run_chain(cfg, sink=np.full(cfg.n_h, -np.inf, dtype=np.float32))
    for key in ("csa_out", "hca_out", "csa_lse", "hca_lse"):
        assert np.array_equal(a[key], b[key]), key


def test_split_index_equals_fused():
    a = run_chain(CASES["csa_h64_k512"])
    b = run_chain(CASES["csa_h64_k512"], split_index=True)
    assert np.array_equal(a["csa_idx"], b["csa_idx"])


def test_window_zero():
    run_chain(CASES["hca_h64_ragged"], W=0)
    run_chain(CASES["csa_h64_k512"], W=0)


def test_deterministic():
    a = run_chain(CASES["pair_h128"])
    b = run_chain(CASES["pair_h128"])
    for key in a:
        if isinstance(a[key], np.ndarray):
            assert np.array_equal(a[key], b[key]), key


def test_pool_bias_and_paths():
    """Positional bias, both pooling kernels (few blocks / many blocks), fp32 and bf16."""
    rng = np.random.default_rng(5)
    for dtype, m, B, n in ((BF16, 4, 2, 4 * 300 + 3), (BF16, 128, 2, 128 * 5 + 7),
                           (BF16, 128, 2, 128 * 300), (F32, 4, 1, 4 * 64), (F32, 128, 1, 128 * 3 + 1),
                           (BF16, 1, 1, 40), (BF16, 3, 1, 3 * 50 + 2)):
        c = 512 if dtype == BF16 else 64
        from synthgen.host import encode
        Xh = encode(rng.standard_normal((B, n, c), dtype=np.float32) * 0.1, dtype)
        Zh = encode(rng.standard_normal((B, n, c), dtype=np.float32), dtype)
        P = rng.standard_normal((m, c)).astype(np.float32)
        for bias in (None, P):
            out = H.run_pool(H.to_dev(Xh), H.to_dev(Zh), m, dtype,
                             P=None if bias is None else H.to_dev(bias))
            check_pool(Xh, Zh, dtype, m, out, P=bias)


def test_window_source_offset():
    """A window source holding only the last W raw tokens (win_pos = n - W) gives the same
    output as the whole raw sequence as source."""
    cfg = CASES["pair_h128"]
    prob = make_problem(cfg)
    n, W, B = prob["n_total"], cfg.W, cfg.B
    q_pos = H.to_dev(prob["q_pos"])
    for layer in ("csa", "hca"):
        X, Z = H.to_dev(prob[f"X_{layer}"]), H.to_dev(prob[f"Z_{layer}"])
        m = cfg.m if layer == "csa" else cfg.m_hca
        C = H.run_pool(X, Z, m, BF16)
        Q = H.to_dev(prob[f"Q_{layer}"])
        tail = X[:, n - W:].contiguous()
        wp0 = H.to_dev(np.zeros(B, np.int32))
        wp1 = H.to_dev(np.full(B, n - W, np.int32))
        if layer == "csa":
            idx, _, _ = H.run_index(H.to_dev(prob["qI"]), H.to_dev(prob["w"]), H.to_dev(prob["KI"]),
                                    q_pos, m, cfg.k, cfg.idx_dtype)
            a, la = H.run_csa_attend(Q, C, idx, X, wp0, q_pos, W, BF16)
            b, lb = H.run_csa_attend(Q, C, idx, tail, wp1, q_pos, W, BF16)
        else:
            a, la = H.run_hca_attend(Q, C, X, wp0, q_pos, m, W, BF16)
            b, lb = H.run_hca_attend(Q, C, tail, wp1, q_pos, m, W, BF16)
        assert torch.equal(a, b) and torch.equal(la, lb), layer


@pytest.mark.parametrize("n_h", [16, 32])
def test_fewer_heads(n_h):
    run_chain(CONFIGS[3].scaled(B=2, n=4 * 700 + 3, n_h=n_h, seed=40 + n_h))
    run_chain(CONFIGS[2].scaled(B=2, n=128 * 9 + 5, n_h=n_h, seed=50 + n_h))


def test_ties_resolve_to_lower_index():
    """Identical indexer keys give identical scores everywhere: the selection must be the
    lowest indices.  All-zero head weights give all-zero scores: same rule."""
    cfg = CONFIGS[3].scaled(B=2, n=4 * 3000, seed=61, plants=0)
    prob = make_problem(cfg)
    KI = prob["KI"].copy()
    KI[:] = KI[:, :1]                       # every key equals key 0
    prob_w0 = dict(prob)
    for name, ki, w in (("identical keys", KI, prob["w"]), ("zero weights", prob["KI"], np.zeros_like(prob["w"]))):
        q_pos = H.to_dev(prob["q_pos"])
        idx, sc, alls = H.run_index(H.to_dev(prob["qI"]), H.to_dev(w), H.to_dev(ki), q_pos, cfg.m, cfg.k,
                                    cfg.idx_dtype)
        got = idx.cpu().numpy()
        for b in range(cfg.B):
            assert np.array_equal(got[b, 0], np.arange(cfg.k)), name
        # and the oracle's selection on the GPU scores agrees
        p2 = dict(prob, KI=ki, w=w)
        check_index(p2, prob["q_pos"], cfg.k, idx, sc, alls)
