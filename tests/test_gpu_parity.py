"""GPU parity: every stage of the HIP path against the CPU oracle on identical input bytes.

Stages are compared on the bytes the GPU consumed (staged comparison): attention uses
the GPU-written compressed cache and the GPU's top-k list, the top-k check uses the
GPU's own fp32 scores.  Tolerances:
  pooling    fp32: max |d| <= 1e-5; bf16: |d| <= one bf16 ulp of the fp64 value
             + 2^-16 * sum_j S_j |x_j| (fp32 rounding of the weighted sum)
  indexer    |d| <= 1e-3 * |ref| + 1e-6 * RMS of the query's scores (the absolute floor
             only matters for ReLU zeros and exact-zero weights)
  top-k      bit-exact index lists (ascending, -1 padded) given the GPU scores
  attention  fp32: max |d| <= 1e-5; bf16: |d| minus half an ulp of the element's own
             bf16 value <= 2e-2 * RMS of the call's output; a query with at most 16 rows
             is held to 2e-2 * the larger of that and the RMS of its own output (see
             check_attend)
"""
import math

import numpy as np
import pytest
import torch

import oracle
from synthgen.configs import BF16, CONFIGS, F32, FP8, MXFP4
from synthgen.host import encode, make_problem
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


def index_tol(ref):
    """1e-3 relative, with an absolute floor of 1e-6 x the row's RMS for zero scores."""
    rms = math.sqrt(float(np.mean(ref * ref))) if ref.size else 0.0
    return 1e-3 * np.abs(ref) + 1e-6 * rms


def check_index(prob, q_pos, k, idx, sc, alls):
    cfg = prob["cfg"]
    qI, KI = decode_keys(prob)
    w = prob["w"]
    idx = idx.cpu().numpy()
    sc = sc.cpu().numpy()
    alls = alls.cpu().numpy()
    B, Tq = qI.shape[:2]
    N_c = KI.shape[1]
    worst = 0.0
    for b in range(B):
        for t in range(Tq):
            p = int(q_pos[b]) + t
            V = oracle.visible(p, cfg.m, N_c)
            ref = oracle.index_scores(qI[b, t], w[b, t], KI[b], V)
            g = alls[b, t, :V].astype(np.float64)
            if V:
                d = np.abs(g - ref)
                tol = index_tol(ref)
                worst = max(worst, float(np.max(d / np.maximum(tol, 1e-300))))
                assert np.all(d <= tol), f"scores b={b} t={t}: worst {np.max(d / tol):.3g} of the tolerance"
            want = oracle.topk(g, k)
            assert np.array_equal(idx[b, t], want), f"top-k b={b} t={t}"
            keff = min(k, V)
            assert np.array_equal(sc[b, t, :keff], alls[b, t, want[:keff]])
            assert np.all(np.isneginf(sc[b, t, keff:]))
    print(f"indexer scores: worst |d| = {worst:.3f} of the tolerance", flush=True)


FEW_ROWS = 16  # queries attending to at most this many rows take their own output's RMS


def check_attend(Qc, dtype, rows_fn, gpu_out, gpu_lse, scale, sink=None, label="", Q_ref=None):
    """rows_fn(b, t) -> fp64 row set for that query (from the GPU-consumed bytes).
    Q_ref: the fp64 queries the oracle attends with, when not the decoded Qc (queries
    normalised inside the call).

    bf16: every element's error beyond the half-ulp rounding of its own bf16 value (which
    no bf16 output avoids: an output of 1.004 in a call whose RMS is 0.147 is 1.25x of
    2e-2 x RMS away from its correctly rounded value) is at most 2e-2 x RMS of the call's
    whole output.  A query with at most FEW_ROWS rows is instead held to 2e-2 x the larger
    of that RMS and the RMS of its own output: its output is close to a single row, up to
    10x the call's RMS when the call also holds many-row queries."""
    Q = oracle.decode(Qc, dtype) if Q_ref is None else Q_ref
    B, Tq = Q.shape[:2]
    got = oracle.decode(H.to_host_codes(gpu_out, dtype), dtype)
    lse = gpu_lse.cpu().numpy().astype(np.float64)
    ref = np.zeros_like(got)
    ref_lse = np.zeros(lse.shape)
    nrows = np.zeros((B, Tq), dtype=np.int64)
    for b in range(B):
        for t in range(Tq):
            rows = rows_fn(b, t)
            nrows[b, t] = rows.shape[0]
            ref[b, t], ref_lse[b, t] = oracle.attend(Q[b, t], rows, scale, sink)
    err = np.abs(got - ref)
    if dtype == F32:
        print(f"attention {label}: max |d| = {err.max():.3g} (tolerance 1e-5)", flush=True)
        assert err.max() <= 1e-5, f"attention max |d| = {err.max()}"
        assert np.max(np.abs(lse - ref_lse)) <= 1e-5
    else:
        rms = math.sqrt(float(np.mean(ref * ref)))
        tol = np.full((B, Tq), 2e-2 * rms)
        few = nrows <= FEW_ROWS
        own = 2e-2 * np.sqrt(np.mean(ref * ref, axis=(2, 3)))
        tol[few] = np.maximum(tol[few], own[few])
        excess = err - 0.5 * bf16_ulp(ref)  # what is left after the output's own rounding
        qerr = excess.max(axis=(2, 3))
        ratio = qerr / tol
        print(f"attention {label}: max |d| = {err.max():.3g} ({err.max() / (2e-2 * rms):.3f} of 2e-2 x RMS), "
              f"beyond the half-ulp {ratio.max():.3f} of the tolerance "
              f"(2e-2 x RMS of the call; {int(few.sum())} of {few.size} queries with <= {FEW_ROWS} rows "
              f"on their own RMS, worst of those {ratio[few].max() if few.any() else 0:.3f}, "
              f"worst of the rest {ratio[~few].max() if (~few).any() else 0:.3f} of 2e-2 x the call's RMS)",
              flush=True)
        assert np.all(qerr <= tol), f"attention max |d| = {err.max()}, RMS = {rms}"
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


def run_chain(cfg, split_index=False, W=None, sink=None, nrq=None):
    """Run every stage on the GPU and check each against the oracle; return outputs.
    sink: optional [n_h] float32 attention sink for both attention calls.
    nrq: optional (gamma [c] float32 or None, d_rope, eps, theta): the attention calls
    normalise and rotate the queries themselves (csa_attend_ex / hca_attend_ex).  The
    kernel multiplies the normalised query as a bf16 MFMA operand, as the separate path
    would store it; the oracle attends with oracle.rope_tail(oracle.rmsnorm(q)) computed
    in fp64 and rounded to bf16 (nearest even) at that same point, and the error against
    the unrounded fp64 query is printed beside it."""
    prob = make_problem(cfg)
    W = cfg.W if W is None else W
    B, c, dt = cfg.B, cfg.c, cfg.dtype
    n_total = prob["n_total"]
    Tq = prob["Tq"]
    q_pos_h = prob["q_pos"]
    q_pos = H.to_dev(q_pos_h)
    scale = 1.0 / math.sqrt(c)
    results = {}
    nrq_dev = None
    if nrq is not None:
        g, d, eps, theta = nrq
        nrq_dev = (None if g is None else H.to_dev(g), d, eps, theta)
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
                                        sink=None if sink is None else H.to_dev(sink), nrq=nrq_dev)
            rows = lambda b, t: oracle.csa_rows(Ch[b], idx_h[b, t], Xd[b], 0, int(q_pos_h[b]) + t, W)
            results["csa_idx"] = idx_h
            if "plant_positions" in prob:
                rec = np.mean([np.isin(prob["plant_positions"][b], idx_h[b, 0]).mean() for b in range(B)])
                results["planted_recall"] = rec
        else:
            if C.shape[1] == 0:
                continue
            out, lse = H.run_hca_attend(Q, C, X, win_pos, q_pos, m, W, dt,
                                        sink=None if sink is None else H.to_dev(sink), nrq=nrq_dev)
            rows = lambda b, t: oracle.hca_rows(Ch[b], m, Xd[b], 0, int(q_pos_h[b]) + t, W)
        Q_ref = None
        if nrq is not None:
            g, d, eps, theta = nrq
            pos = q_pos_h[:, None, None] + np.arange(Tq)[None, :, None]       # [B, Tq, 1]
            q64 = oracle.rope_tail(oracle.rmsnorm(oracle.decode(prob[f"Q_{layer}"], dt), g, eps),
                                   np.broadcast_to(pos, (B, Tq, cfg.n_h)), d, theta)
            Q_ref = oracle.decode(encode(q64, dt), dt)
            got = oracle.decode(H.to_host_codes(out, dt), dt)
            full = np.stack([np.stack([oracle.attend(q64[b, t], rows(b, t), scale, sink)[0]
                                       for t in range(Tq)]) for b in range(B)])
            print(f"{layer}: against the fp64 (unrounded) normalised query max |d| = "
                  f"{np.abs(got - full).max():.3g}, {np.abs(got - full).max() / (2e-2 * np.sqrt(np.mean(full ** 2))):.3f} "
                  f"of 2e-2 x RMS", flush=True)
        check_attend(prob[f"Q_{layer}"], dt, rows, out, lse, scale, sink, label=layer, Q_ref=Q_ref)
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


NR_EPS, NR_THETA = 1e-6, 10000.0


@pytest.mark.parametrize("name,d,gain,sink", [
    ("hca_h64_ragged", 64, True, False),
    ("csa_h128_k1024", 64, True, True),
    ("csa_h64_k512", 128, False, False),
    ("pair_h128", 64, True, False),
    ("prefill_small", 64, True, False),
    ("prefill_odd_tq", 0, True, True),      # norm only
    ("few_heads_h32", 64, True, False),     # two waves, column-split workgroups
])
def test_queries_normalised_inside_attention(name, d, gain, sink):
    """csa_attend_ex / hca_attend_ex with q_norm = 1: RMSNorm + RoPE of the queries in the
    attention kernel, against the oracle attending with rope_tail(rmsnorm(q)) formed in
    fp64 and rounded to bf16 where the kernel rounds it (the MFMA operand, the precision
    the separate row kernel stores)."""
    print(f"[query norm {name} d={d} gain={gain} sink={sink}]", flush=True)
    cfg = CASES[name] if name in CASES else CONFIGS[3].scaled(B=2, n=4 * 700 + 3, n_h=32, seed=72)
    rng = np.random.default_rng(73)
    g = rng.uniform(0.5, 1.5, size=cfg.c).astype(np.float32) if gain else None
    sk = (rng.standard_normal(cfg.n_h) * 3).astype(np.float32) if sink else None
    run_chain(cfg, sink=sk, nrq=(g, d, NR_EPS, NR_THETA))


def test_query_norm_inside_equals_the_row_kernel_first():
    """The fused query norm against csahca_norm_rope on the queries followed by the plain
    call: the same arithmetic up to the order of the sum of squares, so outputs agree to a
    bf16 ulp or two (a normalised query element can round the other way)."""
    cfg = CASES["pair_h128"]
    prob = make_problem(cfg)
    B, c, Tq, n_h, W = cfg.B, cfg.c, prob["Tq"], cfg.n_h, cfg.W
    m = cfg.m_hca
    rng = np.random.default_rng(74)
    g = H.to_dev(rng.uniform(0.5, 1.5, size=c).astype(np.float32))
    q_pos = H.to_dev(prob["q_pos"])
    X, Z = H.to_dev(prob["X_hca"]), H.to_dev(prob["Z_hca"])
    C = H.run_pool(X, Z, m, BF16, fn=H.lib.hca_compress)
    win_pos = H.to_dev(np.zeros(B, np.int32))
    Q = H.to_dev(prob["Q_hca"])
    fused, lf = H.run_hca_attend(Q, C, X, win_pos, q_pos, m, W, BF16, nrq=(g, 64, NR_EPS, NR_THETA))
    Qn = torch.empty_like(Q)
    H.lib.csahca_norm_rope(Q, Qn, g, q_pos, B, Tq, n_h, c, 1, 64, NR_EPS, NR_THETA, 1, BF16)
    two, lt = H.run_hca_attend(Qn, C, X, win_pos, q_pos, m, W, BF16)
    torch.cuda.synchronize()
    a = oracle.decode(H.to_host_codes(fused, BF16), BF16)
    b = oracle.decode(H.to_host_codes(two, BF16), BF16)
    same = float(np.mean(a == b))
    d = np.abs(a - b).max()
    rms = math.sqrt(float(np.mean(b * b)))
    print(f"fused vs two calls: {same:.4f} of outputs bit-identical, max |d| = {d:.3g} "
          f"({d / rms:.3g} x RMS), lse max |d| = {(lf - lt).abs().max().item():.3g}", flush=True)
    assert d <= 2e-3 * rms and same >= 0.9
    assert (lf - lt).abs().max().item() <= 1e-3


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


@pytest.mark.parametrize("n_ih,c_I", [(16, 128), (128, 128), (32, 64), (64, 64), (128, 32), (16, 32)])
def test_indexer_heads_and_widths(n_ih, c_I):
    """Every indexer shape the FP8 path is built for: 16 to 128 heads, key widths 32, 64
    and 128 (widths below 128 take the general scoring kernel and the selection through
    the group maxima), at decode and in a prefill chunk."""
    run_chain(CONFIGS[3].scaled(B=2, n=4 * 900 + 2, n_ih=n_ih, c_I=c_I, seed=100 + n_ih + c_I))
    run_chain(CONFIGS[4].scaled(n=2048 + 7, Tq=33, n_ih=n_ih, c_I=c_I, seed=200 + n_ih + c_I))


@pytest.mark.parametrize("k,W", [(1, 1), (100, 37), (777, 64), (1000, 5)])
def test_window_and_k_sizes(k, W):
    """Windows of any length up to the ring and top-k sizes that are no power of two (the
    attention splits hold whole 32-row tiles, so the compressed/window boundary and the
    list end fall inside tiles); k = 1000 is more than the 900 usable entries."""
    run_chain(CONFIGS[3].scaled(B=2, n=4 * 900 + 2, k=k, W=W, seed=80 + W))
    run_chain(CONFIGS[2].scaled(B=2, n=128 * 9 + 5, W=W, seed=90 + W))


@pytest.mark.parametrize("n_h", [16, 32, 48, 80, 96, 112])
def test_fewer_heads(n_h):
    """Every head count the bfloat16 calls accept (n_h % 16 == 0, n_h <= 128): the head
    groups of a workgroup (64, 32 or 16 heads) must tile n_h exactly."""
    run_chain(CONFIGS[3].scaled(B=2, n=4 * 700 + 3, n_h=n_h, seed=40 + n_h))
    run_chain(CONFIGS[2].scaled(B=2, n=128 * 9 + 5, n_h=n_h, seed=50 + n_h))


@pytest.mark.parametrize("n_h,Tq", [(16, 3), (16, 6), (32, 3), (48, 5), (96, 7)])
def test_prefill_head_and_query_counts(n_h, Tq):
    """HCA prefill packs up to 128 / (heads per workgroup) queries into one workgroup, a
    power of two, so chunks of a few queries with few heads take the same kernels."""
    run_chain(CONFIGS[4].scaled(n=2048 + 7, Tq=Tq, n_h=n_h, seed=70 + n_h + Tq))


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
