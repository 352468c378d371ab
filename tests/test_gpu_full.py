"""Parity at the full workload sizes, in the launch configuration bench.py times.

The workloads are generated on the GPU (seeded), one decode step (or prefill chunk) runs
through the library exactly as bench.py runs it, and sampled outputs are checked against
the CPU oracle one by one: pooled blocks, every indexer score of sampled queries, the
exact top-k list of those queries given the GPU scores, and the attention output of
sampled queries over the rows the GPU attended to.  Tolerances as in test_gpu_parity.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from synthgen.configs import BF16, CONFIGS
from tests import gpu_harness as H
from tests.test_gpu_parity import bf16_ulp

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    H.require_gpu()


def codes(t):
    a = t.detach().cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def dec(t, dtype=BF16):
    return oracle.decode(codes(t), dtype)


def check_pool_blocks(X, Z, C, m, blocks):
    for b, i in blocks:
        Xb = dec(X[b, i * m:(i + 1) * m])
        Zb = dec(Z[b, i * m:(i + 1) * m])
        ref = oracle.pool(Xb, Zb, m)[0]
        cond = oracle.pool(np.abs(Xb), Zb, m)[0]
        got = dec(C[b, i])
        assert np.all(np.abs(got - ref) <= bf16_ulp(ref) + 2.0 ** -16 * cond), (b, i)


def check_index_queries(wl, queries):
    cfg, prob = wl.cfg, wl.prob
    scores = wl.scores.view(cfg.B, wl.Tq, wl.N_c)
    idx = wl.idx
    for b, t in queries:
        p = wl.n - wl.Tq + t
        V = oracle.visible(p, cfg.m, wl.N_c)
        if cfg.idx_dtype == 3:  # MX FP4 keys, FP8 queries
            qI = dec(prob["qI"][b, t], 2)
            KI = oracle.decode_mxfp4(prob["KI"][b, :V].cpu().numpy(), prob["KI_scales"][b, :V].cpu().numpy())
        else:
            qI, KI = dec(prob["qI"][b, t], cfg.idx_dtype), dec(prob["KI"][b, :V], cfg.idx_dtype)
        ref = oracle.index_scores(qI, prob["w"][b, t].cpu().numpy(), KI, V)
        g = scores[b, t, :V].cpu().numpy().astype(np.float64)
        rms = math.sqrt(float(np.mean(ref * ref)))
        tol = 1e-3 * np.abs(ref) + 1e-6 * rms
        d = np.abs(g - ref)
        print(f"scores b={b} t={t}: worst |d| = {np.max(d / tol):.3f} of the tolerance", flush=True)
        assert np.all(d <= tol), (b, t)
        assert np.array_equal(idx[b, t].cpu().numpy(), oracle.topk(g, cfg.k)), (b, t)


def attend_rows(wl, layer, b, t):
    cfg, prob = wl.cfg, wl.prob
    p = wl.n - wl.Tq + t
    X = prob[f"X_{layer}"]
    lo = max(0, p - cfg.W + 1)
    win = dec(X[b, lo:p + 1])
    C = wl.rep[0][f"C_{layer}"]
    if layer == "csa":
        sel = wl.idx[b, t]
        sel = sel[sel >= 0].long()
        comp = dec(C[b, sel])
    else:
        V = oracle.visible(p, cfg.m_hca, wl.N_h)
        comp = dec(C[b, :V])
    return np.concatenate([comp, win], axis=0)


def check_attend_queries(wl, layer, queries):
    cfg = wl.cfg
    refs, gots = [], []
    for b, t in queries:
        Q = dec(wl.prob[f"Q_{layer}"][b, t])
        ref, _ = oracle.attend(Q, attend_rows(wl, layer, b, t), wl.scale)
        refs.append(ref)
        gots.append(dec(wl.out[layer][b, t]))
    ref = np.stack(refs)
    got = np.stack(gots)
    rms = math.sqrt(float(np.mean(ref * ref)))
    err = float(np.max(np.abs(got - ref)))
    print(f"{layer}: max |d| = {err:.3g}, {err / (2e-2 * rms):.3f} of the tolerance", flush=True)
    assert err <= 2e-2 * rms, f"{layer}: max |d| {err} vs RMS {rms}"


def run_workload(ci, fp4=False):
    import bench
    cfg = CONFIGS[ci]
    if fp4:
        cfg = cfg.scaled(idx_dtype=3)
    wl = bench.Workload(cfg, 1)
    wl.step(0)
    torch.cuda.synchronize()
    return wl


def sample_blocks(rng, B, N, count, include_last=True):
    blocks = {(int(rng.integers(B)), int(rng.integers(N))) for _ in range(count)}
    if include_last:
        blocks |= {(b, N - 1) for b in range(B)}
    return sorted(blocks)


@pytest.mark.parametrize("ci", [2, 3, 5])
def test_full_decode(ci):
    print(f"[full-size decode config {ci}]", flush=True)
    wl = run_workload(ci)
    cfg = wl.cfg
    rng = np.random.default_rng(ci)
    for layer in wl.layers:
        m = cfg.m if layer == "csa" else cfg.m_hca
        N = wl.n // m
        check_pool_blocks(wl.prob[f"X_{layer}"], wl.prob[f"Z_{layer}"], wl.rep[0][f"C_{layer}"], m,
                          sample_blocks(rng, cfg.B, N, 6))
    queries = [(b, 0) for b in sorted({int(x) for x in rng.integers(0, cfg.B, 4)})]
    if "csa" in wl.layers:
        check_index_queries(wl, queries)
        # planted keys are retrieved (reported, the pages do not fix a recall)
        rec = np.mean([np.isin(wl.prob["plant_positions"][b].cpu().numpy(), wl.idx[b, 0].cpu().numpy()).mean()
                       for b in range(cfg.B)])
        print(f"planted-key recall {rec:.3f}")
    for layer in wl.layers:
        check_attend_queries(wl, layer, queries)


def test_full_decode_fp4_keys():
    """The Pro 1M decode step with MX FP4 indexer keys: scores, top-k and CSA attention on
    sampled queries, planted-key recall reported."""
    print("[full-size decode config 5, MX FP4 keys]", flush=True)
    wl = run_workload(5, fp4=True)
    cfg = wl.cfg
    queries = [(b, 0) for b in range(cfg.B)]
    check_index_queries(wl, queries)
    rec = np.mean([np.isin(wl.prob["plant_positions"][b].cpu().numpy(), wl.idx[b, 0].cpu().numpy()).mean()
                   for b in range(cfg.B)])
    print(f"planted-key recall {rec:.3f}")
    check_attend_queries(wl, "csa", queries)


def test_full_prefill():
    print("[full-size prefill config 4]", flush=True)
    wl = run_workload(4)
    cfg = wl.cfg
    rng = np.random.default_rng(4)
    for layer in wl.layers:
        m = cfg.m if layer == "csa" else cfg.m_hca
        N = wl.n // m
        n_old = wl.n_old // m
        blocks = sample_blocks(rng, 1, N, 4) + [(0, n_old), (0, n_old + 1)]
        check_pool_blocks(wl.prob[f"X_{layer}"], wl.prob[f"Z_{layer}"], wl.rep[0][f"C_{layer}"], m,
                          sorted(set(blocks)))
    ts = sorted({0, 1, 2, 3, 126, 127, 128, wl.Tq - 1} | {int(x) for x in rng.integers(0, wl.Tq, 4)})
    queries = [(0, t) for t in ts]
    check_index_queries(wl, queries)
    for layer in wl.layers:
        check_attend_queries(wl, layer, queries)
