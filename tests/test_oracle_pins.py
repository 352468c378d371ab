"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each check is a function of an oracle implementation, so that the last test can plant
plausible mistakes in a copy of the oracle (on the CPU) and show that some pin fails.
"""
import itertools
import types

import numpy as np
import pytest
import torch

import oracle
from oracle import csahca as O
from synthgen.codecs import f32_to_bf16_bits, f32_to_e4m3fn_bits
from tests.conftest import read_golden


def _impl(**over):
    ns = types.SimpleNamespace(pool=O.pool, pool_overlap=O.pool_overlap,
                               index_scores=O.index_scores, topk=O.topk,
                               attend=O.attend, visible=O.visible, csa_rows=O.csa_rows,
                               hca_rows=O.hca_rows, entry_counts=O.entry_counts,
                               window_positions=O.window_positions, rmsnorm=O.rmsnorm,
                               rope_tail=O.rope_tail, norm_rope=O.norm_rope,
                               grouped_out_proj=O.grouped_out_proj,
                               entry_positions=O.entry_positions)
    for k, v in over.items():
        setattr(ns, k, v)
    return ns


# ---------------------------------------------------------------------------------------
# checks (each raises AssertionError when the implementation disagrees with its pin)
# ---------------------------------------------------------------------------------------
def check_budget_counts(o):
    g = read_golden("budget_counts.txt")
    stored, attended, hca = o.entry_counts(g["n"], 4, 128, 1024, 128)
    assert stored == g["csa_stored"]
    assert attended == g["csa_attended"]
    assert hca == g["hca_stored"] == g["hca_attended"]


def check_worked_example(o):
    g = read_golden("worked_example.txt")
    for n in (2000, 32000, 1000000):
        _, att, _ = o.entry_counts(n, 4, 128, 1024, 128)
        assert att == g[f"n_{n}_attended"]
        pct = 100.0 * att / n
        want = g[f"n_{n}_percent"]
        # the page rounds to the shown digits
        digits = len(str(want).split(".")[1]) if "." in str(want) else 0
        assert round(pct, digits) == pytest.approx(want)


def check_pool_counts(o):
    g = read_golden("pool_counts.txt")
    X = np.zeros((g["tokens"], 2))
    assert o.pool(X, X, 4).shape[0] == g["entries_m4"]
    assert o.pool(X, X, 128).shape[0] == g["entries_m128"]
    _, _, hca = o.entry_counts(1_000_000, 4, 128, 1024, 128)
    assert abs((hca - 128) - g["hca_entries_1m_approx"]) < 50


def _budget_toy_inputs():
    # Draw order of the page's toy: keys (16 x 6), then 4 position logits, then the query.
    st = np.random.RandomState(0)
    keys = st.randn(16, 6)
    logits = st.randn(4)
    q = st.randn(6)
    return keys, logits, q


def check_budget_toy(o):
    """Position-only softmax gate (Z[j] = logit of position j), then the indexer with one
    head of weight 1 -- its ReLU keeps the two positive winners -- then top-2."""
    g = read_golden("budget_counts.txt")
    keys, logits, q = _budget_toy_inputs()
    Z = np.repeat(np.tile(logits, 4)[:, None], 6, axis=1)
    C = o.pool(keys, Z, 4)
    assert C.shape[0] == g["toy_entries"]
    s = o.index_scores(q[None, :], np.ones(1), C, C.shape[0])
    assert sorted(o.topk(s, 2).tolist()) == sorted(g["toy_top2"])


def _recall_toy_inputs():
    rng = np.random.default_rng(0)
    keys = rng.normal(0, 1, (64, 8))
    query = keys[37] + rng.normal(0, 0.3, 8)
    return keys, query


def check_pooling_recall(o):
    """Mean pooling (constant gate logits) and a single-head indexer of weight 1."""
    g = read_golden("pooling_recall.txt")
    keys, query = _recall_toy_inputs()
    for m in (1, 4, 16):
        C = o.pool(keys, np.zeros_like(keys), m)
        s = o.index_scores(query[None, :], np.ones(1), C, C.shape[0])
        srt = np.sort(s)
        assert int(np.argmax(s)) == g[f"best_entry_m{m}"]
        assert round(srt[-1] - srt[-2], 2) == pytest.approx(g[f"lead_m{m}"])
    C = o.pool(keys, np.zeros_like(keys), 4)
    s = o.index_scores(query[None, :], np.ones(1), C, C.shape[0])
    assert sorted(x for x in o.topk(s, 3).tolist() if x >= 0) == sorted(g["top3_m4"])
    # window of 8 raw tokens + 3 selected entries
    assert len(o.window_positions(63, 8)) + 3 == g["entries_attended"]


def check_pool_closed_forms(o):
    rng = np.random.default_rng(7)
    n, c = 24, 5
    X = rng.normal(size=(n, c))
    Z = rng.normal(size=(n, c)) * 3
    # identical tokens inside each block -> that token, for any gate
    Xi = np.repeat(X[::4], 4, axis=0)
    np.testing.assert_allclose(o.pool(Xi, Z, 4), X[::4], rtol=0, atol=1e-14)
    # gate constant over a block (per channel) -> arithmetic mean of the block
    Zc = np.repeat(rng.normal(size=(n // 4, c)), 4, axis=0)
    np.testing.assert_allclose(o.pool(X, Zc, 4), X.reshape(6, 4, c).mean(1), atol=1e-14)
    # shifting the logits of a block-channel by a constant changes nothing
    Zs = Z + np.repeat(rng.normal(size=(n // 4, c)) * 10, 4, axis=0)
    np.testing.assert_allclose(o.pool(X, Zs, 4), o.pool(X, Z, 4), atol=1e-12)
    # m = 1 is the identity
    np.testing.assert_allclose(o.pool(X, Z, 1), X, atol=0)
    # m = 2 in closed form: weight of the first token is the logistic of z0 - z1, per channel
    a = 1.0 / (1.0 + np.exp(-(Z[0::2] - Z[1::2])))
    np.testing.assert_allclose(o.pool(X, Z, 2), a * X[0::2] + (1 - a) * X[1::2], atol=1e-13)
    # a positional bias alone (Z = 0) is the page's position gate: token j of every block
    # gets exp(P_j) / sum exp(P)
    P = rng.normal(size=(3, c))
    Xp = X[:21]
    wts = np.exp(P) / np.exp(P).sum(0)
    want = (Xp[:21].reshape(7, 3, c) * wts[None]).sum(1)
    np.testing.assert_allclose(o.pool(Xp, np.zeros_like(Xp), 3, P), want, atol=1e-13)
    # ragged tail: 26 tokens with m = 4 -> 6 entries, the last 2 tokens dropped
    assert o.pool(np.vstack([X, X[:2]]), np.vstack([Z, Z[:2]]), 4).shape == (6, c)


def check_pool_overlap_closed_forms(o):
    """Overlapped two-stream pooling ([P2] V.1): entry i pools stream a over block i and
    stream b over block i-1 with one softmax over the 2m logits (m for the first block)."""
    rng = np.random.default_rng(11)
    m, c, N = 4, 3, 6
    n = m * N
    Xa, Xb = rng.normal(size=(n, c)), rng.normal(size=(n, c))
    Za, Zb = rng.normal(size=(n, c)) * 2, rng.normal(size=(n, c)) * 2
    # every one of an entry's 2m raw values equal to v_i -> v_i, for any gate
    v = rng.normal(size=(N, c))
    Xa_i = np.repeat(v, m, axis=0)
    Xb_i = np.repeat(np.vstack([v[1:], v[-1:]]), m, axis=0)  # block i-1 of b carries v_i
    np.testing.assert_allclose(o.pool_overlap(Xa_i, Za, Xb_i, Zb, m), v, rtol=0, atol=1e-14)
    # equal logits -> the mean of the 2m values (of stream a's m values for entry 0)
    Zc = np.zeros((n, c))
    want = [Xa[:m].mean(0)] + [np.vstack([Xa[m * i:m * i + m], Xb[m * i - m:m * i]]).mean(0)
                               for i in range(1, N)]
    np.testing.assert_allclose(o.pool_overlap(Xa, Zc, Xb, Zc, m), np.array(want), atol=1e-14)
    # stream b gated off -> the single-stream pool of stream a
    off = np.full((n, c), -1e300)
    np.testing.assert_allclose(o.pool_overlap(Xa, Za, Xb, off, m), o.pool(Xa, Za, m), atol=1e-14)
    # stream a gated off -> entry i >= 1 is stream b's pool of block i-1
    np.testing.assert_allclose(o.pool_overlap(Xa, off, Xb, Zb, m)[1:], o.pool(Xb, Zb, m)[:N - 1],
                               atol=1e-14)
    # m = 1: a two-token softmax, the weight of stream a is the logistic of za_i - zb_{i-1}
    s = 1.0 / (1.0 + np.exp(-(Za[1:] - Zb[:-1])))
    got = o.pool_overlap(Xa, Za, Xb, Zb, 1)
    np.testing.assert_allclose(got[1:], s * Xa[1:] + (1 - s) * Xb[:-1], atol=1e-13)
    np.testing.assert_allclose(got[0], Xa[0], atol=0)
    # positional bias alone: rows 0..m-1 weigh stream a's positions, m..2m-1 stream b's
    P = rng.normal(size=(2 * m, c))
    wts = np.exp(P) / np.exp(P).sum(0)
    i = 3
    want = (wts[:m] * Xa[m * i:m * i + m]).sum(0) + (wts[m:] * Xb[m * i - m:m * i]).sum(0)
    np.testing.assert_allclose(o.pool_overlap(Xa, Zc, Xb, Zc, m, P)[i], want, atol=1e-13)
    # an append (prev = 1) over blocks i-1 and i emits entry i alone
    sl = slice(m * (i - 1), m * (i + 1))
    np.testing.assert_allclose(o.pool_overlap(Xa[sl], Za[sl], Xb[sl], Zb[sl], m, prev=1)[0],
                               o.pool_overlap(Xa, Za, Xb, Zb, m)[i], atol=1e-14)
    # ragged tail: whole blocks only
    assert o.pool_overlap(Xa[:n - 1], Za[:n - 1], Xb[:n - 1], Zb[:n - 1], m).shape == (N - 1, c)


def check_indexer_closed_forms(o):
    rng = np.random.default_rng(3)
    n_ih, c_I, N = 4, 6, 9
    # indexer queries along the first n_ih axes: q_h . k_s is coordinate h of k_s
    qI = np.eye(n_ih, c_I)
    KI = rng.normal(size=(N, c_I))
    w = rng.random(n_ih)
    got = o.index_scores(qI, w, KI, N)
    for s in range(N):
        want = sum(w[h] * max(0.0, KI[s, h]) for h in range(n_ih))
        assert got[s] == pytest.approx(want, abs=1e-14)
    # all weights zero -> all scores zero
    assert np.all(o.index_scores(qI, np.zeros(n_ih), KI, N) == 0)
    # positive scaling of the weights scales the scores and keeps the selection
    s1 = o.index_scores(rng.normal(size=(n_ih, c_I)), w, KI, N)
    qq = rng.normal(size=(n_ih, c_I))
    s1 = o.index_scores(qq, w, KI, N)
    s2 = o.index_scores(qq, 2.5 * w, KI, N)
    np.testing.assert_allclose(s2, 2.5 * s1, atol=1e-13)
    assert np.array_equal(o.topk(s1, 3), o.topk(s2, 3))
    # only the first V entries are scored
    assert o.index_scores(qq, w, KI, 5).shape == (5,)


def _brute_topk(scores, k):
    """The unique set of min(k, V) indices each of which beats every index outside it
    (higher score, or equal score and lower index)."""
    V = len(scores)
    keff = min(k, V)

    def beats(i, j):
        return scores[i] > scores[j] or (scores[i] == scores[j] and i < j)

    found = []
    for S in itertools.combinations(range(V), keff):
        rest = [j for j in range(V) if j not in S]
        if all(beats(i, j) for i in S for j in rest):
            found.append(S)
    assert len(found) == 1
    return sorted(found[0])


def check_topk_brute(o):
    rng = np.random.default_rng(11)
    for trial in range(60):
        V = int(rng.integers(1, 11))
        k = int(rng.integers(1, 13))
        if trial % 3 == 0:
            s = rng.integers(0, 3, V).astype(np.float64)       # heavy ties
        else:
            s = rng.normal(size=V)
        got = o.topk(s, k)
        keff = min(k, V)
        assert got.shape == (k,)
        assert np.all(got[keff:] == -1)
        assert got[:keff].tolist() == _brute_topk(s, k)
    # all-equal scores, including -0.0 mixed with +0.0: lowest indices win
    s = np.array([0.0, -0.0, 0.0, -0.0, 0.0, -0.0])
    assert o.topk(s, 3).tolist() == [0, 1, 2]
    # k >= V: everything, then padding
    assert o.topk(np.array([3.0, 1.0]), 4).tolist() == [0, 1, -1, -1]


def check_attend_textbook(o):
    rng = np.random.default_rng(5)
    n_h, c, R = 3, 8, 11
    Q = rng.normal(size=(n_h, c))
    rows = rng.normal(size=(R, c))
    scale = 1 / np.sqrt(c)
    Ot, _ = o.attend(Q, rows, scale)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q)[None], torch.from_numpy(rows)[None], torch.from_numpy(rows)[None],
        scale=scale)[0].numpy()
    np.testing.assert_allclose(Ot, ref, atol=1e-12)
    # log-sum-exp against the library routine
    from scipy.special import logsumexp
    _, lse = o.attend(Q, rows, scale)
    np.testing.assert_allclose(lse, logsumexp(scale * Q @ rows.T, axis=1), atol=1e-12)
    # permuting the rows changes nothing
    perm = rng.permutation(R)
    np.testing.assert_allclose(o.attend(Q, rows[perm], scale)[0], Ot, atol=1e-12)
    # two halves merged by their log-sum-exp give the joint softmax
    Oa, la = o.attend(Q, rows[:4], scale)
    Ob, lb = o.attend(Q, rows[4:], scale)
    M = np.maximum(la, lb)
    wa, wb = np.exp(la - M), np.exp(lb - M)
    merged = (wa[:, None] * Oa + wb[:, None] * Ob) / (wa + wb)[:, None]
    np.testing.assert_allclose(merged, Ot, atol=1e-12)
    # a single row is returned exactly
    np.testing.assert_array_equal(o.attend(Q, rows[:1], scale)[0], np.repeat(rows[:1], n_h, 0))


def check_attend_sink(o):
    """Per-head attention sink: a logit that joins the softmax denominator only."""
    rng = np.random.default_rng(13)
    n_h, c, R = 5, 8, 7
    Q = rng.normal(size=(n_h, c))
    rows = rng.normal(size=(R, c))
    scale = 1.0 / np.sqrt(c)
    O0, l0 = o.attend(Q, rows, scale)
    # a sink at -inf changes nothing
    O1, l1 = o.attend(Q, rows, scale, sink=np.full(n_h, -np.inf))
    np.testing.assert_allclose(O1, O0, atol=1e-15)
    np.testing.assert_allclose(l1, l0, atol=1e-15)
    # a sink of 0 is an extra row of zeros (its score q . 0 = 0, its value 0)
    O2, l2 = o.attend(Q, rows, scale, sink=np.zeros(n_h))
    O3, l3 = o.attend(Q, np.vstack([rows, np.zeros((1, c))]), scale)
    np.testing.assert_allclose(O2, O3, atol=1e-14)
    np.testing.assert_allclose(l2, l3, atol=1e-14)
    # the lse gains the sink: log(e^lse + e^sink)
    sk = rng.normal(size=n_h) * 2
    O4, l4 = o.attend(Q, rows, scale, sink=sk)
    np.testing.assert_allclose(l4, np.logaddexp(l0, sk), atol=1e-13)
    # the weights shrink by e^{lse} / (e^{lse} + e^{sink}), the logistic of lse - sink
    np.testing.assert_allclose(O4, O0 * (1.0 / (1.0 + np.exp(sk - l0)))[:, None], atol=1e-13)
    # one row v: O = v * logistic(scale * q . v - sink)
    v = rows[:1]
    z = (Q @ v.T)[:, 0] * scale
    O5, _ = o.attend(Q, v, scale, sink=sk)
    np.testing.assert_allclose(O5, (1.0 / (1.0 + np.exp(sk - z)))[:, None] * v, atol=1e-14)


def check_rows_and_visibility(o):
    rng = np.random.default_rng(9)
    c, m, W = 4, 4, 8
    n = 64
    X = rng.normal(size=(n, c))
    Z = rng.normal(size=(n, c))
    C = o.pool(X, Z, m)
    # visibility: a block becomes usable when its last token is reached
    assert [o.visible(p, 4, 16) for p in (0, 2, 3, 4, 7, 63, 1000)] == [0, 0, 1, 1, 2, 16, 16]
    # window includes the query token; clipped at the sequence start
    assert o.window_positions(0, 8).tolist() == [0]
    assert o.window_positions(20, 8).tolist() == list(range(13, 21))
    assert o.window_positions(5, 0).tolist() == []
    # k >= visible: CSA over every usable entry equals HCA over the same cache
    p = 37
    V = o.visible(p, m, C.shape[0])
    idx = np.full(20, -1)
    idx[:V] = np.arange(V)
    Q = rng.normal(size=(2, c))
    a = o.attend(Q, o.csa_rows(C, idx, X, 0, p, W), 0.5)[0]
    b = o.attend(Q, o.hca_rows(C, m, X, 0, p, W), 0.5)[0]
    np.testing.assert_allclose(a, b, atol=1e-14)
    # p = 0: nothing compressed is visible, the window is token 0 alone -> output = X[0]
    idx0 = np.full(4, -1)
    np.testing.assert_array_equal(o.attend(Q, o.csa_rows(C, idx0, X, 0, 0, W), 0.5)[0],
                                  np.repeat(X[:1], 2, 0))
    # window source with an offset start position
    r1 = o.hca_rows(C, m, X, 0, 50, W)
    r2 = o.hca_rows(C, m, X[30:], 30, 50, W)
    np.testing.assert_array_equal(r1, r2)
    assert r1.shape[0] == o.visible(50, m, C.shape[0]) + W
    # the position an entry carries for RoPE (reading: its block's first raw position).
    # m = 1: an entry is its token, so it carries the token's position.
    assert o.entry_positions(1, 5, 4).tolist() == [5, 6, 7, 8]
    # against the visibility rule: entry s first becomes usable at the last position of
    # its block, which starts m - 1 positions earlier
    for mm in (4, 128):
        for s_ in (0, 1, 7, 300):
            p_first = next(p for p in range(mm * (s_ + 2)) if o.visible(p, mm, 10 ** 6) > s_)
            assert o.entry_positions(mm, s_, 1)[0] == p_first - (mm - 1)
    assert o.entry_positions(4, 3, 3).tolist() == [12, 16, 20]


def check_rmsnorm(o):
    """RMSNorm: values worked by hand, and the invariants of the definition."""
    # [3, 4]: mean square 12.5; with eps = 3.5 the divisor is sqrt(16) = 4
    np.testing.assert_allclose(o.rmsnorm(np.array([3.0, 4.0]), eps=3.5), [0.75, 1.0], atol=1e-15)
    # no centring: [1, 1, 1, 5] has mean square 7 (a LayerNorm would subtract the mean 2)
    np.testing.assert_allclose(o.rmsnorm(np.array([1.0, 1, 1, 5]), eps=0.0),
                               np.array([1.0, 1, 1, 5]) / np.sqrt(7.0), atol=1e-15)
    rng = np.random.default_rng(21)
    x = rng.normal(size=(6, 16)) * 3
    y = o.rmsnorm(x, eps=0.0)
    np.testing.assert_allclose(np.sqrt((y * y).mean(axis=-1)), 1.0, atol=1e-14)  # unit RMS
    np.testing.assert_allclose(o.rmsnorm(2.5 * x, eps=0.0), y, atol=1e-14)      # scale-free
    np.testing.assert_allclose(o.rmsnorm(-x, eps=0.0), -y, atol=1e-14)
    g = rng.uniform(0.5, 2.0, size=16)
    np.testing.assert_allclose(o.rmsnorm(x, g, eps=0.0), y * g, atol=1e-14)     # per-channel gain
    # a constant row returns the gain (with the row's sign)
    np.testing.assert_allclose(o.rmsnorm(np.full(16, -0.3), g, eps=0.0), -g, atol=1e-14)
    assert np.all(o.rmsnorm(np.zeros(8), eps=1e-6) == 0.0)


def check_rope(o):
    """Partial RoPE: consecutive pairs of the last d dimensions rotate by pos * f_i,
    f_i = theta^(-2i/d)."""
    c, d = 12, 8
    rng = np.random.default_rng(22)
    x = rng.normal(size=(5, c))
    np.testing.assert_allclose(o.rope_tail(x, np.zeros(5), d), x, atol=0)        # position 0
    r = o.rope_tail(x, np.arange(5) * 7, d)
    np.testing.assert_array_equal(r[:, :c - d], x[:, :c - d])                    # head untouched
    # one-hot on the first rotated dimension: pair 0 has frequency 1 and rotates
    # counter-clockwise into its partner, the next dimension
    e = np.zeros((1, c))
    e[0, c - d] = 1.0
    for p in (1, 2, 5):
        out = o.rope_tail(e, [p], d)[0]
        np.testing.assert_allclose(out[c - d:c - d + 2], [np.cos(p), np.sin(p)], atol=1e-15)
        np.testing.assert_allclose(np.delete(out, [c - d, c - d + 1]), 0.0, atol=0)
    # pair i = 16 of 64 rotated dimensions: f = 10000^(-1/2) = 0.01, so position 100 turns it
    # by exactly one radian
    e = np.zeros((1, 64))
    e[0, 32] = 1.0
    np.testing.assert_allclose(o.rope_tail(e, [100], 64)[0, 32:34], [np.cos(1.0), np.sin(1.0)],
                               atol=1e-14)
    # theta = 1: every pair turns by the position itself
    e = np.zeros((1, 8))
    e[0, 6] = 1.0
    np.testing.assert_allclose(o.rope_tail(e, [3], 8, theta=1.0)[0, 6:], [np.cos(3), np.sin(3)],
                               atol=1e-15)
    # pair norms are kept; rotations compose; scores depend on the offset only
    pn = lambda a: np.hypot(a[..., c - d::2], a[..., c - d + 1::2])
    np.testing.assert_allclose(pn(r), pn(x), atol=1e-14)
    np.testing.assert_allclose(o.rope_tail(o.rope_tail(x, [3] * 5, d), [1000] * 5, d),
                               o.rope_tail(x, [1003] * 5, d), atol=1e-12)
    q, k = x[0], x[1]
    s1 = o.rope_tail(q, 50, d) @ o.rope_tail(k, 20, d)
    s2 = o.rope_tail(q, 1030, d) @ o.rope_tail(k, 1000, d)
    assert abs(s1 - s2) < 1e-12
    # norm then RoPE: with unit gain the order does not matter (RoPE keeps the RMS)
    np.testing.assert_allclose(o.norm_rope(x, np.arange(5), None, 1e-6, d),
                               o.rmsnorm(o.rope_tail(x, np.arange(5), d), None, 1e-6), atol=1e-14)


def check_grouped_out_proj(o):
    """Grouped output projection: a dense projection whose weight is block diagonal over
    the head groups; one group is a plain linear layer; one-hot inputs pick weights."""
    rng = np.random.default_rng(23)
    T, n_h, c, g, d_g = 3, 6, 4, 3, 5
    K_g = n_h * c // g
    O = rng.normal(size=(T, n_h, c))
    Wg = rng.normal(size=(g, d_g, K_g))
    Y = o.grouped_out_proj(O, Wg)
    assert Y.shape == (T, g * d_g)
    # the same map as one dense [g*d_g, n_h*c] weight with zero blocks off the diagonal,
    # evaluated element by element
    Wd = np.zeros((g * d_g, n_h * c))
    for gi in range(g):
        Wd[gi * d_g:(gi + 1) * d_g, gi * K_g:(gi + 1) * K_g] = Wg[gi]
    X = O.reshape(T, -1)
    dense = np.array([[sum(Wd[j, k] * X[t, k] for k in range(n_h * c)) for j in range(g * d_g)]
                      for t in range(T)])
    np.testing.assert_allclose(Y, dense, atol=1e-12)
    # head h of a one-hot input lands in group h // (n_h / g) only, and picks the weight
    # column of its position inside the group
    for h, ch in ((0, 0), (2, 3), (5, 1)):
        e = np.zeros((1, n_h, c))
        e[0, h, ch] = 1.0
        y = o.grouped_out_proj(e, Wg)[0]
        gi, k = h // (n_h // g), (h % (n_h // g)) * c + ch
        want = np.zeros(g * d_g)
        want[gi * d_g:(gi + 1) * d_g] = Wg[gi][:, k]
        np.testing.assert_array_equal(y, want)
    # g = 1 is the plain linear layer of the concatenated heads
    W1 = rng.normal(size=(1, 2, n_h * c))
    np.testing.assert_allclose(o.grouped_out_proj(O, W1), X @ W1[0].T, atol=1e-12)


ALL_CHECKS = [check_budget_counts, check_worked_example, check_pool_counts, check_budget_toy,
              check_pooling_recall, check_pool_closed_forms, check_pool_overlap_closed_forms,
              check_indexer_closed_forms,
              check_topk_brute, check_attend_textbook, check_attend_sink,
              check_rows_and_visibility, check_rmsnorm, check_rope, check_grouped_out_proj]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(_impl())


# ---------------------------------------------------------------------------------------
# storage decoding pins
# ---------------------------------------------------------------------------------------
def test_e4m3fn_known_codes():
    t = oracle.E4M3FN_TABLE
    assert t[0x38] == 1.0
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x01] == 2.0 ** -9           # smallest subnormal
    assert t[0x08] == 2.0 ** -6           # smallest normal
    assert t[0x07] == 7 * 2.0 ** -9       # largest subnormal
    assert t[0x40] == 2.0 and t[0x3C] == 1.5
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0x80] == 0.0 and np.signbit(t[0x80])
    finite = t[~np.isnan(t)]
    assert len(finite) == 254 and len(np.unique(finite)) == 253   # +0 and -0 compare equal


def test_e4m3fn_roundtrip_and_rounding():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.decode_e4m3fn(codes)
    assert np.array_equal(f32_to_e4m3fn_bits(vals.astype(np.float32)), codes)
    # ties go to the even mantissa; beyond 448 saturates
    enc = lambda x: int(f32_to_e4m3fn_bits(np.array([x], np.float32))[0])
    assert enc(1.0625) == 0x38            # halfway 1.0 / 1.125 -> 1.0 (even)
    assert enc(1.1875) == 0x3A            # halfway 1.125 / 1.25 -> 1.25 (even)
    assert enc(470.0) == 0x7E and enc(1e6) == 0x7E and enc(-1e6) == 0xFE
    assert enc(2.0 ** -10) == 0x00        # halfway 0 / 2^-9 -> 0
    assert enc(3 * 2.0 ** -10) == 0x02    # halfway 2^-9 / 2^-8 -> 2^-8 (even)
    # every encoded value is the nearest representable one
    rng = np.random.default_rng(0)
    x = rng.normal(size=4000).astype(np.float32) * 30
    dec = oracle.decode_e4m3fn(f32_to_e4m3fn_bits(x))
    finite = np.unique(oracle.E4M3FN_TABLE[~np.isnan(oracle.E4M3FN_TABLE)])
    nearest = finite[np.abs(x[:, None].astype(np.float64) - finite[None, :]).argmin(1)]
    assert np.all(np.abs(dec - x) <= np.abs(nearest - x) + 0)


def test_e2m1_known_codes():
    """OCP FP4 E2M1: bias 1, one mantissa bit; codes 0..7 are 0, 0.5, 1, 1.5, 2, 3, 4, 6
    and bit 3 is the sign."""
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    want = np.array(mags + [-v for v in mags])
    np.testing.assert_array_equal(oracle.E2M1_TABLE, want)


def test_mxfp4_packing_and_scales():
    """Two elements per byte, the first in the low nibble; E8M0 scale s is 2^(s - 127)."""
    packed = np.zeros((1, 16), dtype=np.uint8)
    packed[0, 0] = 0x21                      # element 0 = code 1 (0.5), element 1 = code 2 (1.0)
    packed[0, 15] = 0xF7                     # element 30 = 6, element 31 = -6
    v = oracle.decode_mxfp4(packed, np.array([[127]], dtype=np.uint8))
    assert v.shape == (1, 32)
    assert (v[0, 0], v[0, 1], v[0, 30], v[0, 31]) == (0.5, 1.0, 6.0, -6.0)
    assert np.all(v[0, 2:30] == 0)
    np.testing.assert_array_equal(oracle.decode_mxfp4(packed, np.array([[128]], np.uint8)), 2 * v)
    np.testing.assert_array_equal(oracle.decode_mxfp4(packed, np.array([[120]], np.uint8)), v / 128)
    with pytest.raises(ValueError):
        oracle.decode_mxfp4(packed, np.array([[255]], np.uint8))


def test_mxfp4_roundtrip_and_rounding():
    from synthgen.codecs import f32_to_mxfp4
    rng = np.random.default_rng(9)
    # representable blocks: decoding, encoding and decoding again gives the same values
    p = rng.integers(0, 256, size=(50, 64), dtype=np.uint8)
    sc = rng.integers(100, 150, size=(50, 4)).astype(np.uint8)
    v = oracle.decode_mxfp4(p, sc)
    p2, s2 = f32_to_mxfp4(v.astype(np.float32))
    np.testing.assert_array_equal(oracle.decode_mxfp4(p2, s2), v)
    # the block scale puts the largest magnitude in [4, 8): error within one 2^X step
    x = rng.standard_normal((200, 128)) * np.exp2(rng.integers(-6, 6, size=(200, 1)))
    p3, s3 = f32_to_mxfp4(x.astype(np.float32))
    q = oracle.decode_mxfp4(p3, s3)
    step = np.repeat(np.exp2(s3.astype(float) - 127.0), 32, axis=1)
    assert np.all(np.abs(q - x.astype(np.float32)) <= 2.0 * step)
    amax = np.abs(x.astype(np.float32)).reshape(200, 4, 32).max(-1)
    assert np.all((amax / np.exp2(s3.astype(float) - 127.0) >= 4) & (amax / np.exp2(s3.astype(float) - 127.0) < 8))
    # the device generator's encoder (torch; run on the CPU here) writes the same bytes
    from synthgen.device import _mxfp4
    xt = x.astype(np.float32)
    xt[0, :8] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.9]
    pa, sa = f32_to_mxfp4(xt)
    pb, sb = _mxfp4(torch.from_numpy(xt))
    np.testing.assert_array_equal(pa, pb.numpy())
    np.testing.assert_array_equal(sa, sb.numpy())
    # ties go to the even code: 1.25 -> 1.0, 1.75 -> 2.0, 5.0 -> 4.0 (block max 6 -> unit scale)
    t = np.zeros((1, 32), np.float32)
    t[0, :4] = [1.25, 1.75, 5.0, 6.0]
    pt, st = f32_to_mxfp4(t)
    assert st[0, 0] == 127
    np.testing.assert_array_equal(oracle.decode_mxfp4(pt, st)[0, :4], [1.0, 2.0, 4.0, 6.0])


def test_bf16_roundtrip_and_rounding():
    rng = np.random.default_rng(1)
    x = rng.normal(size=10000).astype(np.float32)
    d = oracle.decode_bf16(f32_to_bf16_bits(x))
    assert np.all(np.abs(d - x) <= np.abs(x) * 2.0 ** -8)
    # against torch's conversion (round to nearest even)
    tb = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(d, tb)
    assert oracle.decode_bf16(f32_to_bf16_bits(np.array([1 + 2 ** -8], np.float32)))[0] == 1.0
    assert oracle.decode_bf16(f32_to_bf16_bits(np.array([1 + 3 * 2 ** -8], np.float32)))[0] \
        == 1 + 2 ** -6


# ---------------------------------------------------------------------------------------
# the pins catch plausible mistakes (mistakes planted in copies of the oracle, on the CPU)
# ---------------------------------------------------------------------------------------
_ORIG_POOL, _ORIG_ATTEND = O.pool, O.attend


def _pool_wrong_axis(X, Z, m, P=None):
    X = np.asarray(X, float)
    Z = np.asarray(Z, float)
    n, c = X.shape
    N = n // m
    zb = Z[:N * m].reshape(N, m, c)
    e = np.exp(zb - zb.max(axis=2, keepdims=True))
    S = e / e.sum(axis=2, keepdims=True)                 # softmax over channels
    return (S * X[:N * m].reshape(N, m, c)).sum(1)


def _pool_ceil(X, Z, m, P=None):
    X = np.asarray(X, float)
    pad = (-X.shape[0]) % m
    Xp = np.vstack([X, np.zeros((pad, X.shape[1]))])
    Zp = np.vstack([np.asarray(Z, float), np.zeros((pad, X.shape[1]))])
    return _ORIG_POOL(Xp, Zp, m, P)                      # emits the partial tail block


_ORIG_POOL_OVERLAP = O.pool_overlap


def _overlap_same_block(Xa, Za, Xb, Zb, m, P=None, prev=0):
    # stream b taken over block i instead of block i-1
    Xb2 = np.vstack([np.asarray(Xb, float)[m:], np.zeros((m, np.shape(Xb)[1]))])
    Zb2 = np.vstack([np.asarray(Zb, float)[m:], np.zeros((m, np.shape(Zb)[1]))])
    return _ORIG_POOL_OVERLAP(Xa, Za, Xb2, Zb2, m, P, prev)


def _overlap_two_softmaxes(Xa, Za, Xb, Zb, m, P=None, prev=0):
    # each stream normalised on its own, then summed
    a = O.pool(Xa, Za, m, None if P is None else np.asarray(P)[:m])
    b = O.pool(Xb, Zb, m, None if P is None else np.asarray(P)[m:])
    out = a.copy()
    out[1:] += b[:-1]
    return out[prev:]


def _overlap_zero_block_before_first(Xa, Za, Xb, Zb, m, P=None, prev=0):
    # the missing block -1 treated as zero values with zero logits
    z = np.zeros((m, np.shape(Xa)[1]))
    out = _ORIG_POOL_OVERLAP(np.vstack([z, Xa]), np.vstack([z, Za]), np.vstack([z, Xb]),
                             np.vstack([z, Zb]), m, P, prev)
    return out[1:]


def _scores_no_relu(qI, w, KI, V):
    return (np.asarray(KI, float)[:V] @ np.asarray(qI, float).T) @ np.asarray(w, float)


def _topk_high_index_wins(scores, k):
    s = np.asarray(scores, float)
    V = len(s)
    keff = min(k, V)
    order = np.lexsort((-np.arange(V), -s))
    out = np.full(k, -1)
    out[:keff] = np.sort(order[:keff])
    return out


def _attend_no_scale(Q, rows, scale, sink=None):
    return _ORIG_ATTEND(Q, rows, 1.0, sink)


def _attend_transposed(Q, rows, scale, sink=None):
    Q = np.asarray(Q, float)
    rows = np.asarray(rows, float)
    s = (Q @ rows.T) * scale
    e = np.exp(s - s.max(0, keepdims=True))
    p = e / e.sum(0, keepdims=True)                      # normalised over heads
    return p @ rows, np.zeros(Q.shape[0])


def _attend_sink_scaled(Q, rows, scale, sink=None):
    # the sink multiplied by the attention scale like a dot product
    return _ORIG_ATTEND(Q, rows, scale, None if sink is None else np.asarray(sink) * scale)


def _attend_sink_in_numerator(Q, rows, scale, sink=None):
    # the sink as a row of ones (it then adds to every output value)
    if sink is None:
        return _ORIG_ATTEND(Q, rows, scale)
    Q = np.asarray(Q, float)
    rows = np.asarray(rows, float)
    s = np.hstack([(Q @ rows.T) * scale, np.asarray(sink, float)[:, None]])
    e = np.exp(s - s.max(1, keepdims=True))
    vals = np.vstack([rows, np.ones((1, rows.shape[1]))])
    return (e @ vals) / e.sum(1, keepdims=True), np.log(e.sum(1)) + s.max(1)


def _visible_off_by_one(p, m, N):
    return int(min(N, int(p) // m))


def _window_excl(p, W):
    return np.arange(max(0, int(p) - W), int(p), dtype=np.int64)


def _counts_ceil(n, m, m_hca, k, W):
    nc = -(-n // m)
    return nc + W, min(nc, k) + W, -(-n // m_hca) + W


def _rmsnorm_centred(x, gamma=None, eps=1e-6):
    x = np.asarray(x, dtype=np.float64)
    x = x - x.mean(axis=-1, keepdims=True)
    y = x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    return y if gamma is None else y * gamma


def _rmsnorm_eps_outside(x, gamma=None, eps=1e-6):
    x = np.asarray(x, dtype=np.float64)
    y = x / (np.sqrt((x * x).mean(axis=-1, keepdims=True)) + eps)
    return y if gamma is None else y * gamma


def _rope_variant(half_split=False, sign=1.0, fexp=2.0, head=False):
    def f(x, pos, d_rope=64, theta=10000.0):
        x = np.array(x, dtype=np.float64)
        c = x.shape[-1]
        i = np.arange(d_rope // 2)
        ang = sign * np.asarray(pos, dtype=np.float64)[..., None] * theta ** (-fexp * i / d_rope)
        lo = 0 if head else c - d_rope
        t = x[..., lo:lo + d_rope]
        if half_split:
            a, b = t[..., :d_rope // 2], t[..., d_rope // 2:]
        else:
            a, b = t[..., 0::2], t[..., 1::2]
        ra = a * np.cos(ang) - b * np.sin(ang)
        rb = a * np.sin(ang) + b * np.cos(ang)
        out = x.copy()
        if half_split:
            out[..., lo:lo + d_rope // 2], out[..., lo + d_rope // 2:lo + d_rope] = ra, rb
        else:
            out[..., lo:lo + d_rope:2], out[..., lo + 1:lo + d_rope:2] = ra, rb
        return out
    return f


def _gop_interleaved_groups(O, Wg):
    O = np.asarray(O, dtype=np.float64)
    T, n_h = O.shape[0], O.shape[1]
    g = Wg.shape[0]
    order = np.concatenate([np.arange(gi, n_h, g) for gi in range(g)])  # heads gi, gi+g, ...
    return _gop_plain(O[:, order], Wg)


def _gop_transposed_weight(O, Wg):
    O = np.asarray(O, dtype=np.float64)
    T = O.shape[0]
    X = O.reshape(T, -1)
    g, d_g, K_g = Wg.shape
    Wt = np.asarray(Wg).reshape(g, K_g, d_g)   # reads the weight as in x out
    return np.concatenate([X[:, gi * K_g:(gi + 1) * K_g] @ Wt[gi] for gi in range(g)], axis=1)


def _entry_positions_block_end(m, entry0, N):
    # the block's last raw position instead of its first
    return m * (entry0 + np.arange(N)) + m - 1


def _gop_plain(O, Wg):
    T = O.shape[0]
    X = O.reshape(T, -1)
    g, d_g, K_g = Wg.shape
    return np.concatenate([X[:, gi * K_g:(gi + 1) * K_g] @ Wg[gi].T for gi in range(g)], axis=1)


MUTANTS = {
    "gop_interleaved_head_groups": dict(grouped_out_proj=_gop_interleaved_groups),
    "gop_weight_read_in_by_out": dict(grouped_out_proj=_gop_transposed_weight),
    "rmsnorm_centred": dict(rmsnorm=_rmsnorm_centred),
    "rmsnorm_eps_outside_sqrt": dict(rmsnorm=_rmsnorm_eps_outside),
    "rope_half_split_pairs": dict(rope_tail=_rope_variant(half_split=True)),
    "rope_clockwise": dict(rope_tail=_rope_variant(sign=-1.0)),
    "rope_frequency_exponent": dict(rope_tail=_rope_variant(fexp=1.0)),
    "rope_on_first_dims": dict(rope_tail=_rope_variant(head=True)),
    "pool_softmax_over_channels": dict(pool=_pool_wrong_axis),
    "pool_emits_tail": dict(pool=_pool_ceil),
    "overlap_stream_b_same_block": dict(pool_overlap=_overlap_same_block),
    "overlap_two_softmaxes": dict(pool_overlap=_overlap_two_softmaxes),
    "overlap_zero_block_before_first": dict(pool_overlap=_overlap_zero_block_before_first),
    "indexer_without_relu": dict(index_scores=_scores_no_relu),
    "topk_higher_index_wins": dict(topk=_topk_high_index_wins),
    "attend_without_scale": dict(attend=_attend_no_scale),
    "attend_softmax_over_heads": dict(attend=_attend_transposed),
    "attend_sink_scaled": dict(attend=_attend_sink_scaled),
    "attend_sink_in_numerator": dict(attend=_attend_sink_in_numerator),
    "visibility_off_by_one": dict(visible=_visible_off_by_one),
    "window_excludes_query": dict(window_positions=_window_excl),
    "counts_round_up": dict(entry_counts=_counts_ceil),
    "entry_position_block_end": dict(entry_positions=_entry_positions_block_end),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    over = MUTANTS[name]
    # row builders call the module-level helpers, so patch those too
    for k, v in over.items():
        monkeypatch.setattr(O, k, v)
    o = _impl(**over)
    failed = 0
    for chk in ALL_CHECKS:
        try:
            chk(o)
        except (AssertionError, ValueError, IndexError):
            failed += 1
    assert failed >= 1, f"no pin detects the planted mistake {name}"
