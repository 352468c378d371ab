"""Plain fp64 NumPy definitions of pooling, lightning indexer, top-k and attention.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Slow on purpose: every function
is the definition written out, with no blocking, fusion or reordering.

Pages cited (by title and section):
  [P1] DeepSeek V4 walk-through republished on juhe.plus -- "The Code: Softmax-Gated
       Compressor", "The Code: Compressed Sparse Attention (CSA)", "The Code: Heavily
       Compressed Attention (HCA)".
  [P2] "DeepSeek-V4 Hybrid Attention: CSA, HCA, mHC, MoE" (trishampatil.com) -- section
       IV (hybrid attention block), V.1 (compression), V.2 (lightning indexer, eq. I_{t,s}),
       V.3 (core attention), VI (HCA, eq. o_{t,i}).
  [P3] "DeepSeek-V4 Architecture From Kernels ... C-Kernel-Engine" (shivasnotes.com) --
       section 6 (CSA), 7 (HCA), 9 (heterogeneous KV cache).
  [P4] "DeepSeek-V4: Anatomy of an Open-Source Frontier Model" (modernaiengineering.com
       lesson 6.7) -- "Hybrid attention with CSA and HCA", "One query in a CSA layer, step
       by step", "Worked example, step by step".

Readings where the pages are silent or disagree are stated at each function.
"""
import numpy as np

F32, BF16, FP8 = 0, 1, 2


# ----------------------------------------------------------------------------------------
# storage decoding
# ----------------------------------------------------------------------------------------
def decode_bf16(u16):
    """bfloat16 pattern -> value: the pattern is the upper half of a binary32."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def _build_e4m3fn_table():
    """Value of each OCP FP8 E4M3FN code: bias 7, 3 mantissa bits, subnormals at E = 0,
    no infinities, S.1111.111 = NaN."""
    t = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        mant = code & 0x7
        if e == 0xF and mant == 0x7:
            t[code] = np.nan
        elif e == 0:
            t[code] = sign * (mant / 8.0) * 2.0 ** (1 - 7)
        else:
            t[code] = sign * (1.0 + mant / 8.0) * 2.0 ** (e - 7)
    return t


E4M3FN_TABLE = _build_e4m3fn_table()


def decode_e4m3fn(u8):
    v = E4M3FN_TABLE[np.asarray(u8, dtype=np.uint8)]
    if np.isnan(v).any():
        raise ValueError("E4M3FN NaN code in an input")
    return v


def _build_e2m1_table():
    """Value of each OCP FP4 E2M1 code: bias 1, 1 mantissa bit, subnormal at E = 0."""
    t = np.empty(16, dtype=np.float64)
    for code in range(16):
        sign = -1.0 if code & 0x8 else 1.0
        e = (code >> 1) & 0x3
        mant = code & 0x1
        t[code] = sign * ((mant / 2.0) if e == 0 else (1.0 + mant / 2.0) * 2.0 ** (e - 1))
    return t


E2M1_TABLE = _build_e2m1_table()


def decode_mxfp4(packed, scales):
    """OCP MX FP4: packed [..., K/2] bytes (two E2M1 elements each, the first in the low
    nibble) and scales [..., K/32] E8M0 bytes (2^(s - 127), one per 32 elements; 255 is
    NaN).  Returns [..., K] fp64."""
    p = np.asarray(packed, dtype=np.uint8)
    sc = np.asarray(scales, dtype=np.uint8)
    if np.any(sc == 255):
        raise ValueError("E8M0 NaN scale in an input")
    el = np.stack([p & 0xF, p >> 4], axis=-1).reshape(p.shape[:-1] + (p.shape[-1] * 2,))
    v = E2M1_TABLE[el]
    K = v.shape[-1]
    mult = np.exp2(sc.astype(np.float64) - 127.0)
    return (v.reshape(v.shape[:-1] + (K // 32, 32)) * mult[..., None]).reshape(v.shape)


def decode(arr, dtype):
    if dtype == F32:
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == BF16:
        return decode_bf16(arr)
    if dtype == FP8:
        return decode_e4m3fn(arr)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------------------
# (a1) softmax-gated block pooling
# ----------------------------------------------------------------------------------------
def pool(X, Z, m, P=None):
    """Compressed entries of one sequence.

    [P2] V.1 / VI: an entry is the element-wise (channel-wise) weighted sum of the raw
    entries of its block, the weights being a softmax over the block's compression
    scores Z plus a positional bias.  [P1] "Softmax-Gated Compressor": the sequence is
    truncated to a whole number of blocks (the tail is not emitted) and the gate has one
    weight per position inside the block.

    Reading: Z has one logit per token and channel; the softmax runs over the m tokens of
    a block independently for each channel; the optional bias P has shape [m, c]
    (P1's gate is the case Z = 0).  Non-overlapping blocks (HCA form, and the CSA form
    used by [P1], [P3] section 6 and [P4]).

    X, Z: float arrays [n, c] (decoded).  Returns [n // m, c] fp64.
    """
    X = np.asarray(X, dtype=np.float64)
    Z = np.asarray(Z, dtype=np.float64)
    n, c = X.shape
    N = n // m
    xb = X[:N * m].reshape(N, m, c)              # block i holds tokens m*i .. m*i+m-1
    zb = Z[:N * m].reshape(N, m, c).copy()
    if P is not None:
        zb = zb + np.asarray(P, dtype=np.float64)[None, :, :]
    zb = zb - zb.max(axis=1, keepdims=True)      # softmax over the block's m tokens
    e = np.exp(zb)
    S = e / e.sum(axis=1, keepdims=True)
    out = (S * xb).sum(axis=1)
    return out


def pool_overlap(Xa, Za, Xb, Zb, m, P=None, prev=0):
    """Compressed entries of one sequence, the overlapped two-stream CSA form.

    [P2] V.1, equation C_i^comp: CSA projects two KV streams (a, b) with their own
    compression scores; entry i is the channel-wise weighted sum of stream a over block i
    and stream b over block i-1, so consecutive entries share a block boundary; the
    weights are the softmax pooling weights over the scores plus a positional bias.

    Readings (the pages give the sum, not the normalisation): one joint softmax per
    channel over the 2m logits [Za of block i + P[0:m]; Zb of block i-1 + P[m:2m]]; for
    the first block of a sequence there is no block i-1 and the softmax runs over stream
    a's m logits alone.  `prev` = 1 says that the arrays start one block before the first
    entry to emit (a cache append reads blocks i-1 and i): entry e then pools stream a
    block e+1 and stream b block e, and n//m - 1 entries are returned.

    Xa, Za, Xb, Zb: float arrays [n, c] (decoded).  P: [2m, c] or None.
    Returns [n // m - prev, c] fp64.
    """
    Xa, Za, Xb, Zb = (np.asarray(a, dtype=np.float64) for a in (Xa, Za, Xb, Zb))
    n, c = Xa.shape
    N = n // m
    Pa = np.zeros((m, c)) if P is None else np.asarray(P, dtype=np.float64)[:m]
    Pb = np.zeros((m, c)) if P is None else np.asarray(P, dtype=np.float64)[m:2 * m]
    out = np.empty((max(N - prev, 0), c))
    for e in range(N - prev):
        i = e + prev                                 # block of stream a
        logits = [Za[m * i:m * i + m] + Pa]
        values = [Xa[m * i:m * i + m]]
        if i >= 1:                                   # stream b over block i-1
            logits.append(Zb[m * (i - 1):m * i] + Pb)
            values.append(Xb[m * (i - 1):m * i])
        z = np.concatenate(logits, axis=0)           # [m or 2m, c]
        x = np.concatenate(values, axis=0)
        w = np.exp(z - z.max(axis=0, keepdims=True))
        S = w / w.sum(axis=0, keepdims=True)         # softmax over the tokens, per channel
        out[e] = (S * x).sum(axis=0)
    return out


# ----------------------------------------------------------------------------------------
# RMSNorm and partial RoPE ([P2] section IV: both branches normalise the queries and the
# compressed KV entries and rotate only the last 64 dimensions)
# ----------------------------------------------------------------------------------------
def rmsnorm(x, gamma=None, eps=1e-6):
    """Root-mean-square normalisation over the last axis.

    [P2] IV names RMSNorm on the queries and on the compressed KV entries without writing
    it out.  Reading: the usual definition, y = x / sqrt(mean(x^2) + eps) * gamma, with a
    per-channel gain gamma (1 when None) and eps given by the caller.
    """
    x = np.asarray(x, dtype=np.float64)
    ms = (x * x).mean(axis=-1, keepdims=True)
    y = x / np.sqrt(ms + eps)
    if gamma is not None:
        y = y * np.asarray(gamma, dtype=np.float64)
    return y


def rope_tail(x, pos, d_rope=64, theta=10000.0):
    """Rotary position embedding on the last d_rope dimensions of x.

    [P1] "The Code: RoPE Helpers": the rotated dimensions are taken as consecutive pairs
    (2i, 2i+1), each read as the complex number x[2i] + i x[2i+1] and multiplied by
    e^{i pos f_i} with f_i = theta^(-2i / d_rope), i < d_rope / 2 (theta = 10000 there).
    [P2] IV: only the last 64 dimensions carry RoPE; the others pass unchanged.

    x: [..., c]; pos: broadcastable to x.shape[:-1] (the position of every row).
    """
    x = np.array(x, dtype=np.float64)
    c = x.shape[-1]
    if d_rope == 0:
        return x
    i = np.arange(d_rope // 2, dtype=np.float64)
    f = theta ** (-2.0 * i / d_rope)                            # [d_rope/2]
    ang = np.asarray(pos, dtype=np.float64)[..., None] * f       # [..., d_rope/2]
    tail = x[..., c - d_rope:]
    z = tail[..., 0::2] + 1j * tail[..., 1::2]
    z = z * np.exp(1j * ang)
    out = x.copy()
    out[..., c - d_rope::2] = z.real
    out[..., c - d_rope + 1::2] = z.imag
    return out


def norm_rope(x, pos, gamma=None, eps=1e-6, d_rope=64, theta=10000.0):
    """RMSNorm, then RoPE on the last d_rope dimensions, row by row (x: [..., c])."""
    return rope_tail(rmsnorm(x, gamma, eps), pos, d_rope, theta)


def entry_positions(m, entry0, N):
    """Position a compressed entry carries for RoPE.  The pages do not say; reading: the
    first raw position of its block, m * s for entry s (entries entry0 .. entry0+N-1)."""
    return m * (entry0 + np.arange(N))


# ----------------------------------------------------------------------------------------
# visibility and window
# ----------------------------------------------------------------------------------------
def visible(p, m, N):
    """Number of compressed entries usable by the query at absolute position p.

    [P2] V.2 scores "each preceding compressed block"; [P3] section 9 keeps an incomplete
    block as an uncompressed tail.  Reading: block s is usable iff it is complete,
    m*(s+1) - 1 <= p, and it exists in the cache (s < N).
    """
    return int(min(N, (int(p) + 1) // m))


def window_positions(p, W):
    """Raw positions of the sliding window for the query at p.

    [P4] "Hybrid attention with CSA and HCA": both layer types also attend to the most
    recent 128 tokens uncompressed.  Reading: positions max(0, p-W+1) .. p, including the
    query's own token (causal, as the lower-triangular mask in [P1] CSA/HCA code).
    """
    lo = max(0, int(p) - W + 1)
    return np.arange(lo, int(p) + 1, dtype=np.int64)


# ----------------------------------------------------------------------------------------
# (a2) lightning indexer
# ----------------------------------------------------------------------------------------
def index_scores(qI, w, KI, V):
    """I_s = sum_h w_h * ReLU(qI_h . KI_s) for s < V.

    [P2] V.2, eq. I_{t,s}: sum over the n_ih indexer heads, each with its weight, of the
    ReLU of the indexer query / compressed indexer key dot product.  No scale is applied
    (the equation has none).

    qI: [n_ih, c_I], w: [n_ih], KI: [N, c_I] (decoded); returns [V] fp64.
    """
    qI = np.asarray(qI, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    KI = np.asarray(KI, dtype=np.float64)[:V]
    dots = KI @ qI.T                       # [V, n_ih]
    return np.maximum(dots, 0.0) @ w


# ----------------------------------------------------------------------------------------
# (a3) top-k selection
# ----------------------------------------------------------------------------------------
def topk(scores, k):
    """Indices of the k highest scores, ascending by index, padded with -1.

    [P2] V.2: keep the blocks whose score is among the top k.  [P1] CSA code and [P4]
    "Worked example": at most as many entries as exist are selected
    (K_eff = min(k, V)).  Reading for ties (pages silent): the lower index wins; -0.0
    counts as +0.0.  The output is a set, reported in ascending index order.
    """
    s = np.asarray(scores, dtype=np.float64).copy()
    s[s == 0.0] = 0.0                      # canonicalise -0.0
    V = s.shape[0]
    keff = min(int(k), V)
    idx = np.arange(V)
    order = np.lexsort((idx, -s))          # primary: score descending, then index ascending
    sel = np.sort(order[:keff])
    out = np.full((int(k),), -1, dtype=np.int64)
    out[:keff] = sel
    return out


# ----------------------------------------------------------------------------------------
# (a4, a5) attention over a row set (MQA: one shared K = V row per entry)
# ----------------------------------------------------------------------------------------
def attend(Q, rows, scale, sink=None):
    """O_h = sum_r softmax_r(scale * Q_h . row_r) row_r, and its log-sum-exp.

    [P2] I: softmax(QK^T / sqrt(c)) V; [P2] VI eq. o_{t,i}: key = value = compressed
    entries; [P2] IV / V.3: MQA, all heads share the rows.  Reading: compressed and
    window rows enter one joint softmax ([P4] step 5: ordinary attention over the union),
    without removing rows that appear both raw and inside a compressed entry.

    sink: optional [n_h] per-head learnable attention sink ([P2] IV names it for both
    branches).  Reading: a logit in the same units as scale * q . k that enters the
    softmax denominator only (a row of value zero), so
    O_h = sum_r e^{z_r} row_r / (e^{sink_h} + sum_r e^{z_r}) and the lse includes it.

    Q: [n_h, c]; rows: [R, c].  Returns (O [n_h, c], lse [n_h]).
    """
    Q = np.asarray(Q, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.float64)
    n_h = Q.shape[0]
    sk = None if sink is None else np.asarray(sink, dtype=np.float64).reshape(n_h, 1)
    if rows.shape[0] == 0:
        lse = np.full((n_h,), -np.inf) if sk is None else sk[:, 0].copy()
        return np.zeros_like(Q), lse
    s = (Q @ rows.T) * float(scale)        # [n_h, R]
    mx = s.max(axis=1, keepdims=True)
    if sk is not None:
        mx = np.maximum(mx, sk)
    e = np.exp(s - mx)
    l = e.sum(axis=1, keepdims=True)
    if sk is not None:
        l = l + np.exp(sk - mx)            # the sink's weight: denominator only
    O = (e @ rows) / l
    lse = (mx + np.log(l))[:, 0]
    return O, lse


def csa_rows(C, idx, win_src, win_pos, p, W):
    """Row set of one CSA query: the selected compressed entries plus the window.

    [P2] V.3: core attention over the selected blocks; [P4] steps 3-5: the selected
    entries plus the last 128 raw tokens.  idx holds ascending indices padded with -1.
    """
    idx = np.asarray(idx)
    sel = np.asarray(C)[idx[idx >= 0]]
    wp = window_positions(p, W) - int(win_pos)
    win = np.asarray(win_src)[wp]
    return np.concatenate([sel, win], axis=0)


def hca_rows(Ch, m_hca, win_src, win_pos, p, W):
    """Row set of one HCA query: every usable compressed entry plus the window.

    [P2] VI: dense attention over all compressed entries; [P1] "Heavily Compressed
    Attention (HCA)": no selection step.
    """
    Ch = np.asarray(Ch)
    V = visible(p, m_hca, Ch.shape[0])
    wp = window_positions(p, W) - int(win_pos)
    return np.concatenate([Ch[:V], np.asarray(win_src)[wp]], axis=0)


# ----------------------------------------------------------------------------------------
# grouped output projection ([P2] V.3)
# ----------------------------------------------------------------------------------------
def grouped_out_proj(O, Wg):
    """Grouped output projection of the concatenated head outputs.

    [P2] V.3: the c * n_h concatenated head outputs are split into g groups of heads, each
    group is projected by its own smaller matrix to d_g dimensions, and the g results are
    concatenated (d = g * d_g).  Readings: group gi holds the contiguous heads
    gi*n_h/g .. (gi+1)*n_h/g - 1, in head order; the outputs are concatenated in group
    order; there is no bias.  Weights are laid out as a linear layer's, out x in:
    Wg[gi] has shape [d_g, K_g] with K_g = n_h * c / g.

    O: [T, n_h, c] (or [T, n_h * c]); Wg: [g, d_g, K_g].  Returns [T, g * d_g] fp64.
    """
    O = np.asarray(O, dtype=np.float64)
    Wg = np.asarray(Wg, dtype=np.float64)
    T = O.shape[0]
    X = O.reshape(T, -1)                        # concatenated heads, head-major
    g, d_g, K_g = Wg.shape
    assert X.shape[1] == g * K_g
    out = np.empty((T, g * d_g))
    for gi in range(g):
        Xg = X[:, gi * K_g:(gi + 1) * K_g]      # this group's heads
        out[:, gi * d_g:(gi + 1) * d_g] = Xg @ Wg[gi].T
    return out


# ----------------------------------------------------------------------------------------
# entry counts
# ----------------------------------------------------------------------------------------
def entry_counts(n, m, m_hca, k, W):
    """(CSA entries stored, CSA entries attended, HCA entries) for a context of n tokens.

    [P4] "Worked example, step by step": stored = n/m + window, attended = min(n/m, k) +
    window, HCA = n/m' + window (stored = attended).  Whole blocks only (floor).
    """
    nc = n // m
    return nc + W, min(nc, k) + W, n // m_hca + W
