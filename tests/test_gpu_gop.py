"""GPU parity of the grouped output projection (grouped_out_proj) against the CPU oracle,
on identical bf16 input bytes.

Tolerance per output: |d| <= ulp_bf16(ref) + K_g * 2^-24 * sum_k |o_k w_k| (the fp32
accumulation bound over K_g products, plus the final rounding); in addition at most 1% of
the outputs may differ from the oracle by more than one bf16 ulp.
"""
import numpy as np
import pytest
import torch

import compressed_attention_compress_amd as lib
import oracle
from synthgen.configs import BF16
from synthgen.host import encode
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    H.require_gpu()


def bf16_ulp(x):
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def make(rng, T, g, K_g, d_g, pad_o=0):
    o = encode(rng.standard_normal((T, g * K_g + pad_o), dtype=np.float32), BF16)
    w = encode(rng.standard_normal((g, d_g, K_g), dtype=np.float32) / np.sqrt(K_g), BF16)
    return o, w


def check(got, o, w, g, K_g, rows=None):
    O = oracle.decode(o if rows is None else o[rows], BF16)[:, :g * K_g]
    Wd = oracle.decode(w, BF16)
    ref = oracle.grouped_out_proj(O, Wd)
    cond = oracle.grouped_out_proj(np.abs(O), np.abs(Wd))
    d = np.abs(got - ref)
    assert not (d > bf16_ulp(ref) + K_g * 2.0 ** -24 * cond).any(), f"max |d| {d.max()}"
    assert (d > bf16_ulp(ref)).mean() <= 0.01


def run(o, w, T, g, K_g, d_g, pad_y=0):
    do, dw = H.to_dev(o), H.to_dev(w)
    ldy = g * d_g + pad_y
    y = H.empty((T, ldy), BF16)
    lib.grouped_out_proj(do, dw, y, T, g, K_g, d_g, o.shape[1], ldy, BF16)
    torch.cuda.synchronize()
    return oracle.decode(H.to_host_codes(y, BF16), BF16)[:, :g * d_g]


@pytest.mark.parametrize("T,g,K_g,d_g,pad", [
    (1, 16, 4096, 512, 0),     # a single decode token, Pro-shaped
    (4, 8, 512, 128, 0),
    (17, 2, 128, 48, 8),       # ragged tokens, columns not a multiple of 128, padded rows
    (64, 1, 1024, 16, 0),      # four full 16-token tiles
    (150, 3, 256, 48, 0),      # many tokens with d_g % 128 != 0: 64-token groups
    (65, 2, 512, 256, 0),      # the tile kernel, 65 tokens in one 256-token tile
    (300, 2, 256, 256, 16),    # ragged last tile, padded rows
    (1000, 2, 384, 512, 0),    # several tiles; K_g not a multiple of 256
    (520, 1, 128, 128, 0),     # d_g % 256 != 0: the few-token kernel per 64 tokens
])
def test_gop_parity(T, g, K_g, d_g, pad):
    print(f"[gop T={T} g={g} K_g={K_g} d_g={d_g} pad={pad}]", flush=True)
    rng = np.random.default_rng(T * 7 + g)
    o, w = make(rng, T, g, K_g, d_g, pad)
    got = run(o, w, T, g, K_g, d_g, pad)
    check(got, o, w, g, K_g)


def test_gop_full_prefill_sampled():
    """The prefill shape (8192 tokens of 64 heads x 512 in 8 groups of 4096, d_g = 512) in
    the launch configuration the benchmark times; 96 sampled tokens checked."""
    print("[gop prefill 8192 sampled]", flush=True)
    rng = np.random.default_rng(5)
    T, g, K_g, d_g = 8192, 8, 4096, 512
    o, w = make(rng, T, g, K_g, d_g)
    got = run(o, w, T, g, K_g, d_g)
    rows = np.unique(np.r_[0, 255, 256, T - 1, rng.integers(0, T, 92)])
    check(got[rows], o, w, g, K_g, rows=rows)


def test_gop_tokens_independent():
    """A token's output does not depend on which other tokens share the call (bitwise),
    across the few-token and the tile kernel."""
    rng = np.random.default_rng(9)
    g, K_g, d_g = 4, 512, 256
    o, w = make(rng, 300, g, K_g, d_g)
    big = run(o, w, 300, g, K_g, d_g)
    small = run(o[:5], w, 5, g, K_g, d_g)
    # different kernels: equal within the tolerance; the tile kernel against itself: bitwise
    check(small, o[:5], w, g, K_g)
    again = run(o[:200], w, 200, g, K_g, d_g)
    np.testing.assert_array_equal(again, big[:200])
