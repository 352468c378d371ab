"""The allocation-free indexer entry point (lightning_index_topk_noalloc) against the
workspace one (lightning_index_topk) and the oracle, through the C ABI: two calls in a
row on the shared scratch array, the second with a smaller input.  The two entry points
run the same kernels, so scores and selections must agree bit for bit; the selection is
also checked against oracle.topk of the GPU's own scores, and the scores against the
oracle's at 1e-3 relative."""
import math

import numpy as np
import pytest
import torch

import compressed_attention_compress_amd as lib
import oracle
from synthgen.configs import CONFIGS
from synthgen.host import make_problem
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    H.require_gpu()


def run_both(cfg):
    prob = make_problem(cfg)
    qI, w, KI = H.to_dev(prob["qI"]), H.to_dev(prob["w"]), H.key_buffer(prob)
    q_pos = H.to_dev(prob["q_pos"])
    B, Tq, n_ih, c_I = prob["qI"].shape
    N_c = prob["KI"].shape[1]
    k = cfg.k
    out = {}
    for name in ("workspace", "noalloc"):
        idx = torch.full((B, Tq, k), -7, dtype=torch.int32, device=H.DEV)
        sc = torch.full((B, Tq, k), float("nan"), dtype=torch.float32, device=H.DEV)
        alls = torch.full((B, Tq, N_c), float("nan"), dtype=torch.float32, device=H.DEV)
        if name == "workspace":
            ws_bytes = lib.lightning_index_topk_workspace_size(B, Tq, n_ih, N_c, k)
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device=H.DEV)
            lib.lightning_index_topk(qI, w, KI, cfg.idx_dtype, q_pos, cfg.m, B, Tq, n_ih, c_I, N_c, k,
                                     idx, sc, alls, ws, ws_bytes)
        else:
            lib.lightning_index_topk_noalloc(qI, w, KI, cfg.idx_dtype, q_pos, cfg.m, B, Tq, n_ih, c_I,
                                             N_c, k, idx, sc, alls)
        torch.cuda.synchronize()
        out[name] = (idx.cpu().numpy(), sc.cpu().numpy(), alls.cpu().numpy())
    return prob, out


def check_against_oracle(prob, idx, alls):
    cfg = prob["cfg"]
    qI = oracle.decode(prob["qI"], cfg.idx_dtype)
    KI = oracle.decode(prob["KI"], cfg.idx_dtype)
    B, Tq = qI.shape[:2]
    for b in range(B):
        for t in range(Tq):
            V = oracle.visible(int(prob["q_pos"][b]) + t, cfg.m, KI.shape[1])
            ref = oracle.index_scores(qI[b, t], prob["w"][b, t], KI[b], V)
            g = alls[b, t, :V].astype(np.float64)
            rms = math.sqrt(float(np.mean(ref * ref)))
            assert np.all(np.abs(g - ref) <= 1e-3 * np.abs(ref) + 1e-6 * rms), (b, t)
            assert np.array_equal(idx[b, t], oracle.topk(g, cfg.k)), (b, t)


CASES = [
    # first call: a Pro-shaped decode batch; second: a smaller Flash-shaped one
    ("pro_decode", CONFIGS[5].scaled(kind="index_decode", B=3, n=4 * 20000 + 3, seed=91, plants=16)),
    ("flash_decode_small", CONFIGS[3].scaled(kind="index_decode", B=2, n=4 * 1500 + 1, seed=92, plants=4)),
]


def test_noalloc_matches_workspace_entry_point_two_calls():
    for label, cfg in CASES:
        print(f"[noalloc {label}: B={cfg.B} n={cfg.n} k={cfg.k}]", flush=True)
        prob, out = run_both(cfg)
        (i0, s0, a0), (i1, s1, a1) = out["workspace"], out["noalloc"]
        assert np.array_equal(i0, i1), label
        assert np.array_equal(s0.view(np.uint32), s1.view(np.uint32)), label
        V = [oracle.visible(int(prob["q_pos"][b]), cfg.m, prob["KI"].shape[1]) for b in range(cfg.B)]
        for b in range(cfg.B):
            assert np.array_equal(a0[b, :, :V[b]].view(np.uint32), a1[b, :, :V[b]].view(np.uint32)), label
        check_against_oracle(prob, i1, a1)


def test_noalloc_rejects_oversize():
    B, N_c = 64, 262144  # needs about 68 MiB of scratch
    d = torch.zeros(16, dtype=torch.uint8, device=H.DEV)
    with pytest.raises(lib.CsaHcaError) as e:
        lib.lightning_index_topk_noalloc(d, d, d, 2, d, 4, B, 1, 64, 128, N_c, 1024, d, None, None)
    assert e.value.status == lib.EWORKSPACE
