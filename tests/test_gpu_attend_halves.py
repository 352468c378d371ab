"""csa_attend_begin / _end and hca_attend_begin / _end against the one-call csa_attend_ex /
hca_attend_ex: the same bits in out and lse, with the merge on another stream than the
attention (an event between them), at shapes whose launch plans have several splits
(the merge runs in _end) and one split (_end does nothing), with the query norm and a
sink, and on the float32 path.  The one-call results are held to the oracle by the
other attention tests."""
import pytest
import torch

import compressed_attention_compress_amd as lib
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

BF16, F32 = 1, 0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    H.require_gpu()


CASES = {
    # name: (csa, B, n_h, c, N (cache entries), k, W, Tq, dtype, q_norm)
    "hca_decode_splits": (False, 2, 64, 512, 2048, 0, 128, 1, BF16, 1),
    "csa_decode_splits": (True, 4, 128, 512, 8192, 512, 128, 1, BF16, 0),
    "hca_prefill_splits": (False, 1, 64, 512, 64, 0, 128, 16, BF16, 1),
    "hca_decode_one_split": (False, 2, 64, 512, 16, 0, 16, 1, BF16, 1),
    "csa_f32": (True, 1, 8, 64, 1024, 64, 128, 1, F32, 0),
}


@pytest.mark.parametrize("name", list(CASES))
def test_halves_equal_one_call(name):
    csa, B, n_h, c, N, k, W, Tq, dt, qn = CASES[name]
    print(f"[attend halves {name}]", flush=True)
    g = torch.Generator(device="cuda").manual_seed(17 + len(name))
    tdt = torch.bfloat16 if dt == BF16 else torch.float32
    m = 4 if csa else 128
    n = N * m                        # raw tokens; the query is the last
    L = W + Tq + 7                   # window source rows (a few older ones too)
    q = torch.randn((B, Tq, n_h, c), generator=g, device="cuda").to(tdt)
    ckv = (torch.randn((B, N, c), generator=g, device="cuda") / 8).to(tdt)
    win = (torch.randn((B, L, c), generator=g, device="cuda") / 8).to(tdt)
    q_pos = torch.full((B,), n - Tq, dtype=torch.int32, device="cuda")
    win_pos = torch.full((B,), n - L, dtype=torch.int32, device="cuda")
    sink = torch.randn((n_h,), generator=g, device="cuda") if dt == BF16 else None
    gam = (torch.rand((c,), generator=g, device="cuda") + 0.5) if qn else None
    nr = (sink, gam, qn, 64 if qn else 0, 1e-6, 1e4)
    scale = c ** -0.5
    if csa:
        idx = torch.stack([torch.randperm(N, generator=g, device="cuda")[:k].sort().values
                           for _ in range(B * Tq)]).view(B, Tq, k).to(torch.int32).contiguous()
        ws_b = lib.load().csa_attend_workspace_size(B, Tq, n_h, c, k, W)
        args = (q, ckv, idx, win, win_pos, q_pos, B, Tq, n_h, c, N, k, L, W, scale, *nr, dt)
        one, begin, end = lib.csa_attend_ex, lib.csa_attend_begin, lib.csa_attend_end
    else:
        ws_b = lib.load().hca_attend_workspace_size(B, Tq, n_h, c, N, W)
        args = (q, ckv, win, win_pos, q_pos, m, B, Tq, n_h, c, N, L, W, scale, *nr, dt)
        one, begin, end = lib.hca_attend_ex, lib.hca_attend_begin, lib.hca_attend_end
    ws = torch.empty((max(ws_b, 256),), dtype=torch.uint8, device="cuda")
    o1 = torch.empty((B, Tq, n_h, c), dtype=tdt, device="cuda")
    o2 = torch.full_like(o1, 3)
    l1 = torch.empty((B, Tq, n_h), dtype=torch.float32, device="cuda")
    l2 = torch.full_like(l1, 5.0)
    one(*args, o1, l1, ws, ws_b)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    done = torch.cuda.Event()
    with torch.cuda.stream(s1):
        begin(*args, o2, l2, ws, ws_b)
        done.record(s1)
    s2.wait_event(done)
    with torch.cuda.stream(s2):
        end(*args, o2, l2, ws, ws_b)
    torch.cuda.synchronize()
    iv = torch.int16 if dt == BF16 else torch.int32
    assert torch.equal(o1.view(iv), o2.view(iv)), name
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), name
