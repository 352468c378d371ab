"""The C-ABI library loads, exports every declared symbol, and rejects invalid arguments on
the host before any HIP call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

import compressed_attention_compress_amd as lib
from compressed_attention_compress_amd import EINVAL, ENOTSUP, EWORKSPACE
from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "csahca.h")
FAKE = 1 << 20  # an aligned, never-dereferenced address: validation fails before any use


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\*?\s*([a-z_]+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("csa_compress", "hca_compress", "lightning_index_topk", "csa_attend",
                 "hca_attend", "lightning_index_topk_workspace_size",
                 "csa_attend_workspace_size", "hca_attend_workspace_size", "csahca_last_error"):
        assert want in names


def test_library_exports_every_declared_symbol():
    h = ctypes.CDLL(lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(h, name), name
    # the binding wraps the same set
    assert set(declared_functions()) <= set(lib._SIGNATURES)
    assert lib.version() >= 10000


def _status(fn, *args):
    return getattr(lib.load(), fn)(*args)


def test_pool_validation():
    L = lib.load()
    assert L.csa_compress(None, None, None, None, 1, 8, 8, 4, 1, 64, 16, None) == EINVAL
    assert "non-NULL" in lib.last_error()
    assert L.hca_compress(FAKE, FAKE, None, FAKE, 1, 8, 12, 4, 1, 96, 24, None) == EINVAL  # c % 8
    assert L.csa_compress(FAKE, FAKE, None, FAKE, 1, 8, 8, 4, 2, 64, 16, None) == ENOTSUP  # fp8
    assert L.csa_compress(FAKE, FAKE, None, FAKE, 1, 8, 8, 4, 1, 32, 16, None) == EINVAL   # stride
    assert L.csa_compress(FAKE + 4, FAKE, None, FAKE, 1, 8, 8, 4, 1, 64, 16, None) == EINVAL
    assert L.csa_compress(FAKE, FAKE, None, FAKE, 1, 8, 8, 0, 1, 64, 16, None) == EINVAL   # m
    # fewer tokens than one block: nothing to do, pointers may be NULL
    assert L.csa_compress(None, None, None, None, 1, 3, 8, 4, 1, 24, 0, None) == 0
    # the pair: either side's error is reported (nothing enqueued); both sides empty is a no-op
    pr = L.csahca_compress_pair
    assert pr(FAKE, FAKE, FAKE, 8, 4, 64, 16, None, FAKE, FAKE, 256, 128, 2048, 16, 1, 8, 1,
              None) == EINVAL
    assert "non-NULL" in lib.last_error()
    assert pr(FAKE, FAKE, FAKE, 8, 4, 32, 16, FAKE, FAKE, FAKE, 256, 128, 2048, 16, 1, 8, 1,
              None) == EINVAL  # side a stride
    assert pr(FAKE, FAKE, FAKE, 8, 4, 64, 16, FAKE, FAKE, FAKE, 256, 0, 2048, 16, 1, 8, 1,
              None) == EINVAL  # side b m
    assert pr(FAKE, FAKE, FAKE, 8, 4, 64, 16, FAKE, FAKE, FAKE, 256, 128, 2048, 16, 1, 8, 2,
              None) == ENOTSUP  # dtype
    assert pr(None, None, None, 3, 4, 24, 0, None, None, None, 100, 128, 800, 0, 1, 8, 1,
              None) == 0
    # the pair with the norm: the pair's checks, then the norm's (each side its own gain and
    # first entry)
    pn = L.csahca_compress_pair_norm_rope
    ok = [FAKE, FAKE, None, FAKE, 8, 4, 0, 64, 16, FAKE, FAKE, None, FAKE, 256, 128, 0, 2048, 16, 1, 8,
          8, 1e-6, 1e4, 1, None]
    bad_cases = [(7, 32, EINVAL),          # side a stride
                 (14, 0, EINVAL),          # side b m
                 (20, 12, EINVAL),         # d_rope % 8
                 (20, 16, EINVAL),         # d_rope > c
                 (21, -1.0, EINVAL),       # eps
                 (22, 0.0, EINVAL),        # theta
                 (6, -1, EINVAL),          # entry0_a
                 (15, -3, EINVAL),         # entry0_b
                 (2, FAKE + 4, EINVAL),    # gamma_a alignment
                 (23, 2, ENOTSUP)]         # dtype
    for i, v, want in bad_cases:
        args = list(ok)
        args[i] = v
        assert pn(*args) == want, (i, v)
        assert "csahca_compress_pair_norm_rope" in lib.last_error()
    # ... and with the window rows: the pair's checks, then the rows' (T >= 0; with T > 0
    # every row pointer set and aligned, strides >= T*c and multiples of 8)
    pr_rows = L.csahca_compress_pair_norm_rope_rows
    rows_ok = [1, FAKE, FAKE, None, 8, 8, FAKE, FAKE, None, 8, 8]
    ok_r = ok[:-1] + rows_ok + [None]
    for i, v, want in bad_cases[:3]:
        args = list(ok_r)
        args[i] = v
        assert pr_rows(*args) == want, (i, v)
    R0 = len(ok) - 1  # index of T
    for off, v, want in [(0, -1, EINVAL),         # T
                         (1, None, EINVAL),        # row_x_a
                         (7, None, EINVAL),        # row_y_b
                         (2, FAKE + 4, EINVAL),    # row_y_a alignment
                         (4, 7, EINVAL),           # row_x_bstride_a below T*c
                         (10, 12, EINVAL)]:        # row_y_bstride_b not a multiple of 8
        args = list(ok_r)
        args[R0 + off] = v
        assert pr_rows(*args) == want, (off, v)
        assert "csahca_compress_pair_norm_rope_rows" in lib.last_error()
    # overlapped form: prev is 0 or 1, stream b pointers are required, an append of one
    # block with prev = 1 emits nothing
    ov = L.csa_compress_overlap
    assert ov(FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 8, 8, 4, 2, 1, 64, 16, None) == EINVAL
    assert ov(FAKE, FAKE, None, FAKE, None, FAKE, 1, 8, 8, 4, 0, 1, 64, 16, None) == EINVAL
    assert ov(FAKE, FAKE, FAKE + 4, FAKE, None, FAKE, 1, 8, 8, 4, 0, 1, 64, 16, None) == EINVAL
    assert ov(FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 8, 8, 4, 0, 2, 64, 16, None) == ENOTSUP
    assert ov(None, None, None, None, None, None, 1, 4, 8, 4, 1, 1, 32, 0, None) == 0


def test_indexer_noalloc_validation():
    """The allocation-free variant checks shapes, then its scratch bound, before any HIP
    call (no GPU needed for these)."""
    L = lib.load()
    fn = L.lightning_index_topk_noalloc
    # a call whose workspace would exceed the built scratch array is refused
    big = [FAKE, FAKE, FAKE, 2, FAKE, 4, 64, 1, 64, 128, 262144, 1024, FAKE, None, None, None]
    assert L.lightning_index_topk_workspace_size(64, 1, 64, 262144, 1024) > (32 << 20)
    assert fn(*big) == EWORKSPACE
    assert "scratch" in lib.last_error()
    bad = list(big)
    bad[0] = None
    assert fn(*bad) == EINVAL
    bad = list(big)
    bad[9] = 96  # c_I
    assert fn(*bad) == ENOTSUP


def test_indexer_validation():
    L = lib.load()
    B, Tq, n_ih, c_I, N_c, k = 2, 1, 64, 128, 1000, 64
    ws = L.lightning_index_topk_workspace_size(B, Tq, n_ih, N_c, k)
    NG = -(-N_c // 16)
    up = lambda x: -(-x // 256) * 256
    # one 32-bit maximum key per group of 16 entries, the fp32 scores; a decode call adds
    # each chunk's bound and zero-padded list (the plan for 1000 entries and k = 64 over
    # two queries: 4 chunks of 256, lists of up to 64 keys) and one path word per query
    base = up(B * NG * 4) + up(B * N_c * 4)
    assert ws == base + up(B * 128 * 8) + up(B * 4 * 64 * 8) + up(B * 4)
    # a prefill shape has no chunk lists
    assert L.lightning_index_topk_workspace_size(B, 3, n_ih, N_c, k) == up(3 * B * NG * 4) + up(3 * B * N_c * 4)
    args = [FAKE, FAKE, FAKE, 2, FAKE, 4, B, Tq, n_ih, c_I, N_c, k, FAKE, None, None]
    assert L.lightning_index_topk(*args, FAKE, ws - 1, None) == EWORKSPACE
    assert L.lightning_index_topk(*args, None, ws, None) == EWORKSPACE
    bad = list(args)
    bad[8] = 48 + 8  # n_ih not a multiple of 16
    assert L.lightning_index_topk(*bad, FAKE, ws, None) == ENOTSUP
    for n_ih_bad in (48, 80, 96, 112, 256):  # FP8 / MX FP4 scoring is built for 16, 32, 64, 128 heads
        bad[8] = n_ih_bad
        assert L.lightning_index_topk(*bad, FAKE, ws, None) == ENOTSUP
    bad = list(args)
    bad[9] = 96  # c_I
    assert L.lightning_index_topk(*bad, FAKE, ws, None) == ENOTSUP
    bad = list(args)
    bad[11] = 2048  # k
    assert L.lightning_index_topk(*bad, FAKE, ws, None) == ENOTSUP
    bad = list(args)
    bad[10] = 262144 + 16  # N_c
    assert L.lightning_index_topk(*bad, FAKE, ws, None) == ENOTSUP
    bad = list(args)
    bad[0] = None
    assert L.lightning_index_topk(*bad, FAKE, ws, None) == EINVAL
    bad = list(args)
    bad[3] = 1  # bf16 indexer keys are not a supported type
    assert L.lightning_index_topk(*bad, FAKE, ws, None) == ENOTSUP
    assert L.lightning_index_select(None, FAKE, 4, B, Tq, N_c, k, FAKE, None, FAKE, ws, None) == EINVAL
    assert L.lightning_index_score(*args[:12], None, FAKE, ws, None) == EINVAL
    # the indexer with the CSA block pooled beside it: both calls' rules, checked up front
    pool = [FAKE, FAKE, FAKE, 4 * N_c, 512, 1, 0, 0]
    fused = L.lightning_index_topk_csa_compress
    assert fused(*args, FAKE, ws - 1, *pool, None) == EWORKSPACE
    bad = list(pool)
    bad[0] = None  # kv
    assert fused(*args, FAKE, ws, *bad, None) == EINVAL
    bad = list(pool)
    bad[4] = 7  # c not a multiple of 8
    assert fused(*args, FAKE, ws, *bad, None) == EINVAL
    bad = list(pool)
    bad[3] = -1  # n
    assert fused(*args, FAKE, ws, *bad, None) == EINVAL
    bad = list(pool)
    bad[5] = 9  # dtype
    assert fused(*args, FAKE, ws, *bad, None) == ENOTSUP
    # ... and with the norm and the window rows
    nrp = [FAKE, FAKE, FAKE, FAKE, 4 * N_c, 512, 0, 64, 1e-6, 10000.0, 1, 0, 0]
    rows = [1, FAKE, FAKE, FAKE, 512, 512]
    fnr = L.lightning_index_topk_csa_compress_norm_rope_rows
    assert fnr(*args, FAKE, ws - 1, *nrp, *rows, None) == EWORKSPACE
    bad = list(nrp)
    bad[7] = 60  # d_rope not a multiple of 8
    assert fnr(*args, FAKE, ws, *bad, *rows, None) == EINVAL
    bad = list(nrp)
    bad[6] = -1  # entry0
    assert fnr(*args, FAKE, ws, *bad, *rows, None) == EINVAL
    bad = list(nrp)
    bad[9] = 0.0  # theta
    assert fnr(*args, FAKE, ws, *bad, *rows, None) == EINVAL
    bad = list(nrp)
    bad[2] = FAKE + 4  # gamma not 16-byte aligned
    assert fnr(*args, FAKE, ws, *bad, *rows, None) == EINVAL
    badr = list(rows)
    badr[2] = None  # a row source without its destination
    assert fnr(*args, FAKE, ws, *nrp, *badr, None) == EINVAL
    badr = list(rows)
    badr[4] = 256  # row stride below T * c
    assert fnr(*args, FAKE, ws, *nrp, *badr, None) == EINVAL
    badr = list(rows)
    badr[0] = -1  # T
    assert fnr(*args, FAKE, ws, *nrp, *badr, None) == EINVAL


def test_attend_workspace_sizes_every_head_count():
    """The workspace queries run the launch plan on the host for any head count (float32
    calls take any n_h; bfloat16 calls any multiple of 16 up to 128), with no division by
    an empty head group.  A decode call with one query splits its rows over workgroups,
    so it needs a partial-output workspace."""
    L = lib.load()
    for n_h in list(range(1, 40)) + [48, 64, 72, 80, 96, 112, 128, 200]:
        for Tq in (1, 3, 7, 8192):
            assert L.csa_attend_workspace_size(1, Tq, n_h, 512, 512, 128) >= 0
            assert L.hca_attend_workspace_size(1, Tq, n_h, 512, 1024, 128) >= 0
    for n_h in range(16, 129, 16):
        assert L.csa_attend_workspace_size(1, 1, n_h, 512, 512, 128) > 0
        assert L.hca_attend_workspace_size(1, 1, n_h, 512, 1024, 128) > 0


def test_attend_validation():
    L = lib.load()
    B, Tq, n_h, c, k, W = 2, 1, 64, 512, 512, 128
    ws = L.csa_attend_workspace_size(B, Tq, n_h, c, k, W)
    assert ws > 0  # decode with few queries splits the rows
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, B, Tq, n_h, c, 4096, k, 4096, W]
    assert L.csa_attend(*base, 0.04, 1, FAKE, None, FAKE, ws - 1, None) == EWORKSPACE
    assert L.csa_attend(*base, -1.0, 1, FAKE, None, FAKE, ws, None) == EINVAL
    bad = list(base)
    bad[9] = 256
    assert L.csa_attend(*bad, 0.04, 1, FAKE, None, FAKE, ws, None) == ENOTSUP  # bf16 needs 512
    bad = list(base)
    bad[8] = 72
    assert L.csa_attend(*bad, 0.04, 1, FAKE, None, FAKE, ws, None) == ENOTSUP  # n_h % 16
    bad = list(base)
    bad[2] = None
    assert L.csa_attend(*bad, 0.04, 1, FAKE, None, FAKE, ws, None) == EINVAL
    assert L.csa_attend(*base, 0.04, 2, FAKE, None, FAKE, ws, None) == ENOTSUP  # fp8 attention
    wh = L.hca_attend_workspace_size(B, Tq, n_h, c, 1024, W)
    hb = [FAKE, FAKE, FAKE, FAKE, FAKE, 128, B, Tq, n_h, c, 1024, 4096, W]
    assert L.hca_attend(*hb, 0.04, 1, FAKE, None, FAKE, wh - 1, None) == EWORKSPACE
    hbad = list(hb)
    hbad[5] = 0
    assert L.hca_attend(*hbad, 0.04, 1, FAKE, None, FAKE, wh, None) == EINVAL
    # float32 path limits
    assert L.hca_attend(FAKE, FAKE, FAKE, FAKE, FAKE, 128, B, Tq, 8, 512, 1024, 4096, W, 0.1, 0,
                        FAKE, None, FAKE, wh, None) == ENOTSUP
    # the sink variants check the same arguments (the sink itself may be NULL)
    assert L.csa_attend_sink(*base, 0.04, FAKE, 1, FAKE, None, FAKE, ws - 1, None) == EWORKSPACE
    assert L.csa_attend_sink(*base, -1.0, None, 1, FAKE, None, FAKE, ws, None) == EINVAL
    assert "csa_attend_sink" in lib.last_error()
    assert L.hca_attend_sink(*hbad, 0.04, FAKE, 1, FAKE, None, FAKE, wh, None) == EINVAL
    assert L.hca_attend_sink(*hb, 0.04, FAKE, 2, FAKE, None, FAKE, wh, None) == ENOTSUP
    # the _ex variants: the same checks, then the query norm arguments
    nr = [FAKE, None, 1, 64, 1e-6, 1e4]        # sink, q_gamma, q_norm, d_rope, eps, theta
    assert L.csa_attend_ex(*base, 0.04, *nr, 1, FAKE, None, FAKE, ws - 1, None) == EWORKSPACE
    for i, v in [(2, 2), (3, 136), (3, 60), (3, -8), (4, -1.0), (5, 0.0), (5, float("inf"))]:
        bad = list(nr)
        bad[i] = v
        assert L.csa_attend_ex(*base, 0.04, *bad, 1, FAKE, None, FAKE, ws, None) == EINVAL, (i, v)
        assert "csa_attend_ex" in lib.last_error()
        assert L.hca_attend_ex(*hb, 0.04, *bad, 1, FAKE, None, FAKE, wh, None) == EINVAL, (i, v)
    # the query norm is a bfloat16 path; q_norm = 0 leaves float32 to its own limits
    f32 = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, B, Tq, 8, 64, 4096, 64, 4096, 16]
    assert L.csa_attend_ex(*f32, 0.04, *nr, 0, FAKE, None, FAKE, ws, None) == ENOTSUP
    assert "bfloat16" in lib.last_error()
    assert L.hca_attend_ex(*hbad, 0.04, None, None, 0, 64, 1e-6, 1e4, 1, FAKE, None, FAKE, wh,
                           None) == EINVAL  # m, checked before the norm arguments
    # the two halves (_begin / _end) check exactly what the _ex call checks
    for half in ("begin", "end"):
        cfn, hfn = getattr(L, f"csa_attend_{half}"), getattr(L, f"hca_attend_{half}")
        assert cfn(*base, 0.04, *nr, 1, FAKE, None, FAKE, ws - 1, None) == EWORKSPACE
        assert f"csa_attend_{half}" in lib.last_error()
        assert hfn(*hb, 0.04, *nr, 1, FAKE, None, FAKE, wh - 1, None) == EWORKSPACE
        assert cfn(*base, -1.0, *nr, 1, FAKE, None, FAKE, ws, None) == EINVAL
        assert hfn(*hbad, 0.04, *nr, 1, FAKE, None, FAKE, wh, None) == EINVAL
        for i, v in [(2, 2), (3, 60), (4, -1.0)]:
            bad = list(nr)
            bad[i] = v
            assert cfn(*base, 0.04, *bad, 1, FAKE, None, FAKE, ws, None) == EINVAL, (half, i, v)
            assert hfn(*hb, 0.04, *bad, 1, FAKE, None, FAKE, wh, None) == EINVAL, (half, i, v)


def test_binding_raises_with_message():
    with pytest.raises(lib.CsaHcaError) as e:
        lib.csa_compress(None, None, None, None, 1, 8, 8, 4, 1, 64, 16, stream=0)
    assert e.value.status == EINVAL and "non-NULL" in str(e.value)


def test_kv_cache_validation():
    """Ring size agrees with the simulator's rule; invalid appends and forks are refused on
    the host."""
    from oracle import kvcache
    L = lib.load()
    for W, m in ((128, 4), (128, 128), (0, 4), (5, 3), (128, 1), (1, 4096)):
        assert L.csahca_kv_ring_rows(W, m) == kvcache.ring_rows(W, m)
    assert L.csahca_kv_ring_rows(-1, 4) == 0 and L.csahca_kv_ring_rows(128, 0) == 0
    R = kvcache.ring_rows(128, 4)
    c = 512
    ok = [FAKE, FAKE, FAKE, FAKE, FAKE, None, 2, 6, 10, c, 4, 128, 1, 10 * c, 2 * R * c, 4 * c, None]
    ap = L.csahca_kv_append

    def with_(i, v):
        a = list(ok)
        a[i] = v
        return a
    assert ap(*with_(12, 2)) == ENOTSUP                 # fp8 raw tokens
    assert ap(*with_(9, 12)) == EINVAL                  # c % 8
    assert ap(*with_(14, 2 * R * c - 8)) == EINVAL      # ring too small
    assert ap(*with_(15, 3 * c)) == EINVAL              # entries stride below (6+10)/4 = 4
    assert ap(*with_(13, 9 * c)) == EINVAL              # new tokens stride
    assert ap(*with_(3, FAKE + 4)) == EINVAL            # alignment
    assert ap(*with_(2, None)) == EINVAL                # blocks complete, no entries
    assert "entries" in lib.last_error()
    assert ap(*with_(8, 0)) == 0                        # nothing appended: nothing done
    fk = L.csahca_kv_fork
    fok = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4, c, 4, 128, 1, 2 * R * c, 4 * c, None]
    f = list(fok)
    f[12] = 2 * R * c - 8
    assert fk(*f) == EINVAL
    f = list(fok)
    f[2] = None
    assert fk(*f) == EINVAL
    f = list(fok)
    f[11] = 2
    assert fk(*f) == ENOTSUP
    f = list(fok)
    f[13] = 3 * c
    assert fk(*f) == EINVAL


def test_norm_rope_validation():
    L = lib.load()
    nr = L.csahca_norm_rope
    ok = [FAKE, FAKE, None, None, 2, 3, 4, 512, 1, 64, 1e-6, 10000.0, 1, 1, 3 * 4 * 512, 3 * 4 * 512,
          None]

    def with_(i, v, base=ok):
        a = list(base)
        a[i] = v
        return a
    assert nr(*with_(7, 96)) == EINVAL       # c / 8 = 12 is not a power of two
    assert nr(*with_(7, 1024)) == EINVAL     # c / 8 > 64
    assert nr(*with_(9, 60)) == EINVAL       # d_rope % 8
    assert nr(*with_(9, 520)) == EINVAL      # d_rope > c
    assert nr(*with_(10, -1.0)) == EINVAL    # eps
    assert nr(*with_(11, 0.0)) == EINVAL     # theta
    assert nr(*with_(12, 2)) == EINVAL       # norm flag
    assert nr(*with_(13, 2)) == ENOTSUP      # fp8 rows
    assert nr(*with_(1, FAKE + 8)) == EINVAL  # alignment
    assert nr(*with_(2, FAKE + 4)) == EINVAL  # gain alignment
    assert nr(*with_(0, None)) == EINVAL
    assert nr(*with_(14, 3 * 4 * 512 - 8)) == EINVAL  # stride below T*H*c
    assert nr(*with_(15, 3 * 4 * 512 + 4)) == EINVAL  # stride not a multiple of 8
    assert nr(*with_(5, 0)) == 0             # no rows
    cp = L.csahca_compress_norm_rope
    cok = [FAKE, FAKE, None, None, FAKE, 1, 8, 512, 4, 0, 64, 1e-6, 10000.0, 1, 8 * 512, 2 * 512,
           None]
    assert cp(*with_(7, 96, cok)) == EINVAL
    assert cp(*with_(10, 12, cok)) == EINVAL
    assert cp(*with_(9, -1, cok)) == EINVAL  # entry0
    assert cp(*with_(3, FAKE + 4, cok)) == EINVAL  # gain alignment
    assert "csahca_compress_norm_rope" in lib.last_error()
    assert cp(*with_(13, 2, cok)) == ENOTSUP
    ov = L.csa_compress_overlap_norm_rope
    ook = [FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 1, 8, 512, 4, 0, 0, 64, 1e-6, 10000.0, 1,
           8 * 512, 2 * 512, None]
    assert ov(*with_(12, -3, ook)) == EINVAL
    assert ov(*with_(11, 2, ook)) == EINVAL  # prev
    assert ov(*with_(2, None, ook)) == EINVAL


def test_grouped_out_proj_validation():
    L = lib.load()
    gp = L.grouped_out_proj
    ok = [FAKE, FAKE, FAKE, 4, 16, 4096, 512, 16 * 4096, 16 * 512, 1, None]

    def with_(i, v):
        a = list(ok)
        a[i] = v
        return a
    assert gp(*with_(9, 0)) == ENOTSUP            # fp32
    assert gp(*with_(5, 4096 + 64)) == ENOTSUP    # K_g % 128
    assert gp(*with_(6, 520)) == ENOTSUP          # d_g % 16
    assert gp(*with_(7, 16 * 4096 - 8)) == EINVAL  # ldo
    assert gp(*with_(8, 16 * 512 + 4)) == EINVAL  # ldy % 8
    assert gp(*with_(0, None)) == EINVAL
    assert gp(*with_(2, FAKE + 2)) == EINVAL      # alignment
    assert gp(*with_(3, -1)) == EINVAL
    assert gp(*with_(3, 0)) == 0                  # no tokens
