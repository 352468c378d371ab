#!/usr/bin/env python3
"""Throughput of the CSA + HCA hot path on one MI355X.

A step is one pass of the whole path for one batch: the decode token at position n-1
completes a CSA block (m = 4) and an HCA block (m' = 128), which are pooled into the
caches; the lightning indexer scores every compressed entry and keeps the top-k; CSA
attention runs over the selected entries plus the 128-token window and HCA attention over
every HCA entry plus the window.  The default workload is the Pro-shaped 1M-token decode
(batch 4, 262144 CSA entries, top-1024, 8192 HCA entries, 128 heads of dim 512).
``--config 2|3`` time the 128K HCA / CSA decode layers and ``--config 4`` the 8192-token
prefill chunk.

Inputs are generated on the GPU from a fixed seed, the caches are built with the library's
own pooling (untimed), and the timed steps rotate over ``--replicas`` copies of every tensor a
step reads, so that each step reads HBM rather than the 256 MB last-level cache.  Steps are
replayed from HIP graphs (one per replica).  The indexer scoring kernel, the dominant kernel,
is also timed alone with HIP events around a graph of back-to-back launches.

Prints one JSON line.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode query-tokens/s and achieved HBM GB/s, CSA+HCA at 128K/1M context"
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0  # dense fp8 matrix cores
BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix cores
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--config", type=int, default=5)
    ap.add_argument("--replicas", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only copy 1 GiB device to device (torch), for scaling HBM counters")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="rocprofv3 --pmc output folders: write the traffic record and exit")
    ap.add_argument("--traffic-out", default=PROFILE_TRAFFIC,
                    help="where --traffic-from writes its record")
    ap.add_argument("--fp4-keys", action="store_true",
                    help="indexer keys in MX FP4 (E2M1 + E8M0 per 32) instead of FP8")
    ap.add_argument("--sink", action="store_true",
                    help="run both attention calls with a per-head attention sink "
                         "(csa_attend_sink / hca_attend_sink)")
    ap.add_argument("--serial", action="store_true",
                    help="run the CSA and HCA layers one after the other on one stream")
    ap.add_argument("--norm-rope", action="store_true",
                    help="run the step with RMSNorm + partial RoPE (64 dims): fused into the "
                         "pooling of new blocks, and on the queries and window rows")
    ap.add_argument("--gop", action="store_true",
                    help="time the grouped output projection at the config's shape (its "
                         "tokens, n_h * c inputs in groups of 8 heads, 512 outputs per group)")
    ap.add_argument("--kv-append", action="store_true",
                    help="time the cache lifecycle at the config's shape (csahca_kv_append of a "
                         "chunk and of one decode token, CSA and HCA caches) instead of the step")
    ap.add_argument("--pool", action="store_true",
                    help="time csa_compress / hca_compress over the config's whole context")
    ap.add_argument("--overlap-pool", action="store_true",
                    help="time the overlapped two-stream CSA pooling (full context pass and a "
                         "decode append) at the config's shape instead of the step")
    return ap.parse_args()


class Workload:
    """All device state of one workload: inputs, caches, replicas, outputs, workspaces."""

    NR_D, NR_EPS, NR_THETA = 64, 1e-6, 10000.0

    def __init__(self, cfg, replicas, sink=False, norm_rope=False, serial=False):
        import torch

        import compressed_attention_compress_amd as lib
        from synthgen.device import make_problem_device

        self.lib = lib
        self.cfg = cfg
        self.R = replicas
        # a second stream for the HCA attention at decode (a prefill chunk keeps one: its
        # two attention calls each fill the chip, and measured faster one after the other)
        self.s_hca = None if serial or cfg.kind == "prefill" else torch.cuda.Stream()  # default priority
        dev = "cuda"
        prob = make_problem_device(cfg, dev)
        self.prob = prob
        self.n = prob["n_total"]
        self.Tq = prob["Tq"]
        self.kind = cfg.kind
        self.layers = [l for l in ("csa", "hca") if f"X_{l}" in prob]
        B, c, n, dt = cfg.B, cfg.c, self.n, cfg.dtype
        self.q_pos = prob["q_pos"]
        # storage of KV rows, caches and outputs: float32, or bfloat16 bit patterns in int16
        et = torch.float32 if dt == 0 else torch.int16
        self.win_pos = torch.zeros(B, dtype=torch.int32, device=dev)
        self.scale = 1.0 / math.sqrt(c)
        # the pooled caches as a prefill would leave them (untimed): every complete block
        # before the step's own new blocks
        self.n_old = n - (self.Tq if self.kind == "prefill" else 1)
        self.nr = norm_rope
        self.rows_pooled = False  # the step's window rows were normalised with the pooling
        if norm_rope:  # seeded gains U(0.5, 1.5) for the KV rows and for the queries
            gn = torch.Generator(device=dev).manual_seed(77)
            self.g_kv = torch.rand((c,), generator=gn, device=dev) + 0.5
            self.g_q = torch.rand((c,), generator=gn, device=dev) + 0.5
            # normalised, rotated window rows (positions n - Tq - W + 1 .. n - 1): a row is
            # normalised once, when its token arrives; the rows of earlier tokens are made
            # here (untimed), the step's own Tq rows inside the step.  The queries are
            # normalised by the attention kernel as it loads them.
            self.nr_wpos0 = max(0, n - self.Tq - cfg.W + 1)
            self.nr_L = n - self.nr_wpos0
            self.nr_win_pos = torch.full((B,), self.nr_wpos0, dtype=torch.int32, device=dev)
            self.nr_new_pos = torch.full((B,), n - self.Tq, dtype=torch.int32, device=dev)
            self.nr_win = {l: torch.empty((B, self.nr_L, c), dtype=et, device=dev)
                           for l in self.layers}
            for l in self.layers:
                lib.csahca_norm_rope(prob[f"X_{l}"][:, self.nr_wpos0:], self.nr_win[l], self.g_kv,
                                     self.nr_win_pos, B, self.nr_L, 1, c, 1, self.NR_D, self.NR_EPS,
                                     self.NR_THETA, 1, dt, x_bstride=n * c, y_bstride=self.nr_L * c)
        base = {}
        for l in self.layers:
            m = cfg.m if l == "csa" else cfg.m_hca
            C = torch.zeros((B, n // m, c), dtype=et, device=dev)
            if norm_rope:
                lib.csahca_compress_norm_rope(prob[f"X_{l}"], prob[f"Z_{l}"], None, self.g_kv, C, B,
                                              self.n_old, c, m, 0, self.NR_D, self.NR_EPS,
                                              self.NR_THETA, dt, n * c, (n // m) * c)
            else:
                lib.csa_compress(prob[f"X_{l}"], prob[f"Z_{l}"], None, C, B, self.n_old, c, m, dt,
                                 n * c, (n // m) * c)
            base[f"C_{l}"] = C
            base[f"Q_{l}"] = prob[f"Q_{l}"]
        if "csa" in self.layers:
            for key in ("qI", "w"):
                base[key] = prob[key]
            if "KI_scales" in prob:  # MX FP4 keys: all packed rows, then all scales
                base["KI"] = torch.cat([prob["KI"].reshape(-1), prob["KI_scales"].reshape(-1)])
            else:
                base["KI"] = prob["KI"]
        torch.cuda.synchronize()
        # replicas of everything a step reads (distinct memory, same values)
        self.rep = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(replicas - 1)]
        self.N_c = n // cfg.m
        self.N_h = n // cfg.m_hca
        nq = B * self.Tq
        self.out = {l: torch.empty((B, self.Tq, cfg.n_h, c), dtype=et, device=dev)
                    for l in self.layers}
        if "csa" in self.layers:
            self.idx = torch.empty((B, self.Tq, cfg.k), dtype=torch.int32, device=dev)
            self.iws_b = lib.lightning_index_topk_workspace_size(B, self.Tq, cfg.n_ih, self.N_c, cfg.k)
            self.iws = torch.empty(self.iws_b, dtype=torch.uint8, device=dev)
            self.scores = torch.empty((nq * self.N_c,), dtype=torch.float32, device=dev)
            self.cws_b = lib.csa_attend_workspace_size(B, self.Tq, cfg.n_h, c, cfg.k, cfg.W)
            self.cws = torch.empty(max(self.cws_b, 256), dtype=torch.uint8, device=dev)
        if "hca" in self.layers:
            self.hws_b = lib.hca_attend_workspace_size(B, self.Tq, cfg.n_h, c, self.N_h, cfg.W)
            self.hws = torch.empty(max(self.hws_b, 256), dtype=torch.uint8, device=dev)
        self.sink = None
        if sink:  # seeded per-head logits, N(0, 2^2)
            gs = torch.Generator(device=dev).manual_seed(99)
            self.sink = torch.randn((cfg.n_h,), generator=gs, device=dev) * 2.0
        torch.cuda.synchronize()

    # -- the step -------------------------------------------------------------------------
    def pool_new_blocks(self, r, layers=None):
        """Pool the blocks completed by the step's tokens into replica r's caches."""
        cfg, lib, prob = self.cfg, self.lib, self.prob
        B, c, n = cfg.B, cfg.c, self.n
        layers = self.layers if layers is None else layers
        if self.nr and self.kind != "prefill" and len(self.layers) == 2 and len(layers) == 1:
            # one layer of the pair on its own stream: its pooling with the norm and its new
            # window rows in one launch (the pair call with the other side empty)
            l = layers[0]
            m = cfg.m if l == "csa" else cfg.m_hca
            first_blk = self.n_old // m
            tok0 = first_blk * m
            C = self.rep[r][f"C_{l}"]
            Tq, L = self.Tq, self.nr_L
            side = [prob[f"X_{l}"][:, tok0:], prob[f"Z_{l}"][:, tok0:], self.g_kv, C[:, first_blk:], n - tok0,
                    m, first_blk, n * c, (n // m) * c]
            empty = [None, None, None, None, 0, cfg.m_hca if l == "csa" else cfg.m, 0, c, c]
            rows = [prob[f"X_{l}"][:, n - Tq:], self.nr_win[l][:, L - Tq:], self.nr_new_pos, n * c, L * c]
            no_rows = [None, None, None, c, c]
            a, b = (side, empty) if l == "csa" else (empty, side)
            ra, rb = (rows, no_rows) if l == "csa" else (no_rows, rows)
            lib.csahca_compress_pair_norm_rope_rows(*a, *b, B, c, self.NR_D, self.NR_EPS, self.NR_THETA,
                                                    cfg.dtype, Tq, *ra, *rb)
            self.rows_pooled = True
            return
        if len(layers) == 2:
            # both caches in one call (one launch at decode)
            sides = []
            for l in ("csa", "hca"):
                m = cfg.m if l == "csa" else cfg.m_hca
                first_blk = self.n_old // m
                tok0 = first_blk * m
                C = self.rep[r][f"C_{l}"]
                X, Z = prob[f"X_{l}"][:, tok0:], prob[f"Z_{l}"][:, tok0:]
                if self.nr:
                    sides += [X, Z, self.g_kv, C[:, first_blk:], n - tok0, m, first_blk, n * c,
                              (n // m) * c]
                else:
                    sides += [X, Z, C[:, first_blk:], n - tok0, m, n * c, (n // m) * c]
            if self.nr:
                # the step's new tokens enter both layers' normalised window rows in the same
                # launch (window_rows then has nothing left to do)
                Tq, L = self.Tq, self.nr_L
                rows = []
                for l in ("csa", "hca"):
                    rows += [prob[f"X_{l}"][:, n - Tq:], self.nr_win[l][:, L - Tq:], self.nr_new_pos,
                             n * c, L * c]
                lib.csahca_compress_pair_norm_rope_rows(*sides, B, c, self.NR_D, self.NR_EPS,
                                                        self.NR_THETA, cfg.dtype, Tq, *rows)
                self.rows_pooled = True
            else:
                lib.csahca_compress_pair(*sides, B, c, cfg.dtype)
            return
        for l in layers:
            m = cfg.m if l == "csa" else cfg.m_hca
            first_blk = self.n_old // m          # first block not yet in the cache
            n_new = n // m - first_blk
            if n_new <= 0:
                continue
            X, Z, C = prob[f"X_{l}"], prob[f"Z_{l}"], self.rep[r][f"C_{l}"]
            tok0 = first_blk * m
            if self.nr:
                lib.csahca_compress_norm_rope(X[:, tok0:], Z[:, tok0:], None, self.g_kv,
                                              C[:, first_blk:], B, n_new * m, c, m, first_blk,
                                              self.NR_D, self.NR_EPS, self.NR_THETA, cfg.dtype,
                                              n * c, (n // m) * c)
            else:
                lib.csa_compress(X[:, tok0:], Z[:, tok0:], None, C[:, first_blk:], B, n_new * m, c,
                                 m, cfg.dtype, n * c, (n // m) * c)

    def select(self, r):
        cfg = self.cfg
        self.lib.lightning_index_select(self.scores, self.q_pos, cfg.m, cfg.B, self.Tq, self.N_c,
                                        cfg.k, self.idx, None, self.iws, self.iws_b)

    def index(self, r, split=False, pool_csa=False):
        """The indexer; with pool_csa (norm and rotation) the CSA cache's new blocks and the
        layer's new window rows are pooled and normalised in the same call (in the
        selection launch's spare workgroups at decode)."""
        cfg, lib, rp = self.cfg, self.lib, self.rep[r]
        B = cfg.B
        if split:
            self.index_score(r)
            self.select(r)
        elif pool_csa:
            m, n, c, Tq, L = cfg.m, self.n, cfg.c, self.Tq, self.nr_L
            first_blk = self.n_old // m
            tok0 = first_blk * m
            X, Z, C = self.prob["X_csa"], self.prob["Z_csa"], rp["C_csa"]
            lib.lightning_index_topk_csa_compress_norm_rope_rows(
                rp["qI"], rp["w"], rp["KI"], cfg.idx_dtype, self.q_pos, m, B, Tq, cfg.n_ih, cfg.c_I, self.N_c,
                cfg.k, self.idx, None, self.scores, self.iws, self.iws_b, X[:, tok0:], Z[:, tok0:], self.g_kv,
                C[:, first_blk:], n - tok0, c, first_blk, self.NR_D, self.NR_EPS, self.NR_THETA, cfg.dtype, n * c,
                (n // m) * c, Tq, X[:, n - Tq:], self.nr_win["csa"][:, L - Tq:], self.nr_new_pos, n * c, L * c)
            self.rows_pooled = True
        else:
            lib.lightning_index_topk(rp["qI"], rp["w"], rp["KI"], cfg.idx_dtype, self.q_pos, cfg.m,
                                     B, self.Tq, cfg.n_ih, cfg.c_I, self.N_c, cfg.k, self.idx, None,
                                     self.scores, self.iws, self.iws_b)

    def index_score(self, r):
        cfg, rp = self.cfg, self.rep[r]
        self.lib.lightning_index_score(rp["qI"], rp["w"], rp["KI"], cfg.idx_dtype, self.q_pos, cfg.m,
                                       cfg.B, self.Tq, cfg.n_ih, cfg.c_I, self.N_c, cfg.k,
                                       self.scores, self.iws, self.iws_b)

    def window_rows(self, r, l):
        """The window source of layer l the attention call reads: (rows, win_pos, L).  With
        norm_rope, the step's own Tq tokens enter the normalised window rows first."""
        cfg, lib, prob = self.cfg, self.lib, self.prob
        B, c, n = cfg.B, cfg.c, self.n
        if not self.nr:
            return prob[f"X_{l}"], self.win_pos, n
        Tq, L = self.Tq, self.nr_L
        if self.rows_pooled:  # normalised by the paired pooling launch of this step
            return self.nr_win[l], self.nr_win_pos, L
        lib.csahca_norm_rope(prob[f"X_{l}"][:, n - Tq:], self.nr_win[l][:, L - Tq:], self.g_kv,
                             self.nr_new_pos, B, Tq, 1, c, 1, self.NR_D, self.NR_EPS, self.NR_THETA,
                             1, cfg.dtype, x_bstride=n * c, y_bstride=L * c)
        return self.nr_win[l], self.nr_win_pos, L

    def attend(self, r, layers=None):
        cfg, lib, rp, prob = self.cfg, self.lib, self.rep[r], self.prob
        B, c, n = cfg.B, cfg.c, self.n
        sk = self.sink
        layers = self.layers if layers is None else layers
        # with norm_rope the queries' RMSNorm + RoPE runs inside the attention kernel
        nrq = (self.g_q, 1, self.NR_D, self.NR_EPS, self.NR_THETA) if self.nr else None
        if "csa" in layers:
            win, wpos, L = self.window_rows(r, "csa")
            args = (rp["Q_csa"], rp["C_csa"], self.idx, win, wpos, self.q_pos, B,
                    self.Tq, cfg.n_h, c, self.N_c, cfg.k, L, cfg.W, self.scale)
            tail = (cfg.dtype, self.out["csa"], None, self.cws, self.cws_b)
            if nrq is not None:
                lib.csa_attend_ex(*args, sk, *nrq, *tail)
            elif sk is None:
                lib.csa_attend(*args, *tail)
            else:
                lib.csa_attend_sink(*args, sk, *tail)
        if "hca" in layers:
            win, wpos, L = self.window_rows(r, "hca")
            args = (rp["Q_hca"], rp["C_hca"], win, wpos, self.q_pos, cfg.m_hca, B,
                    self.Tq, cfg.n_h, c, self.N_h, L, cfg.W, self.scale)
            tail = (cfg.dtype, self.out["hca"], None, self.hws, self.hws_b)
            if nrq is not None:
                lib.hca_attend_ex(*args, sk, *nrq, *tail)
            elif sk is None:
                lib.hca_attend(*args, *tail)
            else:
                lib.hca_attend_sink(*args, sk, *tail)

    def step(self, r):
        """One pass of the path.  At decode, with both layers present, a second stream
        carries the pooling of both caches and the HCA attention, while the first stream
        scores and selects; the CSA attention then waits for the CSA pooling, which
        finished long before.  (With norm and rotation each layer's pooling comes with its
        new window row, and the CSA one runs in the selection launch's spare workgroups.)
        The second stream forks at the start of the step and joins at its end.
        Edges between the graph's hardware queues resolve late when the producer is still
        running as the waiting queue reaches them (the waiting node started up to tens of
        microseconds after its producer in kernel traces); here every wait but the final
        join finds its producer done."""
        import torch

        if len(self.layers) == 2 and self.s_hca is not None:
            main = torch.cuda.current_stream()
            start = torch.cuda.Event()
            start.record(main)
            csa_pooled = torch.cuda.Event()
            self.s_hca.wait_event(start)
            with torch.cuda.stream(self.s_hca):
                if not self.nr:
                    self.pool_new_blocks(r, ["csa"])
                    csa_pooled.record(self.s_hca)
                self.pool_new_blocks(r, ["hca"])
                self.attend(r, ["hca"])
            # with norm and rotation the indexer call pools the CSA block and its window row
            self.index(r, pool_csa=self.nr)
            if not self.nr:
                main.wait_event(csa_pooled)
            self.attend(r, ["csa"])
            main.wait_stream(self.s_hca)
            return
        self.pool_new_blocks(r)
        if "csa" in self.layers:
            self.index(r)
        self.attend(r)

    # -- accounting -----------------------------------------------------------------------
    def algorithmic_bytes(self):
        """Bytes the step must move at minimum: every input read once, every output written
        once (compressed caches: only the rows the step reads)."""
        cfg = self.cfg
        B, c, W, Tq, n = cfg.B, cfg.c, cfg.W, self.Tq, self.n
        e = 4 if cfg.dtype == 0 else 2  # bytes per KV / query / output element
        total = 0
        detail = {}
        for l in self.layers:
            m = cfg.m if l == "csa" else cfg.m_hca
            n_new_blocks = n // m - self.n_old // m
            pool = B * n_new_blocks * (2 * m * c * e + c * e)
            total += pool
            detail[f"pool_{l}"] = pool
        qpos = [n - Tq + t for t in range(Tq)]
        if "csa" in self.layers:
            V = [min(self.N_c, (p + 1) // cfg.m) for p in qpos]
            ki = B * max(V) * self.key_row_bytes()  # keys are shared by a sequence's queries
            idx = B * Tq * (cfg.n_ih * cfg.c_I + cfg.n_ih * 4 + cfg.k * 4)
            detail["index"] = ki + idx
            total += ki + idx
            rows = sum(min(cfg.k, v) + min(W, p + 1) for v, p in zip(V, qpos))
            att = B * rows * c * e + 2 * B * Tq * cfg.n_h * c * e + B * Tq * cfg.k * 4
            if Tq > 1:  # rows shared between prefill queries are still read per query (gather)
                pass
            detail["csa_attend"] = att
            total += att
        if "hca" in self.layers:
            Vh = [min(self.N_h, (p + 1) // cfg.m_hca) for p in qpos]
            if Tq == 1:
                rows = B * (Vh[0] + min(W, qpos[0] + 1))
            else:  # one pass over the shared entries and the chunk's raw rows
                rows = B * (max(Vh) + Tq + W - 1)
            att = rows * c * e + 2 * B * Tq * cfg.n_h * c * e
            detail["hca_attend"] = att
            total += att
        if self.nr:  # the step's new window rows read and written once (queries: in attention)
            nrb = len(self.layers) * 2 * B * Tq * c * e
            detail["norm_rope_rows"] = nrb
            total += nrb
        return total, detail

    def index_score_bytes(self):
        cfg = self.cfg
        qpos = [self.n - self.Tq + t for t in range(self.Tq)]
        V = max(min(self.N_c, (p + 1) // cfg.m) for p in qpos)
        return cfg.B * V * self.key_row_bytes() + cfg.B * self.Tq * cfg.n_ih * (cfg.c_I + 4)

    def key_row_bytes(self):
        """Bytes of one indexer key: c_I codes, or for MX FP4 c_I/2 plus a scale per 32."""
        c_I = self.cfg.c_I
        return c_I // 2 + c_I // 32 if self.cfg.idx_dtype == 3 else c_I

    def flops(self):
        cfg = self.cfg
        qpos = [self.n - self.Tq + t for t in range(self.Tq)]
        f8 = bf = 0
        for p in qpos:
            if "csa" in self.layers:
                V = min(self.N_c, (p + 1) // cfg.m)
                f8 += 2 * V * cfg.n_ih * cfg.c_I
                bf += 4 * cfg.n_h * cfg.c * (min(cfg.k, V) + min(cfg.W, p + 1))
            if "hca" in self.layers:
                Vh = min(self.N_h, (p + 1) // cfg.m_hca)
                bf += 4 * cfg.n_h * cfg.c * (Vh + min(cfg.W, p + 1))
        return cfg.B * f8, cfg.B * bf


# the sources the decode scoring kernel is built from (its file and the headers it includes)
SCORE_SOURCES = ("index_score.hip", "fused_topk.hpp", "indexer.hpp", "common.hpp")


def score_source_hash():
    import hashlib
    h = hashlib.sha256()
    for name in SCORE_SOURCES:
        with open(os.path.join(ROOT, "compressed_attention_compress_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_traffic(kernel_name, workload):
    """HBM traffic of the dominant kernel from committed counter runs, if they were taken
    on this workload and the kernel's sources are unchanged since (else None)."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            rec = json.load(f)
        h = score_source_hash()
        ent = rec.get(kernel_name)
        if ent and ent.get("source_sha256") == h and ent.get("workload") == workload:
            return ent["bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        pass
    return None


COPY_BYTES = 1 << 30
COPY_KERNEL = "neg"  # name part of torch's elementwise negation kernel
TRAFFIC_KERNELS = {"index_score_dec128": "index_score_dec128"}  # decode scoring kernel


def _counter_means(folder, counter, name_part):
    """Mean per dispatch of `counter` over the dispatches of kernels whose name contains
    `name_part`, from a rocprofv3 --pmc csv output folder."""
    import csv
    import glob
    vals = []
    for f in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row["Counter_Name"] == counter and name_part in row["Kernel_Name"]:
                    vals.append(float(row["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} samples for kernels named like {name_part!r} in {folder}")
    return sum(vals) / len(vals), len(vals)


def write_traffic(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, out_path, workload):
    """HBM bytes per launch of the dominant kernel: FETCH_SIZE + WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for a plain 1 GiB device copy.
    `workload`: the config the counter runs used (the record applies to it alone)."""
    cf, _ = _counter_means(copy_fetch_dir, "FETCH_SIZE", COPY_KERNEL)
    cw, _ = _counter_means(copy_write_dir, "WRITE_SIZE", COPY_KERNEL)
    f_scale = COPY_BYTES / (cf * 1024.0)   # true bytes per counted byte
    w_scale = COPY_BYTES / (cw * 1024.0)
    rec = {"copy_calibration": {"bytes": COPY_BYTES, "fetch_kib": cf, "write_kib": cw,
                                "fetch_scale": f_scale, "write_scale": w_scale}}
    for key, name in TRAFFIC_KERNELS.items():
        fk, nf = _counter_means(fetch_dir, "FETCH_SIZE", name)
        wk, nw = _counter_means(write_dir, "WRITE_SIZE", name)
        rec[key] = {"fetch_kib_per_dispatch": fk, "write_kib_per_dispatch": wk,
                    "dispatches": [nf, nw],
                    "bytes_per_launch": round(fk * 1024.0 * f_scale + wk * 1024.0 * w_scale),
                    "workload": workload, "source_sha256": score_source_hash()}
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def calibrate_copy():
    import torch
    # torch.neg: one elementwise kernel that reads 1 GiB and writes 1 GiB (the values are
    # irrelevant, so the source is left uninitialised: no fill kernel to tell apart)
    a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES}), flush=True)


def measured_copy_gbs():
    """Achievable HBM rate on this machine: one elementwise pass reading 1 GiB and writing 1 GiB
    (torch.neg), bytes moved / time, best of five."""
    import torch
    a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.neg(a, out=b)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.neg(a, out=b)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, 2 * COPY_BYTES / (e0.elapsed_time(e1) / 1e3) / 1e9)
    del a, b
    torch.cuda.empty_cache()
    return best


def host_cpu():
    """The host the oracle runs on: cores this process may use, BLAS threads, CPU model."""
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas = None
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return cores, blas, model


def cpu_baseline(wl, seconds):
    """The oracle, as it stands, on a bounded sample of the same workload, repeated until
    about `seconds` of CPU time is spent.  Decode: complete steps of whole sequences.  A
    prefill chunk: the pooling of the chunk's new blocks (timed once, its share added per
    query) and complete index / top-k / CSA / HCA passes for queries spread over the chunk."""
    import numpy as np

    import oracle
    from synthgen.configs import BF16

    cores, blas, model = host_cpu()
    cfg, prob = wl.cfg, wl.prob
    n, c, W, Tq = wl.n, cfg.c, cfg.W, wl.Tq

    def codes(t):
        a = t.detach().cpu().numpy()
        return a.view(np.uint16) if a.dtype == np.int16 else a

    def host(**extra):
        return {"cores": cores, "blas_threads": blas, "cpu_model": model, "kind": "oracle", **extra}

    if Tq != 1:
        return prefill_cpu_baseline(wl, seconds, codes, host)
    p = n - 1
    # inputs of each sequence, decoded once (input preparation, not timed)
    seqs = []
    for b in range(cfg.B):
        d = {}
        for l in wl.layers:
            m = cfg.m if l == "csa" else cfg.m_hca
            C = oracle.decode(codes(wl.rep[0][f"C_{l}"][b]), BF16)
            lo = (n // m - 1) * m
            d[f"blk_{l}"] = (oracle.decode(codes(prob[f"X_{l}"][b, lo:n]), BF16),
                             oracle.decode(codes(prob[f"Z_{l}"][b, lo:n]), BF16))
            d[f"win_{l}"] = oracle.decode(codes(prob[f"X_{l}"][b, n - W:n]), BF16)
            d[f"C_{l}"] = C
            d[f"Q_{l}"] = oracle.decode(codes(prob[f"Q_{l}"][b, 0]), BF16)
        if "csa" in wl.layers:
            f4 = cfg.idx_dtype == 3
            d["qI"] = oracle.decode(codes(prob["qI"][b, 0]), 2 if f4 else cfg.idx_dtype)
            d["w"] = prob["w"][b, 0].cpu().numpy()
            if f4:
                d["KI"] = oracle.decode_mxfp4(codes(prob["KI"][b]), codes(prob["KI_scales"][b]))
            else:
                d["KI"] = oracle.decode(codes(prob["KI"][b]), cfg.idx_dtype)
        seqs.append(d)

    done = 0
    t0 = time.perf_counter()
    while True:
        for d in seqs:
            for l in wl.layers:
                m = cfg.m if l == "csa" else cfg.m_hca
                newC = oracle.pool(*d[f"blk_{l}"], m)
                C = d[f"C_{l}"]
                C[-1] = newC[0]
                if l == "csa":
                    V = oracle.visible(p, m, C.shape[0])
                    s = oracle.index_scores(d["qI"], d["w"], d["KI"], V)
                    sel = oracle.topk(s, cfg.k)
                    rows = oracle.csa_rows(C, sel, d["win_csa"], n - W, p, W)
                else:
                    rows = oracle.hca_rows(C, m, d["win_hca"], n - W, p, W)
                oracle.attend(d[f"Q_{l}"], rows, wl.scale)
            done += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": done / el, "unit": "query-tokens/s", **host(
        sample=f"{done} complete decode steps of single sequences of this workload "
               f"({cfg.B} distinct sequences cycled), {el:.1f} s, NumPy fp64")}


def prefill_cpu_baseline(wl, seconds, codes, host):
    """Oracle timing on a prefill chunk: the chunk's pooling once, then whole query passes
    (scores over every visible entry, top-k, CSA and HCA attention) for queries spread
    evenly over the chunk until the time is spent; query-tokens/s counts the pooling at
    its share per query."""
    import numpy as np

    import oracle
    from synthgen.configs import BF16

    cfg, prob = wl.cfg, wl.prob
    n, W, Tq = wl.n, cfg.W, wl.Tq
    n0 = n - Tq
    b = 0
    X = oracle.decode(codes(prob["X_csa"][b]), BF16)     # old context and chunk (shared raw rows)
    Cs = oracle.decode(codes(wl.rep[0]["C_csa"][b]), BF16)
    Ch = oracle.decode(codes(wl.rep[0]["C_hca"][b]), BF16)
    Zc = oracle.decode(codes(prob["Z_csa"][b]), BF16)
    Zh = oracle.decode(codes(prob["Z_hca"][b]), BF16)
    qI = oracle.decode(codes(prob["qI"][b]), cfg.idx_dtype)
    w = prob["w"][b].cpu().numpy()
    KI = oracle.decode(codes(prob["KI"][b]), cfg.idx_dtype)
    Q = oracle.decode(codes(prob["Q_csa"][b]), BF16)
    # the chunk's new blocks, pooled once
    t0 = time.perf_counter()
    for m, Z, C in ((cfg.m, Zc, Cs), (cfg.m_hca, Zh, Ch)):
        f = n0 // m
        C[f:n // m] = oracle.pool(X[f * m:(n // m) * m], Z[f * m:(n // m) * m], m)
    t_pool = time.perf_counter() - t0
    order = np.linspace(0, Tq - 1, 64).astype(int)
    done = 0
    t0 = time.perf_counter()
    while True:
        for t in order:
            p = n0 + int(t)
            V = oracle.visible(p, cfg.m, Cs.shape[0])
            s = oracle.index_scores(qI[t], w[t], KI, V)
            sel = oracle.topk(s, cfg.k)
            oracle.attend(Q[t], oracle.csa_rows(Cs, sel, X, 0, p, W), wl.scale)
            oracle.attend(Q[t], oracle.hca_rows(Ch, cfg.m_hca, X, 0, p, W), wl.scale)
            done += 1
            if time.perf_counter() - t0 >= seconds:
                break
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per_query = el / done + t_pool / Tq
    return {"value": 1.0 / per_query, "unit": "query-tokens/s", **host(
        sample=f"{done} complete query passes (index over up to {Cs.shape[0]} entries, top-{cfg.k}, "
               f"CSA and HCA attention) of the {Tq}-token chunk, queries spread evenly over it, "
               f"{el:.1f} s; plus the chunk's pooling ({t_pool:.1f} s) at its share per query; "
               f"NumPy fp64")}


def overlap_pool(cfg, reps, cpu_seconds, no_cpu):
    """csa_compress_overlap at the config's CSA shape: one pass over the whole context
    (every entry; reads four [B, n, c] arrays, writes [B, n/m, c]) and a decode append
    (the last two blocks, prev = 1, one entry per sequence)."""
    import numpy as np
    import torch

    import compressed_attention_compress_amd as lib

    B, n, c, m = cfg.B, cfg.n, cfg.c, cfg.m
    dt = cfg.dtype
    g = torch.Generator(device="cuda").manual_seed(1234)
    tdt = torch.bfloat16 if dt == 1 else torch.float32
    arrs = []
    for k in range(4):  # X_a, Z_a, X_b, Z_b
        a = torch.randn((B, n, c), generator=g, device="cuda", dtype=torch.float32)
        if k % 2 == 0:
            a.mul_(1.0 / math.sqrt(c))
        arrs.append(a.to(tdt))
        del a
    N = n // m
    out = torch.empty((B, N, c), dtype=tdt, device="cuda")
    st = torch.cuda.current_stream()

    def full():
        lib.csa_compress_overlap(*arrs, None, out, B, n, c, m, 0, dt, n * c, N * c, stream=st)

    full()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        full()
    e1.record(st)
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / reps
    es = 2 if dt == 1 else 4
    nbytes = 4 * B * n * c * es + B * N * c * es

    # decode append: the last 2m tokens of every sequence, one entry each
    tail = [a[:, n - 2 * m:] for a in arrs]
    app_out = out[:, N - 1:N]

    def append():
        lib.csa_compress_overlap(*tail, None, app_out, B, 2 * m, c, m, 1, dt, n * c, N * c, stream=st)

    side = torch.cuda.Stream()
    append()
    torch.cuda.synchronize()
    ga = torch.cuda.CUDAGraph()
    with torch.cuda.graph(ga, stream=side):
        for _ in range(20):
            lib.csa_compress_overlap(*tail, None, app_out, B, 2 * m, c, m, 1, dt, n * c, N * c,
                                     stream=side)
    ga.replay()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        e0.record(side)
        for _ in range(10):
            ga.replay()
        e1.record(side)
    torch.cuda.synchronize()
    app_us = e0.elapsed_time(e1) * 1e3 / 200

    cpu = None
    if not no_cpu:
        import oracle
        rng = np.random.default_rng(5)
        ntok = 1 << 14  # tokens per oracle call (one sequence slice)
        Xa, Za, Xb, Zb = (rng.standard_normal((ntok, c)) for _ in range(4))
        t0 = time.perf_counter()
        done = 0
        while True:
            oracle.pool_overlap(Xa, Za, Xb, Zb, m)
            done += ntok
            el = time.perf_counter() - t0
            if el >= cpu_seconds:
                break
        cpu = {"value": round(done * (4 * c + c / m) * es / el / 1e9, 3), "unit": "GB/s",
               **dict(zip(("cores", "blas_threads", "cpu_model"), host_cpu())), "kind": "oracle",
               "sample": f"{done} tokens in {ntok}-token slices of one sequence, {el:.1f} s, "
                         f"NumPy fp64 (bytes counted at the GPU's storage width)"}
    gbs = nbytes / sec / 1e9
    line = {
        "metric": "overlapped two-stream CSA pooling, achieved HBM GB/s over the full context",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": reps, "warmup": 1,
        "ms_per_pass": round(sec * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if dt == 1 else "f32", "data": "synthetic",
        "config": {"workload": f"csa_overlap_pool_{cfg.name}", "batch": B, "context": n, "c": c,
                   "m": m, "timing": "HIP events around back-to-back launches"},
        "append_us": round(app_us, 2),
        "roofline": {"kernel": "pool_kernel (overlapped)", "bound": "hbm", "achieved": round(gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": None, "avg_launch_us": round(sec * 1e6, 2), "bytes_per_launch": nbytes},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def pool_bench(cfg, reps, cpu_seconds, no_cpu):
    """csa_compress (m) and hca_compress (m') over the config's whole raw context (a prefill
    config: the old context plus the chunk), one line per call and cache: a pass reads X
    and Z [B, n, c] once and writes [B, n/m, c].  The caches a config keeps: config 2 the
    HCA one, configs 1 and 3 the CSA one, configs 4 and 5 both."""
    import numpy as np
    import torch

    import compressed_attention_compress_amd as lib

    B, c, dt = cfg.B, cfg.c, cfg.dtype
    n = cfg.n + (cfg.Tq if cfg.kind == "prefill" else 0)
    layers = {"hca_decode": ["hca"], "csa_decode": ["csa"]}.get(cfg.kind, ["csa", "hca"])
    tdt = torch.bfloat16 if dt == 1 else torch.float32
    es = 2 if dt == 1 else 4
    st = torch.cuda.current_stream()
    g = torch.Generator(device="cuda").manual_seed(4321)
    X = torch.empty((B, n, c), dtype=tdt, device="cuda")
    Z = torch.empty((B, n, c), dtype=tdt, device="cuda")
    for b in range(B):  # generated per sequence, to bound the float32 staging
        X[b].copy_(torch.randn((n, c), generator=g, device="cuda").mul_(cfg.kv_std))
        Z[b].copy_(torch.randn((n, c), generator=g, device="cuda"))
    cpu = None
    if not no_cpu:
        import oracle
        rng = np.random.default_rng(6)
        ntok = 1 << 14  # tokens per oracle call (one sequence slice)
        Xs, Zs = rng.standard_normal((ntok, c)), rng.standard_normal((ntok, c))
        mm = cfg.m if layers[0] == "csa" else cfg.m_hca
        t0 = time.perf_counter()
        done = 0
        while True:
            oracle.pool(Xs, Zs, mm)
            done += ntok
            el = time.perf_counter() - t0
            if el >= cpu_seconds:
                break
        cpu = {"value": round(done * (2 * c + c / mm) * es / el / 1e9, 3), "unit": "GB/s",
               **dict(zip(("cores", "blas_threads", "cpu_model"), host_cpu())), "kind": "oracle",
               "sample": f"{done} tokens in {ntok}-token slices of one sequence, m = {mm}, "
                         f"{el:.1f} s, NumPy fp64 (bytes counted at the GPU's storage width)"}
    for l in layers:
        m = cfg.m if l == "csa" else cfg.m_hca
        N = n // m
        out = torch.empty((B, N, c), dtype=tdt, device="cuda")
        call = lib.csa_compress if l == "csa" else lib.hca_compress

        def run():
            call(X, Z, None, out, B, n, c, m, dt, n * c, N * c, stream=st)

        run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            run()
        e1.record(st)
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) / 1e3 / reps
        nbytes = 2 * B * n * c * es + B * N * c * es
        gbs = nbytes / sec / 1e9
        line = {
            "metric": f"{l.upper()} pooling ({l}_compress, m = {m}), achieved HBM GB/s over the full context",
            "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": reps, "warmup": 1,
            "ms_per_pass": round(sec * 1e3, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16" if dt == 1 else "f32", "data": "synthetic",
            "config": {"workload": f"{l}_pool_{cfg.name}", "batch": B, "context": n, "c": c,
                       "m": m, "timing": "HIP events around back-to-back launches"},
            "roofline": {"kernel": "pool_kernel", "bound": "hbm", "achieved": round(gbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": None, "avg_launch_us": round(sec * 1e6, 2), "bytes_per_launch": nbytes},
            "cpu_baseline": cpu if l == layers[0] else None,
        }
        print(json.dumps(line), flush=True)
        del out


def kv_append(cfg, reps, cpu_seconds, no_cpu):
    """csahca_kv_append at the config's shape, for the CSA (m) and the HCA (m') cache of a
    layer pair.  Every sequence holds n - 1 tokens, so that both caches have a tail of
    m - 1 tokens.  Chunk: the config's prefill chunk (8192 tokens for a decode config) is
    appended to every sequence; bytes counted are the new tokens' values and gate logits
    read once, the tail read back from the ring, the entries written and the last R tokens
    written to the ring once (the ring's second copy is layout, not counted).  Decode: one
    token per sequence, which completes a block of both caches; timed from a graph of 20."""
    import numpy as np
    import torch

    import compressed_attention_compress_amd as lib

    B, c, W, dt = cfg.B, cfg.c, cfg.W, cfg.dtype
    n_old = cfg.n - 1
    chunk = cfg.Tq if cfg.kind == "prefill" else 8192
    es = 2 if dt == 1 else 4
    tdt = torch.bfloat16 if dt == 1 else torch.float32
    g = torch.Generator(device="cuda").manual_seed(4321)
    X = (torch.randn((B, chunk, c), generator=g, device="cuda") / math.sqrt(c)).to(tdt)
    Z = torch.randn((B, chunk, c), generator=g, device="cuda").to(tdt)
    caches = []
    for m in (cfg.m, cfg.m_hca):
        R = lib.csahca_kv_ring_rows(W, m)
        NE = (n_old + chunk) // m
        caches.append(dict(m=m, R=R, NE=NE,
                           rx=torch.zeros((B, 2 * R, c), dtype=tdt, device="cuda"),
                           rz=torch.zeros((B, 2 * R, c), dtype=tdt, device="cuda"),
                           ent=torch.zeros((B, NE, c), dtype=tdt, device="cuda")))
    st = torch.cuda.current_stream()

    def append(k, stream):
        for cc in caches:
            lib.csahca_kv_append(cc["rx"], cc["rz"], cc["ent"], X, Z, None, B, n_old, k, c, cc["m"],
                                 W, dt, chunk * c, 2 * cc["R"] * c, cc["NE"] * c, stream=stream)

    def chunk_bytes(k):
        tot = 0
        for cc in caches:
            m, R = cc["m"], cc["R"]
            t = n_old % m
            made = (n_old + k) // m - n_old // m
            tot += B * c * es * (2 * k + (2 * t if k >= m - t else 0) + made + 2 * min(k, R))
        return tot

    append(chunk, st)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        append(chunk, st)
    e1.record(st)
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / reps
    nbytes = chunk_bytes(chunk)
    gbs = nbytes / sec / 1e9

    side = torch.cuda.Stream()
    ga = torch.cuda.CUDAGraph()
    with torch.cuda.graph(ga, stream=side):
        for _ in range(20):
            append(1, side)
    ga.replay()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        e0.record(side)
        for _ in range(10):
            ga.replay()
        e1.record(side)
    torch.cuda.synchronize()
    dec_us = e0.elapsed_time(e1) * 1e3 / 200

    cpu = None
    if not no_cpu:
        from oracle import kvcache as K
        rng = np.random.default_rng(6)
        ntok = 1024  # tokens per simulator append (one sequence)
        Xc, Zc = rng.standard_normal((ntok, c)), rng.standard_normal((ntok, c))
        el, done = 0.0, 0
        while el < cpu_seconds:  # fresh simulators with an m' - 1 token tail each round
            sims = [K.KVSim(c, cc["m"], W) for cc in caches]
            for s in sims:
                s.append(Xc[:cfg.m_hca - 1], Zc[:cfg.m_hca - 1])
            t0 = time.perf_counter()
            for s in sims:
                s.append(Xc, Zc)
            el += time.perf_counter() - t0
            done += 1
        per = sum(c * es * (2 * ntok + ntok // cc["m"] + 2 * min(ntok, cc["R"])) for cc in caches)
        cpu = {"value": round(done * per / el / 1e9, 4), "unit": "GB/s",
               **dict(zip(("cores", "blas_threads", "cpu_model"), host_cpu())), "kind": "oracle",
               "sample": f"{done} appends of {ntok} tokens to the CSA and HCA simulators of one "
                         f"sequence, {el:.1f} s, NumPy fp64 (bytes counted at the GPU's storage "
                         f"width)"}
    line = {
        "metric": "KV-cache append (CSA + HCA caches), achieved HBM GB/s for a chunk",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": reps, "warmup": 1,
        "ms_per_append": round(sec * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if dt == 1 else "f32", "data": "synthetic",
        "config": {"workload": f"kv_append_{cfg.name}", "batch": B, "n_old": n_old, "chunk": chunk,
                   "c": c, "m": [cfg.m, cfg.m_hca], "W": W,
                   "timing": "HIP events around back-to-back calls"},
        "decode_append_us": round(dec_us, 2),
        "roofline": {"kernel": "csahca_kv_append (pool_kernel + ring_store)", "bound": "hbm",
                     "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "avg_launch_us": round(sec * 1e6, 2), "bytes_per_launch": nbytes},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def gop_bench(cfg, reps, cpu_seconds, no_cpu):
    """grouped_out_proj on the config's attention output: T = B * Tq tokens of n_h * c,
    g = n_h / 8 groups (K_g = 8c), d_g = 512.  Decode shapes are bound by streaming the
    weights (HBM roofline); the prefill chunk by MFMA (bf16 roofline)."""
    import numpy as np
    import torch

    import compressed_attention_compress_amd as lib

    T = cfg.B * cfg.Tq
    g, d_g = cfg.n_h // 8, 512
    K_g = cfg.n_h * cfg.c // g
    gen = torch.Generator(device="cuda").manual_seed(2024)
    o = torch.randn((T, g * K_g), generator=gen, device="cuda").to(torch.bfloat16)
    reps_w = 1 if T > 64 else 8  # decode: rotate weight copies so every call streams HBM
    ws = [(torch.randn((g, d_g, K_g), generator=gen, device="cuda") / math.sqrt(K_g)).to(torch.bfloat16)
          for _ in range(reps_w)]
    y = torch.empty((T, g * d_g), dtype=torch.bfloat16, device="cuda")
    st = torch.cuda.Stream()

    def call(i, stream):
        lib.grouped_out_proj(o, ws[i % reps_w], y, T, g, K_g, d_g, g * K_g, g * d_g, 1, stream=stream)

    call(0, st)
    torch.cuda.synchronize()
    n_in = 40 if T <= 64 else 4
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=st):
        for i in range(n_in):
            call(i, st)
    gr.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(st):
        e0.record(st)
        for _ in range(reps):
            gr.replay()
        e1.record(st)
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / (reps * n_in)
    flops = 2.0 * T * g * K_g * d_g
    nbytes = 2 * (g * d_g * K_g + T * g * K_g + T * g * d_g)
    if T > 64:
        bound, ach, peak, unit = "mfma", flops / sec / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s"
        kname = "gop_gemm"
    else:
        bound, ach, peak, unit = "hbm", nbytes / sec / 1e9, HBM_PEAK_GBS, "GB/s"
        kname = "gop_skinny"
    cpu = None
    if not no_cpu:
        import oracle
        rng = np.random.default_rng(8)
        tk = 4
        Oc = rng.standard_normal((tk, g * K_g))
        Wc = rng.standard_normal((g, d_g, K_g))
        t0 = time.perf_counter()
        done = 0
        while time.perf_counter() - t0 < cpu_seconds:
            oracle.grouped_out_proj(Oc, Wc)
            done += tk
        el = time.perf_counter() - t0
        cpu = {"value": round(done / el, 2), "unit": "tokens/s", **dict(zip(("cores", "blas_threads", "cpu_model"), host_cpu())),
               "kind": "oracle", "sample": f"{done} tokens in calls of {tk}, {el:.1f} s, NumPy fp64"}
    line = {
        "metric": "grouped output projection throughput (tokens/s)",
        "value": round(T / sec, 1), "unit": "tokens/s", "n_gpus": 1, "steps": reps * n_in,
        "warmup": 1, "us_per_call": round(sec * 1e6, 2), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"gop_{cfg.name}", "tokens": T, "groups": g, "K_g": K_g,
                   "d_g": d_g, "timing": "HIP events around graph replays"},
        "roofline": {"kernel": kname, "bound": bound, "achieved": round(ach, 1), "peak": peak,
                     "unit": unit, "frac": round(ach / peak, 4), "traffic": None,
                     "avg_launch_us": round(sec * 1e6, 2),
                     "flops_per_launch" if bound == "mfma" else "bytes_per_launch":
                         flops if bound == "mfma" else nbytes},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.traffic_from:
        from synthgen.configs import CONFIGS as CFGS  # --config: the one the counter runs used
        write_traffic(*args.traffic_from, args.traffic_out, CFGS[args.config].name)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)
    import torch

    from synthgen.configs import CONFIGS

    if args.calibrate_copy:
        calibrate_copy()
        return
    cfg = CONFIGS[args.config]
    if args.fp4_keys:
        if cfg.idx_dtype != 2:
            print("--fp4-keys needs a config with an FP8 indexer", file=sys.stderr)
            sys.exit(2)
        cfg = cfg.scaled(idx_dtype=3)
    if args.gop:
        gop_bench(cfg, args.steps or 10, min(args.cpu_seconds, 10.0), args.no_cpu_baseline)
        return
    if args.kv_append:
        kv_append(cfg, args.steps or 20, min(args.cpu_seconds, 10.0), args.no_cpu_baseline)
        return
    if args.pool:
        pool_bench(cfg, args.steps or 10, min(args.cpu_seconds, 10.0), args.no_cpu_baseline)
        return
    if args.overlap_pool:
        overlap_pool(cfg, args.steps or 10, min(args.cpu_seconds, 10.0), args.no_cpu_baseline)
        return
    decode = cfg.kind != "prefill"
    steps = args.steps if args.steps is not None else (500 if decode else 20)
    warmup = args.warmup if args.warmup is not None else (50 if decode else 3)
    R = args.replicas if args.replicas is not None else (6 if decode else 1)
    torch.cuda.set_device(0)
    wl = Workload(cfg, R, sink=args.sink, norm_rope=args.norm_rope, serial=args.serial)

    # warm up eagerly (also sets the library's one-time kernel attributes)
    for i in range(warmup):
        wl.step(i % R)
    torch.cuda.synchronize()

    # one graph holds R consecutive steps (one per replica), as a decode loop would hold
    # many steps (and layers) in one graph; a second graph holds the K mod R left over
    side = torch.cuda.Stream()

    def capture(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for r in range(n):
                wl.step(r)
        return g

    g_full = capture(R)
    rem = steps % R
    g_rem = capture(rem) if rem else None
    g_full.replay()
    if g_rem is not None:
        g_rem.replay()
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for _ in range(steps // R):
        g_full.replay()
    if g_rem is not None:
        g_rem.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    sec = (t1 - t0) / steps
    qtok = cfg.B * wl.Tq / sec
    abytes, detail = wl.algorithmic_bytes()
    f8, bf = wl.flops()

    roofline = None
    if "csa" in wl.layers:
        gs = torch.cuda.CUDAGraph()
        reps = max(R, 8)
        # the dominant kernel: the indexer's scoring launch as the step makes it (at decode
        # it also cuts and writes every chunk's top-k list); the selection launch follows
        # it in the step and is not part of this figure
        with torch.cuda.graph(gs, stream=side):
            for i in range(reps):
                wl.index_score(i % R)
        gs.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        rounds = 10 if decode else 1
        with torch.cuda.stream(side):
            e0.record(side)
            for _ in range(rounds):
                gs.replay()
            e1.record(side)
        torch.cuda.synchronize()
        dur = e0.elapsed_time(e1) / 1e3 / (rounds * reps)
        kb = wl.index_score_bytes()
        ach = kb / dur / 1e9
        kname = ("index_score_f32" if cfg.idx_dtype == 0 else
                 "index_score_dec128" if decode and cfg.c_I == 128 else
                 "index_score_pre128" if cfg.c_I == 128 else "index_score_fp8")
        if cfg.idx_dtype == 3:
            kname += " (MX FP4 keys)"  # no counter record for this instance
        fused = decode and cfg.c_I == 128 and cfg.idx_dtype in (2, 3)
        if decode or cfg.idx_dtype == 0:
            roofline = {"kernel": (kname + " (scoring with each chunk's top-k list)" if fused else kname),
                        "bound": "hbm",
                        "achieved": round(ach, 1),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                        "traffic": read_traffic(kname, cfg.name) if decode else None,
                        "avg_launch_us": round(dur * 1e6, 2), "bytes_per_launch": kb}
        else:  # a prefill chunk's scoring is bound by the fp8 matrix cores
            tf = f8 / dur / 1e12
            roofline = {"kernel": kname, "bound": "mfma", "achieved": round(tf, 1),
                        "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tf / FP8_PEAK_TFLOPS, 4), "traffic": None,
                        "avg_launch_us": round(dur * 1e6, 2), "flops_per_launch": f8}

    if roofline is None and "hca" in wl.layers:
        # no indexer: the HCA attention call (attention kernel and split merge) is the path
        gh = torch.cuda.CUDAGraph()
        reps = max(R, 8)
        with torch.cuda.graph(gh, stream=side):
            for i in range(reps):
                wl.attend(i % R, ["hca"])
        gh.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        rounds = 10 if decode else 1
        with torch.cuda.stream(side):
            e0.record(side)
            for _ in range(rounds):
                gh.replay()
            e1.record(side)
        torch.cuda.synchronize()
        dur = e0.elapsed_time(e1) / 1e3 / (rounds * reps)
        kb = detail["hca_attend"]
        ach = kb / dur / 1e9
        roofline = {"kernel": "hca_attend (attend_bf16 + split merge)", "bound": "hbm",
                    "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
                    "avg_launch_us": round(dur * 1e6, 2), "bytes_per_launch": kb}

    if roofline is not None and roofline["bound"] == "hbm":
        cg = measured_copy_gbs()  # the same rate against what a plain copy reaches here
        roofline["copy_ceiling_gbs"] = round(cg, 1)
        roofline["frac_of_copy_ceiling"] = round(roofline["achieved"] / cg, 4)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(qtok, 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(sec * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("f32" if cfg.dtype == 0 else "bf16") + "+" +
                 {0: "f32", 2: "fp8e4m3", 3: "mxfp4"}.get(cfg.idx_dtype, "?"),
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.B, "context": wl.n, "query_tokens": wl.Tq,
                   "c": cfg.c, "n_h": cfg.n_h, "m": cfg.m, "m_hca": cfg.m_hca, "k": cfg.k,
                   "n_ih": cfg.n_ih, "c_I": cfg.c_I, "window": cfg.W, "replicas": R,
                   "timing": f"hip graphs of {R} steps (one per replica), rotating replicas",
                   "streams": ("one" if wl.s_hca is None or len(wl.layers) < 2 else
                               "two: HCA attention concurrent with the CSA indexer and attention"),
                   **({"attention_sink": "per-head, N(0, 2^2)"} if args.sink else {}),
                   **({"indexer_keys": "MX FP4 (E2M1, E8M0 per 32), FP8 queries"} if args.fp4_keys else {}),
                   **({"norm_rope": "RMSNorm + RoPE on the last 64 dims: entries when pooled, new window rows, queries inside attention"}
                      if args.norm_rope else {})},
        "hbm_gbs": round(abytes / sec / 1e9, 1),
        "hbm_frac": round(abytes / sec / 1e9 / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_step": abytes,
        "tflops": {"fp8": round(f8 / sec / 1e12, 2), "bf16": round(bf / sec / 1e12, 2)},
        # matrix-core use of the whole step: all FLOPs against the bf16 peak, and each
        # dtype's FLOPs against its own peak (the fraction of the step the matrix cores
        # would need at peak)
        "mfma_frac": {"all_vs_bf16_peak": round((f8 + bf) / sec / 1e12 / BF16_PEAK_TFLOPS, 4),
                      "per_dtype_peak": round((f8 / FP8_PEAK_TFLOPS + bf / BF16_PEAK_TFLOPS)
                                              / sec / 1e12, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
