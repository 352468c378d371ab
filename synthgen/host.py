"""Seeded NumPy generation of one synthetic problem (host memory).

Used for sizes the CPU oracle can check element by element.  Every tensor is drawn in
float32 from its own child stream of ``SeedSequence(cfg.seed)``, then stored in the
config's storage format.  Arrays of storage codes are returned (uint16 for bfloat16,
uint8 for FP8 E4M3FN, float32 otherwise), together with the float32 source values of
the few tensors that are needed to construct planted keys.

Distributions (stated with each workload): raw KV ~ N(0, kv_std^2); gate logits, query
and indexer vectors ~ N(0, 1); indexer head weights ~ U(0, 1).  Planted indexer keys
(decode workloads with ``plants > 0``) are u + N(0, noise^2) where u is the query's
head-weighted indexer vector sum_h w_h q_h rescaled to norm sqrt(c_I); their entry
positions are drawn without replacement from the visible entries.
"""
import numpy as np

from .codecs import f32_to_bf16_bits, f32_to_e4m3fn_bits, f32_to_mxfp4
from .configs import BF16, F32, FP8, MXFP4

_STREAMS = ["X_csa", "Z_csa", "X_hca", "Z_hca", "Q_csa", "Q_hca", "qI", "w", "KI",
            "plant_pos", "plant_noise"]


def encode(x, dtype):
    if dtype == F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == BF16:
        return f32_to_bf16_bits(x)
    if dtype == FP8:
        return f32_to_e4m3fn_bits(x)
    raise ValueError(dtype)


def _rngs(seed):
    kids = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return {name: np.random.default_rng(s) for name, s in zip(_STREAMS, kids)}


def layers_of(cfg):
    return {"csa_decode": ("csa",), "hca_decode": ("hca",),
            "prefill": ("csa", "hca"), "pair_decode": ("csa", "hca"),
            # the indexer's inputs only (no raw KV, queries or gates)
            "index_decode": ("index",), "index_prefill": ("index",)}[cfg.kind]


def make_problem(cfg):
    """Return a dict describing one problem: inputs (storage codes) and positions.

    Sequence layout: every sequence holds ``n_total = n + Tq`` raw tokens for prefill
    (old context followed by the new chunk) and ``n`` tokens for decode; the query tokens
    are the last ``Tq`` positions, so ``q_pos[b] = n_total - Tq``.
    """
    r = _rngs(cfg.seed)
    B, c = cfg.B, cfg.c
    Tq = cfg.Tq
    n_total = cfg.n + (Tq if cfg.kind in ("prefill", "index_prefill") else 0)
    lay = layers_of(cfg)
    out = {"cfg": cfg, "n_total": n_total, "Tq": Tq}
    out["q_pos"] = np.full((B,), n_total - Tq, dtype=np.int32)

    def normal(name, shape, std=1.0):
        return (r[name].standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)

    if "csa" in lay or "hca" in lay:
        X = normal("X_csa", (B, n_total, c), cfg.kv_std)
    if "csa" in lay:
        out["X_csa"] = encode(X, cfg.dtype)
        out["Z_csa"] = encode(normal("Z_csa", (B, n_total, c)), cfg.dtype)
        out["Q_csa"] = encode(normal("Q_csa", (B, Tq, cfg.n_h, c)), cfg.dtype)
    if "hca" in lay:
        if cfg.kind == "prefill":
            out["X_hca"] = out["X_csa"]          # both branches read the same raw chunk
        else:
            out["X_hca"] = encode(normal("X_hca", (B, n_total, c), cfg.kv_std), cfg.dtype)
        out["Z_hca"] = encode(normal("Z_hca", (B, n_total, c)), cfg.dtype)
        if cfg.kind == "prefill":
            out["Q_hca"] = out["Q_csa"]
        else:
            out["Q_hca"] = encode(normal("Q_hca", (B, Tq, cfg.n_h, c)), cfg.dtype)
    if "csa" in lay or "index" in lay:
        N_c = n_total // cfg.m
        qI = normal("qI", (B, Tq, cfg.n_ih, cfg.c_I))
        w = r["w"].random((B, Tq, cfg.n_ih), dtype=np.float32)
        KI = normal("KI", (B, N_c, cfg.c_I))
        if cfg.plants > 0:
            if Tq != 1:
                raise ValueError("planted keys are defined for single-token decode only")
            V = min(N_c, (n_total - 1 + 1) // cfg.m)
            for b in range(B):
                pos = r["plant_pos"].choice(V, size=min(cfg.plants, V), replace=False)
                u = (w[b, 0, :, None] * qI[b, 0]).sum(0)
                u = u * np.float32(np.sqrt(cfg.c_I) / np.linalg.norm(u))
                noise = r["plant_noise"].standard_normal((len(pos), cfg.c_I), dtype=np.float32)
                KI[b, pos] = u[None, :] + np.float32(cfg.plant_noise) * noise
                out.setdefault("plant_positions", []).append(np.sort(pos))
        if cfg.idx_dtype == MXFP4:  # FP8 queries; keys as MX FP4 rows and their scales
            out["qI"] = encode(qI, FP8)
            out["KI"], out["KI_scales"] = f32_to_mxfp4(KI)
        else:
            out["qI"] = encode(qI, cfg.idx_dtype)
            out["KI"] = encode(KI, cfg.idx_dtype)
        out["w"] = w
    return out
