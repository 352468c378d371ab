"""Seeded generation of full-size problems directly in GPU memory (torch's Philox RNG).

Same distributions and planting rule as ``synthgen.host`` (see its docstring); used for
the workload sizes the host cannot generate in reasonable time.  Storage: bfloat16 data
is returned as int16 tensors holding the bf16 bit patterns, FP8 E4M3FN as uint8 codes
(clamped to +-448 before the cast), float32 as float32.  Only random numbers and storage
conversion happen here.
"""
import torch

from .configs import BF16, F32, FP8
from .host import layers_of


def _store(x, dtype):
    if dtype == F32:
        return x.float().contiguous()
    if dtype == BF16:
        return x.to(torch.bfloat16).view(torch.int16).contiguous()
    if dtype == FP8:
        return x.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
    raise ValueError(dtype)


def _normal(gen, shape, std, dtype, device, chunk_rows=1 << 20):
    """N(0, std^2) stored as `dtype`, generated in row chunks to bound fp32 temporaries."""
    out = torch.empty(shape, dtype={F32: torch.float32, BF16: torch.int16, FP8: torch.uint8}[dtype],
                      device=device)
    flat = out.view(-1, shape[-1])
    for r0 in range(0, flat.shape[0], chunk_rows):
        r1 = min(flat.shape[0], r0 + chunk_rows)
        x = torch.randn((r1 - r0, shape[-1]), generator=gen, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        flat[r0:r1] = _store(x, dtype)
    return out


def make_problem_device(cfg, device="cuda"):
    """Same layout and keys as ``synthgen.host.make_problem`` but as device tensors."""
    gen = torch.Generator(device=device)
    gen.manual_seed(cfg.seed)
    B, c, Tq = cfg.B, cfg.c, cfg.Tq
    n_total = cfg.n + (Tq if cfg.kind == "prefill" else 0)
    lay = layers_of(cfg)
    out = {"cfg": cfg, "n_total": n_total, "Tq": Tq}
    out["q_pos"] = torch.full((B,), n_total - Tq, dtype=torch.int32, device=device)
    if "csa" in lay:
        out["X_csa"] = _normal(gen, (B, n_total, c), cfg.kv_std, cfg.dtype, device)
        out["Z_csa"] = _normal(gen, (B, n_total, c), 1.0, cfg.dtype, device)
        out["Q_csa"] = _normal(gen, (B, Tq, cfg.n_h, c), 1.0, cfg.dtype, device)
    if "hca" in lay:
        if cfg.kind == "prefill":
            out["X_hca"] = out["X_csa"]
            out["Q_hca"] = out["Q_csa"]
        else:
            out["X_hca"] = _normal(gen, (B, n_total, c), cfg.kv_std, cfg.dtype, device)
        out["Z_hca"] = _normal(gen, (B, n_total, c), 1.0, cfg.dtype, device)
        if cfg.kind != "prefill":
            out["Q_hca"] = _normal(gen, (B, Tq, cfg.n_h, c), 1.0, cfg.dtype, device)
    if "csa" in lay:
        N_c = n_total // cfg.m
        qI = torch.randn((B, Tq, cfg.n_ih, cfg.c_I), generator=gen, device=device)
        w = torch.rand((B, Tq, cfg.n_ih), generator=gen, device=device)
        KI = _normal(gen, (B, N_c, cfg.c_I), 1.0, cfg.idx_dtype, device)
        if cfg.plants > 0:
            if Tq != 1:
                raise ValueError("planted keys are defined for single-token decode only")
            V = min(N_c, n_total // cfg.m)
            plants = []
            for b in range(B):
                pos = torch.randperm(V, generator=gen, device=device)[:cfg.plants]
                u = (w[b, 0, :, None] * qI[b, 0]).sum(0)
                u = u * (cfg.c_I ** 0.5 / u.norm())
                noise = torch.randn((pos.numel(), cfg.c_I), generator=gen, device=device)
                KI[b, pos] = _store(u[None, :] + cfg.plant_noise * noise, cfg.idx_dtype)
                plants.append(torch.sort(pos).values)
            out["plant_positions"] = plants
        out["qI"] = _store(qI, cfg.idx_dtype)
        out["w"] = w.contiguous()
        out["KI"] = KI
    return out
