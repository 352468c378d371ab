"""Seeded generation of full-size problems directly in GPU memory (torch's Philox RNG).

Same distributions and planting rule as ``synthgen.host`` (see its docstring); used for
the workload sizes the host cannot generate in reasonable time.  Storage: bfloat16 data
is returned as int16 tensors holding the bf16 bit patterns, FP8 E4M3FN as uint8 codes
(clamped to +-448 before the cast), float32 as float32.  Only random numbers and storage
conversion happen here.
"""
import torch

from .configs import BF16, F32, FP8, MXFP4
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


def _mxfp4(x, chunk_rows=1 << 16):
    """MX FP4 encoding of float32 rows [..., K] (K % 32 == 0), as ``synthgen.codecs`` defines
    it: returns (packed uint8 [..., K/2], scales uint8 [..., K/32]).  Nearest value with
    ties to even: below 2 the grid step is 0.5, below 4 it is 1, above it 2, and torch's
    round() rounds halves to even, which is the even code on each of these grids."""
    K = x.shape[-1]
    flat = x.reshape(-1, K)
    packed = torch.empty((flat.shape[0], K // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((flat.shape[0], K // 32), dtype=torch.uint8, device=x.device)
    for r0 in range(0, flat.shape[0], chunk_rows):
        blk = flat[r0:r0 + chunk_rows].float().reshape(-1, K // 32, 32)
        amax = blk.abs().amax(-1)
        _, E = torch.frexp(torch.where(amax > 0, amax, torch.ones_like(amax)))
        X = torch.where(amax > 0, E - 3, torch.full_like(E, -127)).clamp(-127, 127)
        v = blk / torch.exp2(X.float())[..., None]
        a = v.abs().clamp(max=6.0)
        q = torch.where(a < 2, torch.round(a * 2) / 2, torch.where(a < 4, torch.round(a), torch.round(a / 2) * 2))
        code = torch.where(q < 2, q * 2, torch.where(q < 4, q + 2, torch.where(q < 5, 6.0, 7.0))).to(torch.uint8)
        nib = (code | (torch.signbit(v).to(torch.uint8) << 3)).reshape(blk.shape[0], K)
        packed[r0:r0 + chunk_rows] = nib[:, 0::2] | (nib[:, 1::2] << 4)
        scales[r0:r0 + chunk_rows] = (X + 127).to(torch.uint8)
    return packed.reshape(x.shape[:-1] + (K // 2,)), scales.reshape(x.shape[:-1] + (K // 32,))


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
        f4 = cfg.idx_dtype == MXFP4  # keys drawn in fp32, encoded after planting
        KI = _normal(gen, (B, N_c, cfg.c_I), 1.0, F32 if f4 else cfg.idx_dtype, device)
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
                KI[b, pos] = _store(u[None, :] + cfg.plant_noise * noise, F32 if f4 else cfg.idx_dtype)
                plants.append(torch.sort(pos).values)
            out["plant_positions"] = plants
        out["w"] = w.contiguous()
        if f4:
            out["qI"] = _store(qI, FP8)
            out["KI"], out["KI_scales"] = _mxfp4(KI)
            del KI
        else:
            out["qI"] = _store(qI, cfg.idx_dtype)
            out["KI"] = KI
    return out
