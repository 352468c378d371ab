"""The five synthetic workloads, with the shapes the DeepSeek-V4 pages give.

Shapes follow the Pro/Flash settings (Course 1: Architecture, "Model configurations"
table: m = 4, m' = 128, top-k 1024 / 512, 64 indexer heads of dim 128, 128 / 64 query
heads of dim 512, window 128) and the decode / prefill regimes described in the
lesson "DeepSeek-V4: Anatomy of an Open-Source Frontier Model" (section "One query in
a CSA layer, step by step").
"""
from dataclasses import dataclass, replace

F32, BF16, FP8, MXFP4 = 0, 1, 2, 3  # MXFP4: indexer keys only (queries stay FP8)


@dataclass(frozen=True)
class Config:
    name: str
    kind: str            # "csa_decode" | "hca_decode" | "prefill" | "pair_decode"
    B: int               # sequences
    n: int               # raw context length (decode) or old context length (prefill)
    c: int               # KV / query head dim (one shared KV head)
    m: int = 4           # CSA block size
    m_hca: int = 128     # HCA block size
    n_ih: int = 64       # indexer heads
    c_I: int = 128       # indexer dim
    k: int = 512         # top-k
    n_h: int = 64        # query heads
    W: int = 128         # sliding window
    dtype: int = BF16    # attention / KV dtype
    idx_dtype: int = FP8 # indexer dtype
    kv_std: float = 1.0  # raw KV ~ N(0, kv_std^2)
    plants: int = 0      # planted indexer keys per sequence
    plant_noise: float = 0.1
    Tq: int = 1          # query tokens per sequence (prefill chunk length)
    seed: int = 0

    @property
    def N_c(self):
        return self.n // self.m

    @property
    def N_h(self):
        return self.n // self.m_hca

    def scaled(self, **kw):
        return replace(self, **kw)


CONFIGS = {
    1: Config(name="tiny_csa_decode_fp32", kind="csa_decode", B=1, n=4096, c=64, m=4,
              n_ih=4, c_I=32, k=64, n_h=8, W=128, dtype=F32, idx_dtype=F32,
              kv_std=1.0 / 8.0, seed=1001),
    2: Config(name="hca_decode_bf16_128k", kind="hca_decode", B=16, n=131072, c=512,
              m_hca=128, n_h=64, W=128, kv_std=1.0, seed=1002),
    3: Config(name="flash_csa_decode_128k", kind="csa_decode", B=32, n=131072, c=512, m=4,
              n_ih=64, c_I=128, k=512, n_h=64, W=128, kv_std=512 ** -0.5, plants=16,
              seed=1003),
    4: Config(name="csa_hca_prefill_8k_on_256k", kind="prefill", B=1, n=262144, c=512,
              m=4, m_hca=128, n_ih=64, c_I=128, k=512, n_h=64, W=128,
              kv_std=512 ** -0.5, Tq=8192, seed=1004),
    5: Config(name="pro_csa_hca_decode_1m", kind="pair_decode", B=4, n=1048576, c=512,
              m=4, m_hca=128, n_ih=64, c_I=128, k=1024, n_h=128, W=128,
              kv_std=512 ** -0.5, plants=64, seed=1005),
}


def get_config(i):
    return CONFIGS[int(i)]
