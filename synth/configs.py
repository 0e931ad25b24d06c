"""The five synthetic workloads (shapes, dtypes, rotation, budget).

Model-shaped layers stand in for the models the pages evaluate on
(Llama-3.1-8B, Qwen2.5-7B); no weights or datasets are involved.
"""
from dataclasses import dataclass, field


@dataclass(frozen=True)
class Config:
    idx: int
    name: str
    batch: int
    n_kv_heads: int
    n_q_heads: int
    n_tokens: int
    dtype: str          # "f32" or "bf16"
    rotation: str       # "klt", "wht"
    bits_per_elem: float
    marginal: str = "gauss"   # "gauss" or "t3"
    d: int = 128
    n_calib: int = 1024
    decode_steps: int = 1
    n_layers: int = 1   # layers whose caches a timed step sweeps (HBM, not the 256 MB cache)
    notes: dict = field(default_factory=dict)

    @property
    def group(self):
        return self.n_q_heads // self.n_kv_heads


CONFIGS = {
    1: Config(1, "tiny-fp32-klt-2.0", 1, 1, 1, 4096, "f32", "klt", 2.0),
    2: Config(2, "llama3.1-8b-layer-32k-klt-2.76", 1, 8, 32, 32768, "bf16", "klt", 2.76,
              n_layers=32),
    3: Config(3, "batch16-8k-klt-4.0-append", 16, 8, 32, 8192, "bf16", "klt", 4.0,
              decode_steps=64, n_layers=4),
    4: Config(4, "qwen2.5-7b-layer-128k-wht-1.33", 1, 4, 28, 131072, "bf16", "wht", 1.33,
              marginal="t3", n_layers=28),
    5: Config(5, "llama-shape-128k-tiers", 1, 8, 32, 131072, "bf16", "klt", 2.76,
              decode_steps=256, n_layers=8),
}
