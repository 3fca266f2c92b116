"""The five synthetic single-layer workloads.

Shapes follow the long-context settings the KV-cache compression pages evaluate on
(Llama-3-8B-like and Qwen-like GQA layers, 8k to 128k contexts).  The models and datasets
themselves are not available, so every tensor is drawn from a seeded generator
(see ``workloads.gen``) with the structure listed per config.
"""

from dataclasses import dataclass, field
from typing import Optional


@dataclass(frozen=True)
class WorkloadConfig:
    index: int
    name: str
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_keys: int
    n_queries: int
    mode: str                      # "sum" (RDKV w_t) or "max" (KVzip+ s+)
    avg_bits: Optional[float]      # V/K stage budget, bits per element (sum mode)
    keep_fraction: Optional[float]  # top-k keep ratio (max mode)
    fidelity_rows: int             # last query rows used by the fidelity attend
    hidden_dim: int = 0            # D_h (max mode only)
    k_outliers: bool = False       # 4 random K channels per KV head scaled x10
    k_drift: bool = False          # 0.5*sin(t/1000) added to channels c < d/2 of K
    group_size: int = 32
    notes: str = field(default="", compare=False)

    @property
    def gqa(self) -> int:
        return self.n_q_heads // self.n_kv_heads


CONFIGS = (
    WorkloadConfig(0, "tiny_d64_n256", 1, 1, 64, 256, 256, "sum", 4.0, None, 256,
                   notes="Q,K,V ~ N(0,1); one head"),
    WorkloadConfig(1, "llama8b_prefill_n8192", 32, 8, 128, 8192, 8192, "sum", 3.0, None, 64,
                   k_outliers=True,
                   notes="Q,V ~ N(0,1); K ~ N(0,1) with 4 outlier channels per KV head x10"),
    WorkloadConfig(2, "long_prefill_n32768", 32, 8, 128, 32768, 32768, "sum", 2.5, None, 64,
                   k_drift=True,
                   notes="K_t = N(0,1) + 0.5 sin(t/1000) on channels c < 64"),
    WorkloadConfig(3, "kvzip_qwen_n16384", 28, 4, 128, 16384, 16384, "max", None, 0.25, 64,
                   hidden_dim=3584,
                   notes="Q,K,V,hidden ~ N(0,1); W_O ~ N(0, 1/3584); top-25% per KV head"),
    WorkloadConfig(4, "decode_cache_n131072_q512", 32, 8, 128, 131072, 512, "sum", 2.0, None, 512,
                   k_outliers=True,
                   notes="K outliers as config 1; the last 512 positions query the cache"),
)


def get_config(i: int) -> WorkloadConfig:
    return CONFIGS[i]
