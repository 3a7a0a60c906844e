"""The five synthetic workloads of the IndexMem / MomentKV hot path.

Shapes follow the pages' evaluation models (Llama-3.1-8B-shaped layers for IndexMem,
the Qwen3-4B attention shape for MomentKV).  Sizes the pages leave open take the
plainest reading; each such choice is marked "reading".
"""
from dataclasses import dataclass, field, replace
from typing import Tuple


@dataclass(frozen=True)
class Config:
    name: str
    cfg_id: int
    dtype: str            # storage / input type: "f32" or "bf16"
    layers: int
    b: int                # batch
    D: int                # hidden size (0 = no hidden states, MomentKV)
    H_q: int
    H_kv: int
    d: int                # head dim
    L: int                # prefill length
    H_I: int = 0          # indexer heads
    d_I: int = 0          # indexer dim
    W: int = 64           # observation window (last W prefill positions are the queries)
    B: int = 0            # retained budget
    R: int = 0            # recent window
    recent_inclusive: bool = True   # True: R counts inside B; False: B plus R slots
    lam: float = 0.995    # memory decay
    T: int = 0            # decode steps
    needles: int = 0
    qkv_from_hidden: bool = False   # Q/K/V = X W^T (small configs) or drawn directly
    outlier_channels: int = 0       # channels per KV head scaled by outlier_scale (keys)
    outlier_scale: float = 8.0
    streaming: bool = False         # one eviction per decode step
    momentkv: bool = False
    budgets: Tuple[int, ...] = field(default_factory=tuple)  # MomentKV budgets
    eps_rms: float = 1e-6
    eps_mem: float = 1e-6

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    @property
    def keep(self) -> int:
        """Retained prefill slots after pre-eviction."""
        k = self.B if self.recent_inclusive else self.B + self.R
        return min(k, self.L)

    @property
    def n_evict(self) -> int:
        return self.L - self.keep

    @property
    def cap(self) -> int:
        """Cache capacity: retained prefill plus appended decode tokens."""
        return self.keep if self.streaming else self.keep + self.T

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


CFG1 = Config(name="tiny_fp32", cfg_id=1, dtype="f32", layers=1, b=1, D=256, H_q=1, H_kv=1,
              d=64, L=512, H_I=4, d_I=32, W=32, B=64, R=0, lam=0.99, T=16, needles=4,
              qkv_from_hidden=True)
CFG2 = Config(name="llama8b_layer_4k", cfg_id=2, dtype="bf16", layers=1, b=1, D=4096, H_q=32,
              H_kv=8, d=128, L=4096, H_I=32, d_I=64, W=64, B=410, R=32, lam=0.995, T=256,
              needles=16, qkv_from_hidden=True)
# Reading: W, R and lambda are not given for the 32-layer stack; they inherit the
# single-layer Llama-shaped workload's values.
CFG3 = Config(name="llama8b_32L_16k_b8", cfg_id=3, dtype="bf16", layers=32, b=8, D=4096,
              H_q=32, H_kv=8, d=128, L=16384, H_I=32, d_I=64, W=64, B=1638, R=32, lam=0.995,
              T=512, needles=16)
CFG4 = Config(name="llama8b_layer_131k_stream", cfg_id=4, dtype="bf16", layers=1, b=1, D=4096,
              H_q=32, H_kv=8, d=128, L=131072, H_I=32, d_I=64, W=64, B=1024, R=64,
              recent_inclusive=False, lam=0.995, T=2048, outlier_channels=3, streaming=True)
CFG5 = Config(name="qwen3_4b_momentkv_32k", cfg_id=5, dtype="bf16", layers=36, b=4, D=0,
              H_q=32, H_kv=8, d=128, L=32768, W=64, B=128, R=0, T=256, momentkv=True,
              budgets=(128, 256, 512, 1024))

WORKLOADS = {c.name: c for c in (CFG1, CFG2, CFG3, CFG4, CFG5)}


def workload(name: str) -> Config:
    return WORKLOADS[name]
