"""Workload table for the Flash-Cache denoising step.

The method (Flash-dLLM, arXiv 2609.26796; figure captions page, Fig. 2) runs one
fixed-size query of beta_m tokens per sequence -- the current masked window plus
the top-k tracked decoded positions -- against that sequence's whole KV cache.
The pages give no model shapes; the shapes below are LLaDA-8B-like layers
(d_model 4096, 32 MHA heads of 128) and a tiny fp32 case.

Names C0..C4 follow the order of the workload list:
  C0  tiny fp32 step (d=256, 4 heads x 64), B=1, cache 128, query 32
  C1  one LLaDA-8B-shaped layer, bf16, B=1, cache 768, query 128
  C2  batched varlen step, bf16, B=32, caches 768..1536, query 128 each
  C3  C2's batch through 32 layers x 32 denoising steps (block length 16)
  C4  Flash-Verify-shaped step: B=32, cache 4096, two views, vocab 126464
"""
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class StepConfig:
    name: str
    seed: int
    batch: int
    d_model: int
    n_heads: int
    head_dim: int
    dtype: str                      # "f32" or "bf16" (interface and storage dtype)
    rope_base: float
    # prompt length: fixed, or uniform integer range [lo, hi] per sequence
    prompt: Tuple[int, int]
    gen_len: int                    # generated positions per sequence
    window: int                     # masked-window tokens in the query
    track: int                      # tracking budget k
    page_size: int = 16
    # multi-layer / multi-step driver (C3)
    layers: int = 1
    steps: int = 1
    block_len: int = 16
    # verify-shaped step (C4)
    verify: bool = False
    verify_len: Tuple[int, int] = (0, 0)   # uniform range of verified positions per sequence
    vocab: int = 0
    tau: float = 0.9
    planted_frac: float = 0.3
    logit_std: float = 2.0
    hidden_std: float = 1.0
    weight_std: float = 0.02
    cache_len_fixed: Optional[int] = None  # C4: every cache has this length
    rms_eps: float = 1e-5           # layer-input RMS normalisation of the layer stack
    extra: dict = field(default_factory=dict)

    @property
    def beta_m(self) -> int:
        return self.window + self.track

    @property
    def kv_std(self) -> float:
        # prefill scale of the stale cache: the projection of N(0,1) states by
        # N(0, weight_std) weights has std sqrt(d) * weight_std
        return (self.d_model ** 0.5) * self.weight_std


C0 = StepConfig(name="C0", seed=0, batch=1, d_model=256, n_heads=4, head_dim=64,
                dtype="f32", rope_base=10000.0, prompt=(64, 64), gen_len=64,
                window=16, track=16)
C1 = StepConfig(name="C1", seed=1, batch=1, d_model=4096, n_heads=32, head_dim=128,
                dtype="bf16", rope_base=500000.0, prompt=(512, 512), gen_len=256,
                window=64, track=64)
C2 = StepConfig(name="C2", seed=2, batch=32, d_model=4096, n_heads=32, head_dim=128,
                dtype="bf16", rope_base=500000.0, prompt=(256, 1024), gen_len=512,
                window=64, track=64)
C3 = StepConfig(name="C3", seed=3, batch=32, d_model=4096, n_heads=32, head_dim=128,
                dtype="bf16", rope_base=500000.0, prompt=(256, 1024), gen_len=512,
                window=16, track=48, layers=32, steps=32, block_len=16)
C4 = StepConfig(name="C4", seed=4, batch=32, d_model=4096, n_heads=32, head_dim=128,
                dtype="bf16", rope_base=500000.0, prompt=(0, 0), gen_len=0,
                window=0, track=0, verify=True, verify_len=(16, 128), vocab=126464,
                tau=0.9, cache_len_fixed=4096)

CONFIGS = {c.name: c for c in (C0, C1, C2, C3, C4)}


def small_variant(cfg: StepConfig, **kw) -> StepConfig:
    """A shrunken copy of a config (same structure, smaller sizes) for fast tests."""
    return replace(cfg, **kw)
