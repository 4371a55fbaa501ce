"""The five seeded synthetic workloads of the DFlash / DFlash2 draft block step.

Each workload fixes the draft layer's shapes, the storage types and a seed.
The shapes follow the pages' settings: a Qwen-27B-class draft width, blocks of
8 or 16 drafted tokens, and 1k / 32k / 64k injected contexts ("dflash: port
#219 onto feature", benchmark sweep; "spec : add DFlash2 support", Overview
table). Nothing here does arithmetic of the method.

Field names follow the pages' notation:
  d      draft hidden width              d_t   target hidden width
  L_t    number of target layers whose hidden states are concatenated
  n_ctx  context tokens injected before the block step
  B      block size (drafted tokens per block)
  Hq/Hkv query / key-value heads         hd    head dim
  C/G/T  conv channels / groups / taps   V     vocabulary
  K      top-K candidates per position   r     selector rank
  d_ff   width of the feed-forward site's gated MLP (the pages give none:
         17408 at d = 5120 and 21504 at d = 5376, widths of public model
         families at those d; 512 in the tiny fp32 config)
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class Config:
    name: str
    seed: int
    act: str                  # "f32" or "bf16": activations, KV cache, conv base, codebooks
    weight: str               # "f32", "bf16" or "q8_0": fc, Wq, Wk, Wv, Wo, LM head
    d: int
    d_t: int
    L_t: int
    n_ctx: int
    B: int
    Hq: int
    Hkv: int
    hd: int
    C: int
    G: int
    T: int
    V: int
    K: int
    r: int
    d_ff: int = 0
    eps: float = 1e-6
    # long-context decode regime: rows of seeded K/V already in the cache,
    # tokens injected per step and number of steps
    prefill_kv: int = 0
    inject_per_step: int = 0
    steps: int = 1
    capacity: int = 0
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def kv(self) -> int:
        return self.Hkv * self.hd

    @property
    def qdim(self) -> int:
        return self.Hq * self.hd

    @property
    def fc_in(self) -> int:
        return self.L_t * self.d_t

    @property
    def cap(self) -> int:
        """KV-cache capacity in rows (a multiple of 64, as the library requires)."""
        if self.capacity:
            return -(-self.capacity // 64) * 64
        return -(-(self.prefill_kv + self.n_ctx + self.inject_per_step * self.steps + 64) // 64) * 64


def _qwen27b(**kw) -> Config:
    base = dict(act="bf16", weight="bf16", d=5120, d_t=5120, L_t=5, B=16,
                Hq=32, Hkv=8, hd=128, C=5120, G=64, T=4, V=151936, K=8, r=64, d_ff=17408)
    base.update(kw)
    return Config(**base)


CONFIGS: list[Config] = [
    Config(name="c0_tiny_fp32", seed=0, act="f32", weight="f32", d=256, d_t=256, L_t=2,
           n_ctx=64, B=8, Hq=4, Hkv=2, hd=64, C=256, G=8, T=4, V=1024, K=4, r=16, d_ff=512,
           notes="tiny fp32 step; the oracle finishes it in well under a second"),
    _qwen27b(name="c1_qwen27b_1k", seed=1, n_ctx=1024,
             notes="one Qwen-27B-shaped draft layer, 1024 injected tokens"),
    _qwen27b(name="c2_prefill_32k", seed=2, n_ctx=32768,
             notes="32768-token prefill injection, then one block step over 32768+16 keys"),
    _qwen27b(name="c3_decode_64k", seed=3, n_ctx=0, prefill_kv=65536, inject_per_step=16,
             steps=64, capacity=65536 + 1024,
             notes="cache pre-filled with 65536 seeded K/V rows; each step injects 16 rows, "
                   "then runs a block step; 64 steps"),
    Config(name="c4_q8_0_32k", seed=4, act="bf16", weight="q8_0", d=5376, d_t=5376, L_t=5,
           n_ctx=32768, B=8, Hq=32, Hkv=8, hd=128, C=5376, G=64, T=4, V=262144, K=8, r=64, d_ff=21504,
           notes="Q8_0 fc / Wq / Wk / Wv / Wo / LM head, bf16 activations, 32768-token context"),
]

BY_NAME = {c.name: c for c in CONFIGS}


def get(i_or_name) -> Config:
    if isinstance(i_or_name, int):
        return CONFIGS[i_or_name]
    return BY_NAME[i_or_name]


def shrink(cfg: Config, **kw) -> Config:
    """A copy with some fields replaced (used for small parity cases)."""
    return replace(cfg, **kw)
