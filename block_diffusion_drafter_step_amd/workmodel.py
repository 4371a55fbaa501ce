"""Algorithmic work of each call: the bytes the method must move and the flops
it must do, with every weight read once and the KV cache read once.

These figures are what throughput and roofline fractions are computed from.
They count no intermediate the implementation chooses to write (split-K
partials, fp32 norm inputs), so a measured rate against them is never
flattered by extra traffic.
"""
from __future__ import annotations

ACT_BYTES = {"f32": 4, "bf16": 2}


def weight_bytes(rows: int, cols: int, dtype: str) -> int:
    if dtype == "q8_0":
        return rows * cols + rows * (cols // 32) * 2   # int8 codes + one fp16 per 32
    return rows * cols * ACT_BYTES[dtype]


def inject_flops(n: int, L_t: int, d_t: int, d: int, kv: int) -> int:
    """fc over the concatenated features plus the Wk and Wv projections."""
    return 2 * n * (L_t * d_t * d + 2 * kv * d)


def fc_flops(n: int, fc_in: int, fc_out: int) -> int:
    return 2 * n * fc_in * fc_out


def inject_bytes(cfg, n: int, kv: str = None) -> int:
    a = ACT_BYTES[cfg.act]
    return (n * cfg.L_t * cfg.d_t * a                      # features
            + weight_bytes(cfg.d, cfg.fc_in, cfg.weight)   # fc
            + 2 * weight_bytes(cfg.kv, cfg.d, cfg.weight)  # Wk, Wv
            + 2 * n * cfg.Hkv * kv_row_bytes(cfg, kv))     # cache rows written


def conv_bytes(cfg, n_blocks: int = 1) -> int:
    a = ACT_BYTES[cfg.act]
    return (2 * n_blocks * cfg.B * cfg.C * a               # x in, u out
            + cfg.T * cfg.C * a                            # base
            + weight_bytes(cfg.T * cfg.G, cfg.C, cfg.act))  # W_delta


def ffn_bytes(cfg, n_blocks: int = 1) -> int:
    """The feed-forward site: h in, out, its conv pair and the gate, up and
    down weights."""
    a = ACT_BYTES[cfg.act]
    return (2 * n_blocks * cfg.B * cfg.d * a
            + cfg.T * cfg.d * a + weight_bytes(cfg.T * cfg.G, cfg.d, cfg.act)
            + 2 * weight_bytes(cfg.d_ff, cfg.d, cfg.weight) + weight_bytes(cfg.d, cfg.d_ff, cfg.weight))


def attn_weight_bytes(cfg) -> int:
    return (weight_bytes(cfg.qdim, cfg.d, cfg.weight) + 2 * weight_bytes(cfg.kv, cfg.d, cfg.weight)
            + weight_bytes(cfg.d, cfg.qdim, cfg.weight))


def kv_row_bytes(cfg, kv: str = None) -> int:
    """Bytes of one cached position of one KV head, for K or for V: the act
    type, or Q8_0 codes plus one fp16 scale per 32 dims."""
    if kv == "q8_0":
        return cfg.hd + (cfg.hd // 32) * 2
    return cfg.hd * ACT_BYTES[cfg.act]


def attn_kv_bytes(cfg, n_ctx: int, kv: str = None) -> int:
    return 2 * cfg.Hkv * n_ctx * kv_row_bytes(cfg, kv)


def attn_bytes(cfg, n_ctx: int, kv: str = None) -> int:
    a = ACT_BYTES[cfg.act]
    return attn_weight_bytes(cfg) + attn_kv_bytes(cfg, n_ctx, kv) + 3 * cfg.B * cfg.d * a


def attn_core_bytes(cfg, n_ctx: int, kv: str = None) -> int:
    """What the attention kernels alone must move: KV plus Q in, O out."""
    a = ACT_BYTES[cfg.act]
    return attn_kv_bytes(cfg, n_ctx, kv) + 2 * cfg.B * cfg.qdim * a + 2 * cfg.B * cfg.kv * a


def lmhead_bytes(cfg) -> int:
    a = ACT_BYTES[cfg.act]
    return weight_bytes(cfg.V, cfg.d, cfg.weight) + cfg.B * cfg.d * a + cfg.B * cfg.K * 8


def lmhead_flops(cfg) -> int:
    return 2 * cfg.B * cfg.V * cfg.d


def selector_bytes(cfg) -> int:
    a = ACT_BYTES[cfg.act]
    return (cfg.r * cfg.d * a + cfg.B * cfg.d * a + 2 * cfg.B * cfg.K * cfg.r * a
            + cfg.B * cfg.K * cfg.K * 4)


def selector_params(V: int, r: int) -> int:
    """Parameters of the two materialised selector codebooks [V][r]."""
    return 2 * V * r


def selector_params_factorised(d: int, r: int) -> int:
    """Predecessor / successor projections of a [.][d] embedding plus the hidden
    projection, all to rank r."""
    return 3 * d * r


def step_bytes(cfg, n_ctx: int, inject_n: int = 0, kv: str = None) -> int:
    """One block step (conv, attention over n_ctx context keys plus the block,
    LM head, selector, accept), plus an injection of inject_n rows when the
    step injects; kv = "q8_0" for a Q8_0 KV cache."""
    b = conv_bytes(cfg) + attn_bytes(cfg, n_ctx, kv) + lmhead_bytes(cfg) + selector_bytes(cfg)
    if inject_n:
        b += inject_bytes(cfg, inject_n, kv)
    return b
