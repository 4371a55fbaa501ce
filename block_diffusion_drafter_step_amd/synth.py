"""Seeded synthetic inputs for the draft block step.

This module only draws random numbers and packs them into the storage
formats the library reads (fp32, bf16 bit patterns, Q8_0 int8 + fp16 scales).
It holds none of the method's arithmetic, so that the CPU oracle and the GPU
path can both take their inputs from it without sharing any computation.

Every tensor has its own random stream, derived from the workload seed and a
CRC of the tensor's name, and large tensors are drawn in row chunks that each
have their own sub-stream.  Any row of any tensor can therefore be re-drawn
on its own, which is how sampled-row checks at full size get their inputs.

Distributions (the variance reading of N(0, s)): weights N(0, 1/fan_in),
hidden states and block inputs N(0, 1), conv base N(0, 0.5), selector
codebooks N(0, 1/4), pre-filled K/V N(0, 1), Q8_0 codes uniform integers in
[-127, 127] with per-block scales uniform in [0.001, 0.02] rounded to fp16.
"""
from __future__ import annotations

import os
import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

QBLOCK = 32                      # Q8_0 block length along the input dim
_CHUNK_ELEMS = 1 << 20           # elements per independently seeded chunk
_POOL = None


def _pool() -> ThreadPoolExecutor:
    global _POOL
    if _POOL is None:
        n = min(16, len(os.sched_getaffinity(0)))
        _POOL = ThreadPoolExecutor(max_workers=max(1, n))
    return _POOL


def _rng(seed: int, name: str, chunk: int = 0) -> np.random.Generator:
    key = (zlib.crc32(name.encode()), chunk)
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Pack float32 values as bf16 bit patterns, rounding to nearest even."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def _rows_per_chunk(ncols: int) -> int:
    return max(1, _CHUNK_ELEMS // max(1, ncols))


def _draw_rows(seed, name, nrows, ncols, r0, r1, draw):
    """Rows [r0, r1) of a [nrows][ncols] tensor, each chunk from its own stream."""
    rpc = _rows_per_chunk(ncols)
    c0, c1 = r0 // rpc, (r1 - 1) // rpc
    parts = []
    for c in range(c0, c1 + 1):
        lo, hi = c * rpc, min(nrows, (c + 1) * rpc)
        blk = draw(_rng(seed, name, c), (hi - lo, ncols))
        parts.append(blk[max(r0, lo) - lo: min(r1, hi) - lo])
    return np.concatenate(parts, axis=0) if len(parts) > 1 else parts[0]


def _fill(seed, name, shape, draw, out_dtype, convert=None):
    shape = tuple(int(s) for s in shape)
    ncols = shape[-1]
    nrows = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    out = np.empty((nrows, ncols), dtype=out_dtype)
    rpc = _rows_per_chunk(ncols)
    nchunks = (nrows + rpc - 1) // rpc

    def work(c):
        lo, hi = c * rpc, min(nrows, (c + 1) * rpc)
        blk = draw(_rng(seed, name, c), (hi - lo, ncols))
        out[lo:hi] = convert(blk) if convert else blk

    if nchunks == 1:
        work(0)
    else:
        list(_pool().map(work, range(nchunks)))
    return out.reshape(shape)


def normal(seed: int, name: str, shape, var: float, dtype: str = "bf16") -> np.ndarray:
    """N(0, var) values: float32 for dtype "f32", bf16 bit patterns (uint16) for "bf16"."""
    std = np.float32(np.sqrt(var))

    def draw(rng, shp):
        return rng.standard_normal(shp, dtype=np.float32) * std

    if dtype == "f32":
        return _fill(seed, name, shape, draw, np.float32)
    if dtype == "bf16":
        return _fill(seed, name, shape, draw, np.uint16, convert=f32_to_bf16_bits)
    raise ValueError(dtype)


def normal_rows(seed: int, name: str, shape, var: float, dtype: str, rows) -> np.ndarray:
    """The given rows of the 2-D tensor ``normal(seed, name, shape, var, dtype)``."""
    nrows, ncols = int(shape[0]), int(shape[1])
    std = np.float32(np.sqrt(var))

    def draw(rng, shp):
        return rng.standard_normal(shp, dtype=np.float32) * std

    out = []
    for r in rows:
        v = _draw_rows(seed, name, nrows, ncols, int(r), int(r) + 1, draw)
        out.append(f32_to_bf16_bits(v) if dtype == "bf16" else v.astype(np.float32))
    return np.concatenate(out, axis=0)


def q8_0(seed: int, name: str, rows: int, cols: int):
    """Q8_0 weight: int8 codes [rows][cols] and fp16 scales [rows][cols/32]."""
    if cols % QBLOCK:
        raise ValueError("Q8_0 needs cols % 32 == 0")

    def draw_q(rng, shp):
        return rng.integers(-127, 128, size=shp, dtype=np.int8)

    def draw_s(rng, shp):
        return rng.uniform(0.001, 0.02, size=shp).astype(np.float16)

    q = _fill(seed, name + ".q", (rows, cols), draw_q, np.int8)
    s = _fill(seed, name + ".s", (rows, cols // QBLOCK), draw_s, np.float16)
    return q, s


def integers(seed: int, name: str, low: int, high: int, shape) -> np.ndarray:
    """Uniform int32 values in [low, high)."""
    return _rng(seed, name).integers(low, high, size=shape, dtype=np.int64).astype(np.int32)


def distinct_indices(seed: int, name: str, rows: int, k: int, V: int) -> np.ndarray:
    """[rows][k] int32, each row k distinct values in [0, V)."""
    rng = _rng(seed, name)
    return np.stack([rng.choice(V, size=k, replace=False) for _ in range(rows)]).astype(np.int32)


def weight(seed: int, name: str, rows: int, cols: int, dtype: str) -> dict:
    """A weight of shape [out=rows][in=cols] drawn N(0, 1/cols), or Q8_0 codes."""
    if dtype == "q8_0":
        q, s = q8_0(seed, name, rows, cols)
        return {"dtype": "q8_0", "rows": rows, "cols": cols, "data": q, "scales": s}
    return {"dtype": dtype, "rows": rows, "cols": cols,
            "data": normal(seed, name, (rows, cols), 1.0 / cols, dtype), "scales": None}


def targets_with_mismatch(seed: int, name: str, path: np.ndarray, V: int):
    """Target tokens that agree with ``path`` up to a seeded first mismatch m ~ U{0..B}.

    Returns (targets [n_seq][B] int32, m [n_seq]).  At m < B the token is
    replaced by (path[m] + 1 + u) mod V, u ~ U{0..V-2}, so it always differs.
    """
    path = np.asarray(path, dtype=np.int64)
    n_seq, B = path.shape
    rng = _rng(seed, name)
    m = rng.integers(0, B + 1, size=n_seq)
    u = rng.integers(0, max(1, V - 1), size=n_seq)
    tgt = path.copy()
    for s in range(n_seq):
        if m[s] < B:
            tgt[s, m[s]] = (path[s, m[s]] + 1 + u[s]) % V
    return tgt.astype(np.int32), m.astype(np.int32)


class Workload:
    """Lazily drawn tensors of one config; each tensor is drawn once and cached."""

    def __init__(self, cfg):
        self.cfg = cfg
        self._cache = {}

    def _get(self, key, fn):
        if key not in self._cache:
            self._cache[key] = fn()
        return self._cache[key]

    def drop(self, *keys):
        for k in keys:
            self._cache.pop(k, None)

    # --- injection inputs --------------------------------------------------
    def hidden(self, layer: int, n: int | None = None, tag: str = "ctx"):
        c = self.cfg
        n = c.n_ctx if n is None else n
        nm = f"hidden.{tag}.{layer}"
        return self._get((nm, n), lambda: normal(c.seed, nm, (n, c.d_t), 1.0, c.act))

    def hidden_rows(self, layer: int, n: int, rows, tag: str = "ctx"):
        c = self.cfg
        return normal_rows(c.seed, f"hidden.{tag}.{layer}", (n, c.d_t), 1.0, c.act, rows)

    def fc(self):
        c = self.cfg
        return self._get("fc", lambda: weight(c.seed, "fc", c.d, c.fc_in, c.weight))

    def wq(self):
        c = self.cfg
        return self._get("wq", lambda: weight(c.seed, "wq", c.qdim, c.d, c.weight))

    def wk(self):
        c = self.cfg
        return self._get("wk", lambda: weight(c.seed, "wk", c.kv, c.d, c.weight))

    def wv(self):
        c = self.cfg
        return self._get("wv", lambda: weight(c.seed, "wv", c.kv, c.d, c.weight))

    def wo(self):
        c = self.cfg
        return self._get("wo", lambda: weight(c.seed, "wo", c.d, c.qdim, c.weight))

    def kv_prefill(self):
        """Seeded K and V rows already in the cache: [Hkv][prefill_kv][hd] each."""
        c = self.cfg
        shp = (c.Hkv, c.prefill_kv, c.hd)
        return self._get("kvp", lambda: (normal(c.seed, "kv_prefill.k", shp, 1.0, c.act),
                                         normal(c.seed, "kv_prefill.v", shp, 1.0, c.act)))

    # --- block-step inputs ---------------------------------------------------
    def x(self, n_blocks: int = 1, tag: str = "blk"):
        c = self.cfg
        nm = f"x.{tag}"
        return self._get((nm, n_blocks), lambda: normal(c.seed, nm, (n_blocks, c.B, c.d), 1.0, c.act))

    def conv_base(self):
        c = self.cfg
        return self._get("base", lambda: normal(c.seed, "conv_base", (c.T, c.C), 0.5, c.act))

    def w_delta(self):
        c = self.cfg
        # W_delta stays in the activation type (bf16 in the quantised config too)
        return self._get("wdelta", lambda: weight(c.seed, "w_delta", c.T * c.G, c.C, c.act))

    def w_lm(self):
        c = self.cfg
        return self._get("wlm", lambda: weight(c.seed, "w_lm", c.V, c.d, c.weight))

    def sel_proj(self):
        c = self.cfg
        return self._get("selP", lambda: weight(c.seed, "sel_P", c.r, c.d, c.act))

    def codebooks(self):
        c = self.cfg
        return self._get("cb", lambda: (normal(c.seed, "cb_pred", (c.V, c.r), 0.25, c.act),
                                        normal(c.seed, "cb_succ", (c.V, c.r), 0.25, c.act)))

    # --- feed-forward site (second conv pair and the gated MLP) --------------
    def h_ffn(self, n_blocks: int = 1, tag: str = "ffn"):
        c = self.cfg
        nm = f"h.{tag}"
        return self._get((nm, n_blocks), lambda: normal(c.seed, nm, (n_blocks, c.B, c.d), 1.0, c.act))

    def ffn_conv_base(self):
        c = self.cfg
        return self._get("ffn_base", lambda: normal(c.seed, "ffn_conv_base", (c.T, c.d), 0.5, c.act))

    def ffn_w_delta(self):
        c = self.cfg
        return self._get("ffn_wdelta", lambda: weight(c.seed, "ffn_w_delta", c.T * c.G, c.d, c.act))

    def w_gate(self):
        c = self.cfg
        return self._get("wgate", lambda: weight(c.seed, "w_gate", c.d_ff, c.d, c.weight))

    def w_up(self):
        c = self.cfg
        return self._get("wup", lambda: weight(c.seed, "w_up", c.d_ff, c.d, c.weight))

    def w_down(self):
        c = self.cfg
        return self._get("wdown", lambda: weight(c.seed, "w_down", c.d, c.d_ff, c.weight))

    def anchor(self, n_seq: int = 1):
        c = self.cfg
        return integers(c.seed, "anchor", 0, c.V, (n_seq,))
