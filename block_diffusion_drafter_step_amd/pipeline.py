"""Device staging and orchestration of the draft block step (host logic only).

`to_device` moves the seeded inputs of synth.Workload onto the GPU in the
storage formats libdflash reads; `BlockStep` owns the outputs and
workspaces of one block step and enqueues the library calls: in order on
one stream, or (run(overlap=True)) with the injection on a second stream
beside the conv and the attention's projection.  No arithmetic of the method happens here.
"""
from __future__ import annotations

import numpy as np
import torch

from . import dflash as D
from . import synth


def act_tensor(a: np.ndarray, act: str, device="cuda") -> torch.Tensor:
    if act == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def weight_tensor(w: dict, device="cuda") -> D.Weight:
    if w["dtype"] == "q8_0":
        return D.Weight("q8_0", torch.from_numpy(w["data"]).to(device),
                        torch.from_numpy(w["scales"]).to(device))
    return D.Weight(w["dtype"], act_tensor(w["data"], w["dtype"], device))


def act_dtype(act: str):
    return torch.bfloat16 if act == "bf16" else torch.float32


def new_cache(cfg, device="cuda", kv: str = None) -> D.KVCache:
    """Zeroed cache: K [Hkv][cap][hd], V in transposed panels [Hkv][cap/32][hd][32],
    in the activation type, or Q8_0 codes with fp16 scales [Hkv][cap][hd/32]
    (kv="q8_0")."""
    if kv == "q8_0":
        return D.KVCache(torch.zeros((cfg.Hkv, cfg.cap, cfg.hd), dtype=torch.int8, device=device),
                         torch.zeros((cfg.Hkv, cfg.cap // 32, cfg.hd, 32), dtype=torch.int8, device=device),
                         torch.zeros((cfg.Hkv, cfg.cap, cfg.hd // 32), dtype=torch.float16, device=device),
                         torch.zeros((cfg.Hkv, cfg.cap, cfg.hd // 32), dtype=torch.float16, device=device))
    dt = act_dtype(cfg.act)
    return D.KVCache(torch.zeros((cfg.Hkv, cfg.cap, cfg.hd), dtype=dt, device=device),
                     torch.zeros((cfg.Hkv, cfg.cap // 32, cfg.hd, 32), dtype=dt, device=device))


class DeviceWeights:
    """All weights of one draft layer plus the shared head and selector."""

    def __init__(self, w: synth.Workload, device="cuda", drop_host: bool = True):
        cfg = w.cfg
        self.cfg = cfg
        self.fc = weight_tensor(w.fc(), device)
        self.wq = weight_tensor(w.wq(), device)
        self.wk = weight_tensor(w.wk(), device)
        self.wv = weight_tensor(w.wv(), device)
        self.wo = weight_tensor(w.wo(), device)
        self.base = act_tensor(w.conv_base(), cfg.act, device)
        self.w_delta = weight_tensor(w.w_delta(), device)
        self.w_lm = weight_tensor(w.w_lm(), device)
        if drop_host:
            w.drop("wlm")
        self.sel_P = weight_tensor(w.sel_proj(), device)
        A, Bc = w.codebooks()
        self.cb_pred = act_tensor(A, cfg.act, device)
        self.cb_succ = act_tensor(Bc, cfg.act, device)


class BlockStep:
    """Buffers of one block step: conv -> block attention (+ residual) ->
    LM-head top-K -> selector edges + path -> accept length (the last three
    in one call, run(); or one at a time); optionally an injection of
    `inject_n` rows first."""

    def __init__(self, cfg, weights: DeviceWeights, cache: D.KVCache, inject_n: int = 0, device="cuda"):
        self.cfg, self.W, self.cache = cfg, weights, cache
        dt = act_dtype(cfg.act)
        B, d = cfg.B, cfg.d
        self.u = torch.empty((1, B, cfg.C), dtype=dt, device=device)
        self.h = torch.empty((B, d), dtype=dt, device=device)
        self.idx = torch.empty((B, cfg.K), dtype=torch.int32, device=device)
        self.unary = torch.empty((B, cfg.K), dtype=torch.float32, device=device)
        self.edges = torch.empty((B, cfg.K, cfg.K), dtype=torch.float32, device=device)
        self.path = torch.empty((1, B), dtype=torch.int32, device=device)
        self.accept = torch.empty((1,), dtype=torch.int32, device=device)
        self.inject_n = inject_n
        n_ctx_max = cache.k.shape[1]
        sizes = [D.dflash_conv_workspace(1, B, cfg.C, cfg.G, cfg.T),
                 D.dflash_block_attn_workspace(B, d, cfg.Hq, cfg.Hkv, cfg.hd, n_ctx_max),
                 D.dflash_topk_unary_workspace(B, cfg.V, cfg.K),
                 D.dflash_selector_edges_workspace(B, cfg.r, d, cfg.K),
                 D.dflash_topk_select_workspace(B, cfg.V, cfg.K, cfg.r, d)]
        # one workspace reused by the calls of the main stream (stream-ordered);
        # the injection has its own, as run(overlap=True) overlaps it with the
        # conv and the attention's projection
        self.ws = D.workspace(max(sizes), device)
        if inject_n:
            self.ws_inj = D.workspace(D.dflash_inject_workspace(cfg.L_t, inject_n, cfg.d_t, d, cfg.kv, cfg.act),
                                      device)
            self.side = torch.cuda.Stream(device=device)   # default priority
            self.injected = torch.cuda.Event()

    def inject(self, hidden, pos0: int, stream=None):
        W = self.W
        D.dflash_inject(hidden, W.fc, None, self.cfg.eps, W.wk, W.wv, self.cache, pos0, self.ws_inj, stream)

    def conv(self, x, stream=None):
        D.dflash_conv(x, self.cfg.G, self.W.base, self.W.w_delta, self.u, self.ws, stream)

    def attn(self, x, n_ctx: int, stream=None, after=None):
        """Block attention; `after` (a recorded event): the kernels that read
        the cache wait for it (dflash_block_attn_after)."""
        W = self.W
        if after is None:
            D.dflash_block_attn(self.u[0], x[0], self.cfg.Hq, W.wq, W.wk, W.wv, W.wo, self.cache, n_ctx, 0.0,
                                self.h, self.ws, stream)
        else:
            D.dflash_block_attn_after(self.u[0], x[0], self.cfg.Hq, W.wq, W.wk, W.wv, W.wo, self.cache, n_ctx,
                                      0.0, self.h, self.ws, after, stream)

    def topk(self, stream=None):
        D.dflash_topk_unary(self.h, self.W.w_lm, self.cfg.K, self.idx, self.unary, self.ws, stream)

    def select(self, anchor: int, target=None, stream=None):
        """Edges and path; with `target` ([1][B] int32) also the accept length,
        in the selector's own kernel."""
        W = self.W
        D.dflash_selector_edges(self.h, W.sel_P, W.cb_pred, W.cb_succ, self.idx, self.unary, anchor,
                                self.edges, self.path[0], self.ws, stream,
                                target=None if target is None else target[0], accept=
                                None if target is None else self.accept)

    def topk_select(self, anchor: int, target=None, stream=None):
        """topk() then select() as one call (dflash_topk_select)."""
        W = self.W
        D.dflash_topk_select(self.h, W.w_lm, self.cfg.K, W.sel_P, W.cb_pred, W.cb_succ, anchor, self.idx,
                             self.unary, self.edges, self.path[0], self.ws, stream,
                             target=None if target is None else target[0],
                             accept=None if target is None else self.accept)

    def accept_len(self, target, stream=None):
        D.dflash_accept_len(self.path, target, self.accept, stream)

    def run(self, x, n_ctx: int, anchor: int, target, hidden=None, pos0: int = 0, stream=None,
            overlap: bool = False):
        """One block step.  With an injection and `overlap`, the injection runs
        on the side stream once everything enqueued before on `stream` is
        done, and the attention's cache-reading kernels wait for it; the conv
        and the attention's Q | Kb | Vb projection run meanwhile.  The inputs
        must stay alive until the step has completed on `stream`.  (On one
        MI355X the overlap measured slower on the bf16 32k workload, 2172 ->
        2139 steps/s, and 0.4 % faster on the Q8_0 one: the fc and the
        projection share HBM, and the two cross-stream waits per step cost
        about what the latency-bound kernels hide.)"""
        main = stream if stream is not None else torch.cuda.current_stream()
        if self.inject_n and overlap:
            self.side.wait_stream(main)
            self.inject(hidden, pos0, self.side)
            self.injected.record(self.side)
            self.conv(x, main)
            self.attn(x, n_ctx, main, after=self.injected)
        else:
            if self.inject_n:
                self.inject(hidden, pos0, main)
            self.conv(x, main)
            self.attn(x, n_ctx, main)
        self.topk_select(anchor, target, main)
