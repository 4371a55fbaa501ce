"""Python binding of libdflash (ctypes; argument marshalling only).

Every function here has the name of the C entry point it calls (see
include/dflash.h for the operation, layouts and error behaviour).  Tensors
are PyTorch device tensors; PyTorch only provides the memory and the stream.
A non-OK status raises DFlashError with the library's message.  There is no
fallback: if libdflash.so is missing, the first call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdflash.so")
_lib = None

F32, BF16, Q8_0 = 0, 1, 2
_DT = {"f32": F32, "bf16": BF16, "q8_0": Q8_0}
_TORCH_ACT = {F32: torch.float32, BF16: torch.bfloat16}

STATUS = {0: "DFLASH_OK", 1: "DFLASH_ERR_INVALID_ARG", 2: "DFLASH_ERR_UNSUPPORTED",
          3: "DFLASH_ERR_CAPACITY", 4: "DFLASH_ERR_WORKSPACE", 5: "DFLASH_ERR_LAUNCH"}


class DFlashError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class _Weight(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("data", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class _Cache(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("capacity", ctypes.c_int64), ("k", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("k_scales", ctypes.c_void_p), ("v_scales", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I32, _I64, _F32, _SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_PW = ctypes.POINTER(_Weight)
_PC = ctypes.POINTER(_Cache)

_SIGS = {
    "dflash_inject": ([ctypes.POINTER(ctypes.c_void_p), _I32, _I64, _I32, _I32, _PW, _P, _F32, _PW, _PW,
                       _PC, _I64, _P, _SZ, _P], _I32),
    "dflash_inject_workspace": ([_I32, _I64, _I32, _I32, _I32, _I32], _SZ),
    "dflash_inject_z_offset": ([_I32, _I64, _I32, _I32, _I32, _I32], _SZ),
    "dflash_conv": ([_P, _I32, _I32, _I32, _I32, _I32, _I32, _P, _PW, _P, _P, _SZ, _P], _I32),
    "dflash_conv_workspace": ([_I32, _I32, _I32, _I32, _I32], _SZ),
    "dflash_ffn_block": ([_P, _I32, _I32, _I32, _I32, _I32, _I32, _P, _PW, _PW, _PW, _PW, _P, _P, _SZ, _P],
                         _I32),
    "dflash_ffn_block_workspace": ([_I32, _I32, _I32, _I32, _I32, _I32], _SZ),
    "dflash_ffn_block_u_offset": ([_I32, _I32, _I32, _I32, _I32, _I32], _SZ),
    "dflash_ffn_block_act_offset": ([_I32, _I32, _I32, _I32, _I32, _I32], _SZ),
    "dflash_block_attn": ([_P, _P, _I32, _I32, _I32, _I32, _PW, _PW, _PW, _PW, _PC, _I64, _F32, _P, _P,
                           _SZ, _P], _I32),
    "dflash_block_attn_after": ([_P, _P, _I32, _I32, _I32, _I32, _PW, _PW, _PW, _PW, _PC, _I64, _F32, _P,
                                 _P, _SZ, _P, _P], _I32),
    "dflash_block_attn_workspace": ([_I32, _I32, _I32, _I32, _I32, _I64], _SZ),
    "dflash_block_attn_qkv_offset": ([_I32, _I32, _I32, _I32, _I32, _I64], _SZ),
    "dflash_block_attn_o_offset": ([_I32, _I32, _I32, _I32, _I32, _I64], _SZ),
    "dflash_topk_unary": ([_P, _I32, _I32, _PW, _I32, _P, _P, _P, _SZ, _P], _I32),
    "dflash_topk_unary_workspace": ([_I32, _I64, _I32], _SZ),
    "dflash_topk_unary_noalloc": ([_P, _I32, _I32, _PW, _I32, _P, _P, _P], _I32),
    "dflash_selector_edges": ([_P, _I32, _I32, _PW, _P, _P, _I64, _P, _P, _I32, _I32, _P, _P, _P, _P, _P,
                               _SZ, _P], _I32),
    "dflash_selector_edges_workspace": ([_I32, _I32, _I32, _I32], _SZ),
    "dflash_topk_select": ([_P, _I32, _I32, _PW, _I32, _PW, _P, _P, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P],
                           _I32),
    "dflash_topk_select_workspace": ([_I32, _I64, _I32, _I32, _I32], _SZ),
    "dflash_accept_len": ([_P, _P, _I32, _I32, _P, _P], _I32),
    "dflash_topk_rows": ([_P, _I64, _I64, _I32, _P, _P, _P, _SZ, _P], _I32),
    "dflash_topk_rows_workspace": ([_I64, _I64, _I32], _SZ),
    "dflash_status_string": ([_I32], ctypes.c_char_p),
    "dflash_last_error": ([], ctypes.c_char_p),
    "dflash_version": ([], _I32),
}


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libdflash.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m block_diffusion_drafter_step_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib


def _check(st: int):
    if st != 0:
        raise DFlashError(st, load().dflash_last_error().decode())


@dataclass
class Weight:
    """A weight [rows][cols] (out x in) on the device: fp32 / bf16 values, or
    Q8_0 int8 codes with fp16 scales [rows][cols/32]."""
    dtype: str
    data: torch.Tensor
    scales: Optional[torch.Tensor] = None

    @property
    def rows(self):
        return self.data.shape[0]

    @property
    def cols(self):
        return self.data.shape[1]

    def c(self) -> _Weight:
        return _Weight(_DT[self.dtype], 0, self.data.shape[0], self.data.shape[1], _ptr(self.data),
                       _ptr(self.scales) if self.scales is not None else None)


@dataclass
class KVCache:
    """K [n_kv_heads][capacity][head_dim] and V in transposed 32-position
    panels, [n_kv_heads][capacity/32][head_dim][32]; capacity is a multiple of
    64.  In the activation type, or Q8_0: int8 codes in those layouts plus
    fp16 scales k_scales / v_scales [n_kv_heads][capacity][head_dim/32].
    `v_panels` / `v_rows` convert V between [n_kv_heads][positions][head_dim]
    and the panel layout."""
    k: torch.Tensor
    v: torch.Tensor
    k_scales: Optional[torch.Tensor] = None
    v_scales: Optional[torch.Tensor] = None

    @property
    def dtype(self) -> str:
        if self.k.dtype == torch.int8:
            return "q8_0"
        return "f32" if self.k.dtype == torch.float32 else "bf16"

    def c(self) -> _Cache:
        h, cap, hd = self.k.shape
        if tuple(self.v.shape) != (h, cap // 32, hd, 32):
            raise ValueError(f"V must be [n_kv_heads][capacity/32][head_dim][32] = "
                             f"{(h, cap // 32, hd, 32)}, got {tuple(self.v.shape)}")
        if self.dtype == "q8_0":
            for s in (self.k_scales, self.v_scales):
                if s is None or s.dtype != torch.float16 or tuple(s.shape) != (h, cap, hd // 32):
                    raise ValueError(f"Q8_0 scales must be fp16 [{h}][{cap}][{hd // 32}]")
        return _Cache(_DT[self.dtype], h, hd, 0, cap, _ptr(self.k), _ptr(self.v), _ptr(self.k_scales),
                      _ptr(self.v_scales))


def v_panels(v_rows: torch.Tensor) -> torch.Tensor:
    """[h][positions][hd] (positions a multiple of 32) -> [h][positions/32][hd][32]."""
    h, n, hd = v_rows.shape
    return v_rows.reshape(h, n // 32, 32, hd).permute(0, 1, 3, 2).contiguous()


def v_rows(v_panel: torch.Tensor) -> torch.Tensor:
    """[h][positions/32][hd][32] -> [h][positions][hd]."""
    h, p, hd, _ = v_panel.shape
    return v_panel.permute(0, 1, 3, 2).reshape(h, p * 32, hd)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libdflash takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libdflash takes contiguous tensors")
    return t.data_ptr()


def _act_of(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise ValueError(f"activations must be float32 or bfloat16, not {t.dtype}")


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ws(ws: Optional[torch.Tensor]):
    if ws is None:
        return None, 0
    return _ptr(ws), ws.numel() * ws.element_size()


# ---- workspace queries ---------------------------------------------------------

def dflash_inject_workspace(n_layers, n_tokens, d_t, d, kv, act="bf16") -> int:
    return load().dflash_inject_workspace(n_layers, n_tokens, d_t, d, kv, _DT[act])


def dflash_inject_z_offset(n_layers, n_tokens, d_t, d, kv, act="bf16") -> int:
    return load().dflash_inject_z_offset(n_layers, n_tokens, d_t, d, kv, _DT[act])


def dflash_block_attn_qkv_offset(B, d, n_q_heads, n_kv_heads, head_dim, n_ctx) -> int:
    return load().dflash_block_attn_qkv_offset(B, d, n_q_heads, n_kv_heads, head_dim, n_ctx)


def dflash_block_attn_o_offset(B, d, n_q_heads, n_kv_heads, head_dim, n_ctx) -> int:
    return load().dflash_block_attn_o_offset(B, d, n_q_heads, n_kv_heads, head_dim, n_ctx)


def ws_view(ws: torch.Tensor, offset: int, shape, dtype) -> torch.Tensor:
    """A view of `shape` elements of `dtype` at byte `offset` of a workspace."""
    n = 1
    for s in shape:
        n *= s
    es = torch.empty((), dtype=dtype).element_size()
    return ws[offset:offset + n * es].view(dtype).view(*shape)


def dflash_conv_workspace(n_blocks, B, C, G, T) -> int:
    return load().dflash_conv_workspace(n_blocks, B, C, G, T)


def dflash_ffn_block_workspace(n_blocks, B, d, G, T, d_ff) -> int:
    return load().dflash_ffn_block_workspace(n_blocks, B, d, G, T, d_ff)


def dflash_ffn_block_u_offset(n_blocks, B, d, G, T, d_ff) -> int:
    return load().dflash_ffn_block_u_offset(n_blocks, B, d, G, T, d_ff)


def dflash_ffn_block_act_offset(n_blocks, B, d, G, T, d_ff) -> int:
    return load().dflash_ffn_block_act_offset(n_blocks, B, d, G, T, d_ff)


def dflash_block_attn_workspace(B, d, n_q_heads, n_kv_heads, head_dim, n_ctx) -> int:
    return load().dflash_block_attn_workspace(B, d, n_q_heads, n_kv_heads, head_dim, n_ctx)


def dflash_topk_unary_workspace(B, V, K) -> int:
    return load().dflash_topk_unary_workspace(B, V, K)


def dflash_selector_edges_workspace(B, r, d, K) -> int:
    return load().dflash_selector_edges_workspace(B, r, d, K)


def dflash_topk_select_workspace(B, V, K, r, d) -> int:
    return load().dflash_topk_select_workspace(B, V, K, r, d)


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A workspace of at least `nbytes` (no initial contents needed)."""
    return torch.empty(max(16, nbytes), dtype=torch.uint8, device=device)


# ---- the six calls -------------------------------------------------------------

def dflash_inject(layer_hidden: Sequence[torch.Tensor], fc: Weight, gamma, eps: float, wk: Weight,
                  wv: Weight, cache: KVCache, pos0: int, ws: torch.Tensor, stream=None):
    act = _act_of(layer_hidden[0])
    n, d_t = layer_hidden[0].shape
    arr = (ctypes.c_void_p * len(layer_hidden))(*[_ptr(t) for t in layer_hidden])
    f, k, v, c = fc.c(), wk.c(), wv.c(), cache.c()
    wsp, wsb = _ws(ws)
    _check(load().dflash_inject(arr, len(layer_hidden), n, d_t, act, ctypes.byref(f), _ptr(gamma), eps,
                                ctypes.byref(k), ctypes.byref(v), ctypes.byref(c), pos0, wsp, wsb,
                                _stream(stream)))


def dflash_conv(x: torch.Tensor, G: int, base: torch.Tensor, w_delta: Weight, out: torch.Tensor,
                ws: torch.Tensor, stream=None):
    nb, B, C = x.shape
    T = base.shape[0]
    w = w_delta.c()
    wsp, wsb = _ws(ws)
    _check(load().dflash_conv(_ptr(x), nb, B, C, G, T, _act_of(x), _ptr(base), ctypes.byref(w), _ptr(out),
                              wsp, wsb, _stream(stream)))


def dflash_ffn_block(h: torch.Tensor, G: int, base: torch.Tensor, w_delta: Weight, w_gate: Weight,
                     w_up: Weight, w_down: Weight, out: torch.Tensor, ws: torch.Tensor, stream=None):
    """The feed-forward site: h [n_blocks][B][d] -> out (same shape)."""
    nb, B, d = h.shape
    T = base.shape[0]
    wd, wg, wu, wn = w_delta.c(), w_gate.c(), w_up.c(), w_down.c()
    wsp, wsb = _ws(ws)
    _check(load().dflash_ffn_block(_ptr(h), nb, B, d, G, T, _act_of(h), _ptr(base), ctypes.byref(wd),
                                   ctypes.byref(wg), ctypes.byref(wu), ctypes.byref(wn), _ptr(out), wsp, wsb,
                                   _stream(stream)))


def dflash_block_attn(u: torch.Tensor, residual, n_q_heads: int, wq: Weight, wk: Weight, wv: Weight,
                      wo: Weight, cache: KVCache, n_ctx: int, scale: float, out: torch.Tensor,
                      ws: torch.Tensor, stream=None):
    B, d = u.shape
    q, k, v, o, c = wq.c(), wk.c(), wv.c(), wo.c(), cache.c()
    wsp, wsb = _ws(ws)
    _check(load().dflash_block_attn(_ptr(u), _ptr(residual), B, d, n_q_heads, _act_of(u), ctypes.byref(q),
                                    ctypes.byref(k), ctypes.byref(v), ctypes.byref(o), ctypes.byref(c),
                                    n_ctx, scale, _ptr(out), wsp, wsb, _stream(stream)))


def dflash_block_attn_after(u: torch.Tensor, residual, n_q_heads: int, wq: Weight, wk: Weight, wv: Weight,
                            wo: Weight, cache: KVCache, n_ctx: int, scale: float, out: torch.Tensor,
                            ws: torch.Tensor, cache_ready: torch.cuda.Event, stream=None):
    """dflash_block_attn whose stream waits for `cache_ready` (a recorded
    torch.cuda.Event) before the kernels that read the cache."""
    B, d = u.shape
    q, k, v, o, c = wq.c(), wk.c(), wv.c(), wo.c(), cache.c()
    wsp, wsb = _ws(ws)
    _check(load().dflash_block_attn_after(_ptr(u), _ptr(residual), B, d, n_q_heads, _act_of(u),
                                          ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), ctypes.byref(o),
                                          ctypes.byref(c), n_ctx, scale, _ptr(out), wsp, wsb, _stream(stream),
                                          cache_ready.cuda_event))


def dflash_topk_unary(h: torch.Tensor, lm_head: Weight, K: int, idx: torch.Tensor, unary: torch.Tensor,
                      ws: torch.Tensor, stream=None):
    B = h.shape[0]
    w = lm_head.c()
    wsp, wsb = _ws(ws)
    _check(load().dflash_topk_unary(_ptr(h), B, _act_of(h), ctypes.byref(w), K, _ptr(idx), _ptr(unary),
                                    wsp, wsb, _stream(stream)))


def dflash_topk_unary_noalloc(h: torch.Tensor, lm_head: Weight, K: int, idx: torch.Tensor,
                              unary: torch.Tensor, stream=None):
    """dflash_topk_unary with the library's static scratch (no workspace)."""
    B = h.shape[0]
    w = lm_head.c()
    _check(load().dflash_topk_unary_noalloc(_ptr(h), B, _act_of(h), ctypes.byref(w), K, _ptr(idx),
                                            _ptr(unary), _stream(stream)))


def dflash_selector_edges(h: torch.Tensor, proj: Weight, cb_pred: torch.Tensor, cb_succ: torch.Tensor,
                          idx: torch.Tensor, unary: torch.Tensor, anchor: int, edges: torch.Tensor,
                          path: torch.Tensor, ws: torch.Tensor, stream=None, target=None, accept=None):
    """target int32 [B] / accept int32 [1] (both or neither): also the accept length."""
    B = h.shape[0]
    K = idx.shape[1]
    w = proj.c()
    wsp, wsb = _ws(ws)
    _check(load().dflash_selector_edges(_ptr(h), B, _act_of(h), ctypes.byref(w), _ptr(cb_pred),
                                        _ptr(cb_succ), cb_pred.shape[0], _ptr(idx), _ptr(unary), K, anchor,
                                        _ptr(edges), _ptr(path), _ptr(target), _ptr(accept), wsp, wsb,
                                        _stream(stream)))


def dflash_topk_select(h: torch.Tensor, lm_head: Weight, K: int, proj: Weight, cb_pred: torch.Tensor,
                       cb_succ: torch.Tensor, anchor: int, idx: torch.Tensor, unary: torch.Tensor,
                       edges: torch.Tensor, path: torch.Tensor, ws: torch.Tensor, stream=None, target=None,
                       accept=None):
    """dflash_topk_unary then dflash_selector_edges (V = lm_head rows) in one call."""
    B = h.shape[0]
    wl, wp = lm_head.c(), proj.c()
    wsp, wsb = _ws(ws)
    _check(load().dflash_topk_select(_ptr(h), B, _act_of(h), ctypes.byref(wl), K, ctypes.byref(wp), _ptr(cb_pred),
                                     _ptr(cb_succ), anchor, _ptr(idx), _ptr(unary), _ptr(edges), _ptr(path),
                                     _ptr(target), _ptr(accept), wsp, wsb, _stream(stream)))


def dflash_accept_len(draft: torch.Tensor, target: torch.Tensor, accept: torch.Tensor, stream=None):
    n_seq, B = draft.shape
    _check(load().dflash_accept_len(_ptr(draft), _ptr(target), n_seq, B, _ptr(accept), _stream(stream)))


def dflash_topk_rows_workspace(n_rows, n_cols, K) -> int:
    return load().dflash_topk_rows_workspace(n_rows, n_cols, K)


def dflash_topk_rows(x: torch.Tensor, K: int, idx: torch.Tensor, val: torch.Tensor, ws: torch.Tensor,
                     stream=None):
    """Row-wise top-K of an fp32 matrix: idx int32 [rows][K], val fp32 [rows][K]."""
    if x.dtype != torch.float32:
        raise ValueError("dflash_topk_rows takes fp32 scores")
    n_rows, n_cols = x.shape
    wsp, wsb = _ws(ws)
    _check(load().dflash_topk_rows(_ptr(x), n_rows, n_cols, K, _ptr(idx), _ptr(val), wsp, wsb,
                                   _stream(stream)))
