"""The C ABI on the host: the library loads, exports every symbol the header
declares, and rejects bad arguments before it touches a GPU.

Every call here fails validation (no launch ever happens), and the
fake-pointer cases are skipped where a GPU is visible so that no kernel can
ever see a made-up address.
"""
import ctypes
import os
import re
import subprocess

import pytest
import torch

from block_diffusion_drafter_step_amd import dflash as D

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash.h")

no_gpu = pytest.mark.skipif(torch.cuda.is_available(), reason="fake device pointers only without a GPU")


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(D.lib_path()):
        from block_diffusion_drafter_step_amd import build
        build.build(verbose=False)
    return D.load()


def test_exports_every_declared_symbol(lib):
    names = declared()
    assert len(names) >= 14
    out = subprocess.run(["nm", "-D", "--defined-only", D.lib_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (dflash_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        getattr(lib, n)


def test_status_strings_and_version(lib):
    assert lib.dflash_status_string(0) == b"ok"
    assert b"workspace" in lib.dflash_status_string(4)
    assert lib.dflash_status_string(99) == b"unknown status"
    assert lib.dflash_version() >= 100


def test_workspace_queries_are_host_only(lib):
    a = lib.dflash_inject_workspace(5, 16, 5120, 5120, 1024, 1)
    b = lib.dflash_inject_workspace(5, 32768, 5120, 5120, 1024, 1)
    assert 0 < a < b
    assert lib.dflash_block_attn_workspace(16, 5120, 32, 8, 128, 32768) > \
        lib.dflash_block_attn_workspace(16, 5120, 32, 8, 128, 1024)
    assert lib.dflash_topk_unary_workspace(16, 151936, 8) > 0
    # a workspace sized for a longer context fits every shorter one
    sizes = [lib.dflash_block_attn_workspace(16, 5120, 32, 8, 128, n) for n in range(0, 40000, 61)]
    assert all(a <= b for a, b in zip(sizes, sizes[1:]))
    assert lib.dflash_conv_workspace(1, 16, 5120, 64, 4) > 0
    assert lib.dflash_selector_edges_workspace(16, 64, 5120, 8) > 0
    assert lib.dflash_inject_workspace(0, 16, 5120, 5120, 1024, 1) == 0


def test_intermediate_offsets_lie_inside_the_workspace(lib):
    """z, Q | Kb | Vb and O sit after the counters, 256-byte aligned, and
    inside the workspace the matching query returns."""
    for n in (1, 16, 64, 1000, 32768):
        ws = lib.dflash_inject_workspace(5, n, 5120, 5120, 1024, 1)
        z = lib.dflash_inject_z_offset(5, n, 5120, 5120, 1024, 1)
        assert z >= 65536 and z % 256 == 0 and z + n * 5120 * 2 <= ws
    for n_ctx in (0, 1, 1024, 32768, 65552):
        ws = lib.dflash_block_attn_workspace(16, 5120, 32, 8, 128, n_ctx)
        q = lib.dflash_block_attn_qkv_offset(16, 5120, 32, 8, 128, n_ctx)
        o = lib.dflash_block_attn_o_offset(16, 5120, 32, 8, 128, n_ctx)
        assert 65536 <= q < o and q % 256 == 0 and o % 256 == 0
        assert q + 16 * 6144 * 2 <= o and o + 16 * 4096 * 2 <= ws
    assert lib.dflash_inject_z_offset(0, 16, 5120, 5120, 1024, 1) == 0
    for nb in (1, 3, 2048):
        ws = lib.dflash_ffn_block_workspace(nb, 16, 5120, 64, 4, 17408)
        u = lib.dflash_ffn_block_u_offset(nb, 16, 5120, 64, 4, 17408)
        a = lib.dflash_ffn_block_act_offset(nb, 16, 5120, 64, 4, 17408)
        M = nb * 16
        assert 65536 <= u < a and u % 256 == 0 and a % 256 == 0
        assert u + M * 5120 * 2 <= a and a + M * 17408 * 2 <= ws
    assert lib.dflash_ffn_block_workspace(0, 16, 5120, 64, 4, 17408) == 0
    assert lib.dflash_ffn_block_act_offset(1, 16, 5120, 64, 4, 0) == 0


FAKE = 0x10000        # aligned, never dereferenced: every case below is invalid


def W(dtype, rows, cols, data=FAKE, scales=None):
    return D._Weight(dtype, 0, rows, cols, data, scales)


def cache(dtype=1, h=8, hd=128, cap=4096, k=FAKE, v=FAKE):
    return D._Cache(dtype, h, hd, 0, cap, k, v)


def err(lib):
    return lib.dflash_last_error().decode()


@no_gpu
def test_inject_rejections(lib):
    arr = (ctypes.c_void_p * 2)(FAKE, FAKE)
    fc, wk, wv, c = W(1, 256, 512), W(1, 1024, 256), W(1, 1024, 256), cache()
    ref = ctypes.byref

    def call(arr=arr, n_layers=2, n=16, d_t=256, act=1, fc=fc, wk=wk, wv=wv, c=c, pos0=0, ws=FAKE, wsb=1 << 30):
        return lib.dflash_inject(arr, n_layers, n, d_t, act, ref(fc), None, 1e-6, ref(wk), ref(wv), ref(c),
                                 pos0, ws, wsb, None)

    assert call(act=7) == 1
    assert call(n_layers=0) == 1
    assert call(n_layers=17) == 1
    assert call(n=0) == 1
    assert call(d_t=100) == 1
    assert call(fc=W(1, 256, 500)) == 1 and "fc" in err(lib)
    assert call(fc=W(0, 256, 512)) == 1                       # fp32 weight with bf16 activations
    assert call(fc=W(2, 256, 512, scales=None)) == 1          # Q8_0 without scales
    assert call(fc=W(1, 256, 512, data=FAKE + 8)) == 1        # misaligned
    assert call(wk=W(1, 512, 256)) == 1                       # kv mismatch with the cache
    assert call(wk=W(2, 1024, 256, scales=FAKE)) == 2         # wk / wv dtypes differ
    assert call(c=cache(hd=96)) == 2
    assert call(c=cache(dtype=0)) == 1
    assert call(pos0=4090) == 3 and "capacity" in err(lib)
    assert call(c=cache(cap=4000)) == 1 and "capacity" in err(lib)   # not a multiple of 64
    assert call(pos0=-1) == 3
    assert call(ws=None) == 4
    assert call(wsb=16) == 4
    bad = (ctypes.c_void_p * 2)(FAKE, None)
    assert call(arr=bad) == 1


@no_gpu
def test_conv_rejections(lib):
    ref = ctypes.byref
    wd = W(1, 4 * 8, 256)

    def call(nb=1, B=8, C=256, G=8, T=4, act=1, w=wd, ws=FAKE, wsb=1 << 30):
        return lib.dflash_conv(FAKE, nb, B, C, G, T, act, FAKE, ref(w), FAKE, ws, wsb, None)

    assert call(C=200) == 1
    assert call(G=7) == 1
    assert call(T=0) == 1
    assert call(T=17) == 1
    assert call(B=0) == 1
    assert call(B=17) == 1
    assert call(w=W(1, 33, 256)) == 1
    assert call(w=W(2, 32, 256, scales=FAKE)) == 2            # W_delta cannot be Q8_0
    assert call(wsb=8) == 4


@no_gpu
def test_ffn_block_rejections(lib):
    ref = ctypes.byref
    wd, wg, wu, wn = W(1, 4 * 8, 256), W(1, 512, 256), W(1, 512, 256), W(1, 256, 512)

    def call(h=FAKE, nb=1, B=8, d=256, G=8, T=4, act=1, wd=wd, wg=wg, wu=wu, wn=wn, out=FAKE + 4096,
             ws=FAKE, wsb=1 << 30):
        return lib.dflash_ffn_block(h, nb, B, d, G, T, act, FAKE, ref(wd), ref(wg), ref(wu), ref(wn), out,
                                    ws, wsb, None)

    assert call(act=5) == 1
    assert call(h=None) == 1
    assert call(out=FAKE) == 1 and "overlap" in err(lib)       # out == h
    assert call(nb=0) == 1
    assert call(B=17) == 1
    assert call(d=200) == 1
    assert call(G=7) == 1
    assert call(T=17) == 1
    assert call(wd=W(1, 33, 256)) == 1
    assert call(wd=W(2, 32, 256, scales=FAKE)) == 2            # W_delta cannot be Q8_0
    assert call(wg=W(1, 500, 256), wu=W(1, 500, 256), wn=W(1, 256, 500)) == 1 and "d_ff" in err(lib)
    assert call(wu=W(1, 512, 128)) == 1                        # up's input width is not d
    assert call(wn=W(1, 256, 448)) == 1                        # down's input width is not d_ff
    assert call(wg=W(0, 512, 256)) == 1                        # fp32 weight with bf16 activations
    assert call(wg=W(2, 512, 256, scales=FAKE)) == 2           # gate and up dtypes differ
    assert call(wn=W(2, 256, 512, scales=None)) == 1           # Q8_0 without scales
    assert call(act=0) == 1                                    # bf16 weights with fp32 activations
    assert call(ws=None) == 4
    assert call(wsb=64) == 4


@no_gpu
def test_attn_rejections(lib):
    ref = ctypes.byref
    wq, wk, wv, wo = W(1, 4096, 5120), W(1, 1024, 5120), W(1, 1024, 5120), W(1, 5120, 4096)

    def call(B=16, d=5120, Hq=32, c=cache(), n_ctx=1024, wq=wq, wk=wk, wo=wo, scale=0.0, wsb=1 << 30):
        return lib.dflash_block_attn(FAKE, None, B, d, Hq, 1, ref(wq), ref(wk), ref(wv), ref(wo), ref(c), n_ctx,
                                     scale, FAKE, FAKE, wsb, None)

    assert call(B=0) == 1
    assert call(B=17) == 1
    assert call(B=17) == 1
    assert call(Hq=30) == 1
    assert call(Hq=80, wq=W(1, 80 * 128, 5120), wo=W(1, 5120, 80 * 128)) == 2   # 10 q heads per kv head
    assert call(n_ctx=5000) == 3
    assert call(n_ctx=-1) == 3
    assert call(wo=W(1, 5120, 4000)) == 1
    assert call(wk=W(2, 1024, 5120, scales=FAKE)) == 2
    assert call(scale=-1.0) == 1
    assert call(wsb=1024) == 4
    # the variant that waits for the cache's event: the same checks, and the
    # event itself is required
    after = lambda ev, B=16: lib.dflash_block_attn_after(FAKE, None, B, 5120, 32, 1, ref(wq), ref(wk), ref(wv),
                                                         ref(wo), ref(cache()), 1024, 0.0, FAKE, FAKE, 1 << 30,
                                                         None, ev)
    assert after(None) == 1
    assert after(FAKE, B=17) == 1


@no_gpu
def test_topk_and_selector_rejections(lib):
    ref = ctypes.byref
    lm = W(1, 1000, 256)
    assert lib.dflash_topk_unary(FAKE, 16, 1, ref(lm), 0, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    assert lib.dflash_topk_unary(FAKE, 16, 1, ref(lm), 33, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    assert lib.dflash_topk_unary(FAKE, 16, 1, ref(W(1, 20, 256)), 21, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    assert lib.dflash_topk_unary(FAKE, 17, 1, ref(lm), 8, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    assert lib.dflash_topk_unary(FAKE, 16, 1, ref(lm), 8, FAKE, FAKE, FAKE, 4, None) == 4
    assert lib.dflash_topk_unary(FAKE, 16, 1, ref(W(2, 1000, 250, scales=FAKE)), 8, FAKE, FAKE, FAKE, 1 << 30,
                                 None) == 1
    P = W(1, 64, 256)

    def sel(r=64, V=1000, K=8, anchor=3, B=16, P=P, wsb=1 << 30, target=None, accept=None):
        return lib.dflash_selector_edges(FAKE, B, 1, ref(P), FAKE, FAKE, V, FAKE, FAKE, K, anchor, FAKE, FAKE,
                                         target, accept, FAKE, wsb, None)

    assert sel(P=W(1, 63, 256)) == 1
    assert sel(P=W(1, 512, 256)) == 1
    assert sel(anchor=1000) == 1
    assert sel(anchor=-2) == 1
    assert sel(K=33) == 1
    assert sel(V=4) == 1
    assert sel(wsb=0) == 4
    assert sel(target=FAKE) == 1          # target without accept
    assert sel(accept=FAKE) == 1          # accept without target
    assert lib.dflash_accept_len(FAKE, FAKE, 0, 8, FAKE, None) == 1
    assert lib.dflash_accept_len(None, FAKE, 1, 8, FAKE, None) == 1

    # the combined call checks both calls' arguments (V = the LM head's rows)
    def tks(lm=lm, K=8, P=P, anchor=3, B=16, wsb=1 << 30, target=None, accept=None):
        return lib.dflash_topk_select(FAKE, B, 1, ref(lm), K, ref(P), FAKE, FAKE, anchor, FAKE, FAKE, FAKE, FAKE,
                                      target, accept, FAKE, wsb, None)

    assert tks(K=0) == 1
    assert tks(K=33) == 1
    assert tks(B=17) == 1
    assert tks(P=W(1, 63, 256)) == 1
    assert tks(P=W(1, 64, 320)) == 1       # proj and lm_head disagree on d
    assert tks(anchor=1000) == 1           # anchor past the LM head's rows
    assert tks(target=FAKE) == 1
    assert tks(wsb=4) == 4
    need = lib.dflash_topk_select_workspace(16, 1000, 8, 64, 256)
    assert need >= lib.dflash_topk_unary_workspace(16, 1000, 8) + lib.dflash_selector_edges_workspace(16, 64, 256, 8) - 65536
    assert tks(wsb=need - 1) == 4
    assert lib.dflash_topk_select_workspace(16, 1000, 8, 63, 256) == 0
    assert lib.dflash_topk_select_workspace(17, 1000, 8, 64, 256) == 0


@no_gpu
def test_topk_rows_rejections_and_workspace(lib):
    wide = lib.dflash_topk_rows_workspace(2, 200000, 1024)
    assert wide > lib.dflash_topk_rows_workspace(2, 2000, 8) > 0
    assert lib.dflash_topk_rows_workspace(2, 100, 101) == 0
    assert lib.dflash_topk_rows_workspace(2, 5000, 1025) == 0

    def call(rows=4, cols=1000, K=8, wsb=1 << 30, x=FAKE):
        return lib.dflash_topk_rows(x, rows, cols, K, FAKE, FAKE, FAKE, wsb, None)

    assert call(K=0) == 1
    assert call(K=1025, cols=5000) == 1
    assert call(K=1001) == 1
    assert call(rows=0) == 1
    assert call(rows=70000) == 1
    assert call(cols=1 << 31, K=8) == 1
    assert call(x=None) == 1
    assert call(wsb=0) == 4


def test_binding_refuses_host_tensors():
    x = torch.zeros(4, 4)
    with pytest.raises(ValueError):
        D._ptr(x)


@no_gpu
def test_noalloc_topk_validates_before_any_device_call(lib):
    """Bad arguments and a vocabulary beyond the static scratch are rejected
    on the host (no device is touched: there is none here)."""
    h, idx, un = FAKE, FAKE, FAKE
    w = W(1, (1 << 20) + 16, 64)
    assert lib.dflash_topk_unary_noalloc(h, 16, 1, ctypes.byref(w), 32, idx, un, None) == 2
    assert b"static array" in lib.dflash_last_error()
    w = W(1, 1000, 64)
    assert lib.dflash_topk_unary_noalloc(h, 16, 1, ctypes.byref(w), 33, idx, un, None) == 1
    assert lib.dflash_topk_unary_noalloc(h, 17, 1, ctypes.byref(w), 8, idx, un, None) == 1
    assert lib.dflash_topk_unary_noalloc(None, 16, 1, ctypes.byref(w), 8, idx, un, None) == 1


@no_gpu
def test_q8_0_cache_validation(lib):
    """A Q8_0 cache needs bf16 activations, head_dim 128 and both scale
    arrays; the attention also needs group x block <= 64 query rows."""
    hid = (ctypes.c_void_p * 1)(FAKE)
    fc, wk = W(1, 512, 512), W(1, 1024, 512)
    ok = D._Cache(2, 8, 128, 0, 4096, FAKE, FAKE, FAKE, FAKE)
    ws_big = 1 << 40
    st = lib.dflash_inject(hid, 1, 16, 512, 0, ctypes.byref(W(0, 512, 512)), None, 1e-6, ctypes.byref(W(0, 1024, 512)),
                           ctypes.byref(W(0, 1024, 512)), ctypes.byref(ok), 0, FAKE, ws_big, None)
    assert st == 1 and b"bf16" in lib.dflash_last_error()
    hd64 = D._Cache(2, 8, 64, 0, 4096, FAKE, FAKE, FAKE, FAKE)
    wk64 = W(1, 512, 512)
    assert lib.dflash_inject(hid, 1, 16, 512, 1, ctypes.byref(fc), None, 1e-6, ctypes.byref(wk64), ctypes.byref(wk64),
                             ctypes.byref(hd64), 0, FAKE, ws_big, None) == 2
    noscale = D._Cache(2, 8, 128, 0, 4096, FAKE, FAKE, None, FAKE)
    assert lib.dflash_inject(hid, 1, 16, 512, 1, ctypes.byref(fc), None, 1e-6, ctypes.byref(wk), ctypes.byref(wk),
                             ctypes.byref(noscale), 0, FAKE, ws_big, None) == 1
    assert b"k_scales" in lib.dflash_last_error()
    # attention over a Q8_0 cache of head_dim 64: not implemented
    wq, wkv, wo = W(1, 64 * 64, 512), W(1, 512, 512), W(1, 512, 64 * 64)
    st = lib.dflash_block_attn(FAKE, None, 16, 512, 64, 1, ctypes.byref(wq), ctypes.byref(wkv), ctypes.byref(wkv),
                               ctypes.byref(wo), ctypes.byref(hd64), 100, 0.0, FAKE, FAKE, ws_big, None)
    assert st == 2

