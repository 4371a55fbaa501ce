"""GPU parity: every libdflash call against the CPU oracle on the same seeded
inputs, element by element, at small sizes that still span several tiles and
a ragged tail, and at the workloads' full sizes on sampled outputs.

Floats: per element |gpu - ref| <= atol + rtol |ref|, (2e-2, 1e-2) for bf16
workloads and (1e-4, 1e-4) for fp32.  Checks are stage-wise where a call has
internal bf16 rounding points: each oracle stage is fed the GPU's own output
of the stage before it, once that output has itself passed (the injection's
encoder output z; the attention's Q | Kb | Vb and O, read from the call's
workspace).  Two allowances are named where they apply: the softmax weights
the attention rounds to bf16 before its P.V product (a per-element bound the
oracle computes), and, for end-to-end comparisons of the Q8_0 workload, the
propagation of the stage-checked differences at the upstream rounding point.
Integer results (top-K indices, the path, accept lengths) are exact wherever
the oracle's score gap makes them unique (> 1e-3) and valid elsewhere.
"""
import numpy as np
import pytest
import torch

import oracle as O
from block_diffusion_drafter_step_amd import configs, synth
from block_diffusion_drafter_step_amd import dflash as D
from block_diffusion_drafter_step_amd import pipeline as P
from tests.gpu_util import GAP, act_np, assert_close, check_topk, dev, f64, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    D.load()            # raises if libdflash.so was not built: no fallback
    yield
    torch.cuda.synchronize()


def cfg_small(i, **kw):
    return configs.shrink(configs.get(i), **kw)


def wdev(w):
    return P.weight_tensor(w)


def wnp(w):
    return O.weight_to_f64(w)


def garbage(ws: torch.Tensor, seed: int):
    """Fill a workspace with seeded random bytes (stale counters included)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    ws.copy_(torch.randint(0, 256, ws.shape, generator=g, device="cuda", dtype=torch.int32).to(torch.uint8))


def rows_of_cache(cache, pos):
    """K and V rows [len(pos)][Hkv*hd] of the cache at positions `pos`."""
    p = torch.as_tensor(np.asarray(pos), device="cuda")
    n = len(pos)
    gk = f64(cache.k[:, p, :].permute(1, 0, 2).reshape(n, -1))
    gv = f64(D.v_rows(cache.v)[:, p, :].permute(1, 0, 2).reshape(n, -1))   # V^T panels
    return gk, gv


# ---------------------------------------------------------------------------
# (1) injection
# ---------------------------------------------------------------------------

def check_inject(cfg, hid_rows, fc, gamma, wk, wv, zg, gk, gv, what):
    """Stage-wise and end-to-end checks of injected rows: the GPU's z against
    the oracle's encoder; its K / V against the oracle's projections of that
    same z; then K / V against the oracle chain (Q8_0 weights: plus the
    propagation |W| |z_gpu - z_ref| of the stage-checked z differences)."""
    bp = cfg.act == "bf16"
    Wk, Wv = wnp(wk), wnp(wv)
    enc = O.encode(hid_rows, wnp(fc), gamma, cfg.eps, bp)
    assert_close(zg, enc["z"], cfg.act, f"{what} z")
    st = O.kv_project(zg, Wk, Wv, bp)
    assert_close(gk, st["k"], cfg.act, f"{what} K from the GPU's z")
    assert_close(gv, st["v"], cfg.act, f"{what} V from the GPU's z")
    ref = O.kv_project(enc["z"], Wk, Wv, bp)
    if cfg.weight == "q8_0":
        dz = np.abs(zg - enc["z"])
        assert_close(gk, ref["k"], cfg.act, f"{what} K end to end", term=dz @ np.abs(Wk).T)
        assert_close(gv, ref["v"], cfg.act, f"{what} V end to end", term=dz @ np.abs(Wv).T)
    else:
        assert_close(gk, ref["k"], cfg.act, f"{what} K end to end")
        assert_close(gv, ref["v"], cfg.act, f"{what} V end to end")


def run_inject(cfg, n, pos0, rows=None, prefill=None, gamma=None, garbage_seed=None, tag=None,
               cache=None, hid=None):
    """GPU injection of n seeded rows at pos0; oracle checks on `rows`.
    Returns (cache, K rows, V rows) of the checked rows."""
    say(f"inject {cfg.name} n={n} pos0={pos0} weight={cfg.weight} gamma={gamma is not None} "
        f"garbage_ws={garbage_seed is not None}")
    w = synth.Workload(cfg)
    if hid is None:
        hid = [w.hidden(l, n, tag=tag or f"inj{n}") for l in range(cfg.L_t)]
    fc, wk, wv = w.fc(), w.wk(), w.wv()
    if cache is None:
        cache = P.new_cache(cfg)
        if prefill is not None:
            cache.k.fill_(prefill)
            cache.v.fill_(prefill)
    ws = D.workspace(D.dflash_inject_workspace(cfg.L_t, n, cfg.d_t, cfg.d, cfg.kv, cfg.act))
    if garbage_seed is not None:
        garbage(ws, garbage_seed)
    gdev = dev(gamma, cfg.act) if gamma is not None else None
    D.dflash_inject([dev(h, cfg.act) for h in hid], wdev(fc), gdev, cfg.eps, wdev(wk), wdev(wv), cache, pos0,
                    ws)
    torch.cuda.synchronize()
    rows = np.arange(n) if rows is None else np.asarray(rows)
    zoff = D.dflash_inject_z_offset(cfg.L_t, n, cfg.d_t, cfg.d, cfg.kv, cfg.act)
    zg = f64(D.ws_view(ws, zoff, (n, cfg.d), P.act_dtype(cfg.act))[torch.as_tensor(rows, device="cuda")])
    gk, gv = rows_of_cache(cache, pos0 + rows)
    gam = act_np(gamma, cfg.act) if gamma is not None else None
    check_inject(cfg, [act_np(h[rows], cfg.act) for h in hid], fc, gam, wk, wv, zg, gk, gv, cfg.name)
    return cache, gk, gv


@pytest.mark.parametrize("n,pos0", [(64, 0), (16, 5), (5, 100), (70, 3)])
def test_inject_tiny_fp32(n, pos0):
    cfg = cfg_small(0, capacity=256)
    cache, _, _ = run_inject(cfg, n, pos0, prefill=7.0)
    # rows outside [pos0, pos0 + n) are untouched
    k = cache.k.cpu()
    assert torch.all(k[:, :pos0] == 7.0) and torch.all(k[:, pos0 + n:] == 7.0)


@pytest.mark.parametrize("n,pos0", [(16, 9), (3, 0), (200, 40)])
def test_inject_qwen27b_shapes(n, pos0):
    run_inject(cfg_small(1, capacity=512), n, pos0)


def test_inject_gamma():
    """A non-trivial RMSNorm gain (gamma != NULL) on the weight-streaming
    (16 rows) and tile (200 rows) paths, bf16 and fp32."""
    for ci, n in [(1, 16), (1, 200), (0, 16)]:
        cfg = cfg_small(ci, capacity=512)
        gamma = synth.normal(cfg.seed, "gamma", (cfg.d,), 1.0, cfg.act)
        run_inject(cfg, n, 7, gamma=gamma, tag=f"gam{n}")


def test_inject_wide_rows_rmsnorm():
    """d > 8192: the RMSNorm reads a row twice (its two-pass path)."""
    cfg = cfg_small(1, d=8320, d_t=512, L_t=2, Hkv=1, capacity=256)
    run_inject(cfg, 5, 11, tag="wide")
    run_inject(cfg, 40, 64, tag="wide40")


def test_inject_decode_rows_at_64k():
    """Config 3: 16 rows injected behind 65536 pre-filled rows."""
    cfg = configs.get(3)
    cache, _, _ = run_inject(cfg, 16, 65536, prefill=0.5)
    assert torch.all(cache.k[:, 65536 + 16:].cpu().float() == 0.5)
    assert torch.all(cache.k[:, :65536].cpu().float() == 0.5)


@pytest.mark.parametrize("ci", [2, 4])
def test_inject_prefill_32k_sampled(ci):
    """The 32768-token prefill (MFMA tile path) at full size, checked on
    sampled rows including the last (ragged) tile."""
    cfg = configs.get(ci)
    rows = [0, 1, 127, 128, 4095, 17000, 32640, 32700, 32766, 32767]
    run_inject(cfg, cfg.n_ctx, 0, rows=rows)


@pytest.mark.parametrize("d,d_t,L_t", [(5184, 1024, 2), (5120, 1088, 1)])
def test_inject_prefill_tile_forms(d, d_t, L_t):
    """6400 rows on the 256 x 256 prefill tiles: a ragged last 256-column
    tile (d = 5184) and K = 1088 (34 k-steps); checked on sampled rows
    including the last tile."""
    rows = [0, 1, 255, 256, 3333, 6143, 6144, 6399]
    run_inject(cfg_small(1, d=d, d_t=d_t, L_t=L_t, capacity=6400), 6400, 0, rows=rows)


@pytest.mark.parametrize("n", [32, 48, 64, 256, 1024, 2048])
def test_inject_batched_blocks(n):
    """Deferred injection: the rows of several stashed blocks at once (split-K
    GEMMs while the tiles leave CUs idle), Qwen-27B shapes; every row up to
    64, sampled rows (first, last, tile edges) beyond."""
    rows = None if n <= 64 else [0, 1, 127, 128, n // 2, n - 2, n - 1]
    run_inject(cfg_small(1, capacity=max(2048, n + 64)), n, 5, rows=rows)


@pytest.mark.parametrize("d,d_t,n", [(512, 256, 16), (512, 256, 5), (576, 192, 16), (576, 192, 5)])
def test_inject_q8_0_decode_rows(d, d_t, n):
    """Q8_0 weight streaming for a few rows: with every K a multiple of 128
    (fc 768, Wk/Wv 512) the four block scales of a chunk come from one 8-byte
    load; with K = 576 the 2-byte scale loads."""
    run_inject(cfg_small(4, d=d, d_t=d_t, L_t=3, Hkv=2, capacity=256), n, 3)


def test_inject_q8_0_batched_rows():
    """Q8_0 weights with 40 rows (split-K direct-to-LDS ring of raw codes)."""
    run_inject(cfg_small(4, d=512, d_t=256, L_t=3, Hkv=2, capacity=256), 40, 9)


@pytest.mark.parametrize("d,d_t,L_t,n", [(576, 320, 3, 100), (448, 192, 2, 300), (640, 128, 4, 17),
                                          (512, 256, 3, 32)])
def test_inject_q8_0_ring_shapes(d, d_t, L_t, n):
    """Q8_0 weights with 17 ... 767 rows through the direct-to-LDS ring of raw
    codes: a ragged last 256-column tile (d = 576, 448, 640), k-splits of
    several 64-wide steps (K = 960, 576, 512, 640), the unsplit form (K = 384
    and 448, fewer than eight steps), ragged row tiles (100, 300, 17, 32
    rows; 17 and 32 rows multiply two 16-row fragments per wave), activation
    sources of 320, 192, 128 and 256 columns."""
    run_inject(cfg_small(4, d=d, d_t=d_t, L_t=L_t, Hkv=2, capacity=512), n, 7)


@pytest.mark.parametrize("d_t,L_t", [(256, 2), (448, 1)])
def test_inject_q8_0_ring_128_row_tiles(d_t, L_t):
    """767 rows against a 2816-wide fc: 64-row tiles would leave no k-split
    over the CUs, so the fc takes 128-row tiles, split (K = 512) and unsplit
    (K = 448, fewer than eight 64-wide steps); checked on sampled rows."""
    run_inject(cfg_small(4, d=2816, d_t=d_t, L_t=L_t, Hkv=2, capacity=1024), 767, 0, rows=[0, 100, 700, 766])


def test_inject_q8_0_ring_full_width():
    """The Q8_0 workload's own fc and Wk / Wv (d = 5376) on 48 rows, checked
    on sampled rows."""
    run_inject(cfg_small(4, capacity=512), 48, 0, rows=[0, 1, 31, 47])


@pytest.mark.parametrize("n", [767, 800, 4133])
def test_inject_q8_0_around_expansion_threshold(n):
    """Q8_0 fc / Wk / Wv on every row just below 768 tokens (the ring of raw
    codes) and above (one bf16 expansion per call), ragged tails."""
    cfg = cfg_small(4, d=512, d_t=256, L_t=3, Hkv=2, capacity=4224)
    run_inject(cfg, n, 17)


@pytest.mark.parametrize("n", [16, 64])
def test_inject_deterministic(n):
    """Bitwise-equal caches from two calls: the counter-based small-weight
    GEMM (16 rows; two KV heads make Wk|Wv 512 rows, four k-groups per tile)
    and the split-K tile path (64 rows) sum in a fixed order."""
    cfg = cfg_small(1, Hkv=2, capacity=256)
    a, _, _ = run_inject(cfg, n, 3, tag="det")
    b, _, _ = run_inject(cfg, n, 3, tag="det", garbage_seed=n)
    assert torch.equal(a.k, b.k) and torch.equal(a.v, b.v)


def test_inject_q8_0_ring_deterministic():
    """Q8_0 weights on the ring of raw codes (40 rows, 64-row tiles split
    along k): two calls, the second on a workspace of random bytes, give
    bitwise-equal caches (the partials are summed in k-piece order)."""
    cfg = cfg_small(4, d=512, d_t=256, L_t=3, Hkv=2, capacity=256)
    a, _, _ = run_inject(cfg, 40, 3, tag="detq")
    b, _, _ = run_inject(cfg, 40, 3, tag="detq", garbage_seed=40)
    assert torch.equal(a.k, b.k) and torch.equal(a.v, b.v)


def test_inject_garbage_workspace():
    """A workspace full of random bytes (any stale completion counter) gives
    correct rows: the counters carry each launch's own stamp."""
    run_inject(cfg_small(1, capacity=256), 16, 40, garbage_seed=7, tag="garb")
    run_inject(cfg_small(1, Hkv=2, capacity=256), 16, 40, garbage_seed=9, tag="garb")
    run_inject(cfg_small(0, capacity=256), 16, 40, garbage_seed=8, tag="garb")


# ---------------------------------------------------------------------------
# (2) conv
# ---------------------------------------------------------------------------

def run_conv(cfg, nb, tag="conv", garbage_seed=None):
    say(f"conv {cfg.name} n_blocks={nb} B={cfg.B} C={cfg.C} G={cfg.G} T={cfg.T}")
    w = synth.Workload(cfg)
    x = synth.normal(cfg.seed, f"{tag}.x.{nb}", (nb, cfg.B, cfg.C), 1.0, cfg.act)
    base, wd = w.conv_base(), w.w_delta()
    out = torch.empty((nb, cfg.B, cfg.C), dtype=P.act_dtype(cfg.act), device="cuda")
    ws = D.workspace(D.dflash_conv_workspace(nb, cfg.B, cfg.C, cfg.G, cfg.T))
    if garbage_seed is not None:
        garbage(ws, garbage_seed)
    D.dflash_conv(dev(x, cfg.act), cfg.G, dev(base, cfg.act), wdev(wd), out, ws)
    torch.cuda.synchronize()
    ref = O.conv(act_np(x, cfg.act), act_np(base, cfg.act), wnp(wd), cfg.G, cfg.act == "bf16")
    assert_close(f64(out), ref["u"], cfg.act, f"{cfg.name} conv u (n_blocks={nb})")


@pytest.mark.parametrize("ci,nb", [(0, 1), (0, 3), (1, 1), (1, 3), (4, 1), (1, 64), (4, 64), (0, 2048)])
def test_conv(ci, nb):
    run_conv(configs.get(ci), nb)


def test_conv_single_tap_and_narrow_groups():
    """T = 1; groups of 3 channels (a thread's 4 channels span two groups);
    T = 3 with 16 groups."""
    run_conv(cfg_small(1, C=384, G=128, T=1, B=7), 2, tag="conv1")
    run_conv(cfg_small(0, T=3, G=16, B=5), 2, tag="conv3")


def test_conv_group_spans_and_long_filters():
    """Every kernel arrangement, with few blocks (one thread per position)
    and with many (one thread per block): 12 channels per group at B = 16 (an
    8-channel chunk spans two groups, as with 84 per group); fp32 at B = 16;
    T = 6 and T = 16 filters; T = 9 and T = 2 with 3-channel groups."""
    run_conv(cfg_small(1, C=768, G=64, T=4, B=16), 3, tag="conv12")
    run_conv(cfg_small(0, C=256, G=8, T=4, B=16), 2, tag="convf16")
    run_conv(cfg_small(0, C=256, G=8, T=6, B=16), 2, tag="conv6")
    run_conv(cfg_small(1, C=128, G=16, T=16, B=16), 2, tag="conv16")
    run_conv(cfg_small(0, C=192, G=64, T=9, B=3), 2, tag="conv9")
    # the same arrangements over enough blocks for the per-block kernel
    run_conv(cfg_small(1, C=768, G=64, T=4, B=16), 200, tag="conv12b")
    run_conv(cfg_small(1, C=384, G=128, T=2, B=8), 400, tag="conv3b")
    run_conv(cfg_small(0, C=256, G=8, T=6, B=16), 600, tag="conv6b")


def test_conv_one_launch_shapes():
    """At most 16 rows with whole 8-channel chunks per group take the
    one-launch kernel with 8-column taps (delta formed per tile of groups, the last workgroup
    of a tile applies the taps): T = 16 (one group per tile), T = 5 and 3
    (tiles of 3 and 5 groups, 15 of 16 rows used, a short last tile), two
    blocks of 8, fp32, and the Qwen-27B width with one k-group per wave
    pair."""
    run_conv(cfg_small(1, C=128, G=16, T=16, B=16), 1, tag="conv1l16")
    run_conv(cfg_small(1, C=512, G=16, T=5, B=16), 1, tag="conv1l5")
    run_conv(cfg_small(0, C=256, G=16, T=3, B=16), 1, tag="conv1l3")
    run_conv(cfg_small(1, C=1024, G=32, T=4, B=8), 2, tag="conv1l2b")
    run_conv(cfg_small(0, C=256, G=8, T=6, B=16), 1, tag="conv1lf")
    run_conv(configs.get(2), 1, tag="conv1lq")


def test_conv_one_launch_four_channel_chunks():
    """Groups of a multiple of 4 but not 8 channels (C / G = 20, 12, and the
    Q8_0 workload's 84) take the one-launch kernel with 4-column taps: bf16
    (8-byte loads), fp32 (16-byte loads), one block of 8 rows and two of 8."""
    run_conv(cfg_small(1, C=320, G=16, T=4, B=16), 1, tag="conv4c20")
    run_conv(cfg_small(0, C=192, G=16, T=3, B=16), 1, tag="conv4c12f")
    run_conv(configs.get(4), 1, tag="conv4cq")
    run_conv(cfg_small(4, B=8), 2, tag="conv4cq2")


def test_conv_batched_32k_tokens():
    """2048 blocks of 16 (32768 tokens, the 32k workload's token count) at
    the Qwen-27B width, checked on every output; then 2050 blocks, whose
    delta product ends in a ragged 32-row tile."""
    run_conv(configs.get(2), 2048, tag="convb")
    run_conv(configs.get(2), 2050, tag="convr")


def test_conv_garbage_workspace():
    run_conv(configs.get(1), 1, tag="convg", garbage_seed=3)
    run_conv(configs.get(0), 1, tag="convg", garbage_seed=4)


# ---------------------------------------------------------------------------
# (2b) feed-forward site: second conv pair, gated SiLU MLP, residual
# ---------------------------------------------------------------------------

def fp32_sum_term(x, W):
    """Higham's bound on fp32 summation of the products x_j W[c, j], n = K + 64
    of them (a k split adds at most 64 partials) in any order, each addition
    correctly rounded: gamma_n sum_j |x_j| |W[c, j]|, gamma_n = n u / (1 - n u),
    u = 2^-24.  It matters only where a long product cancels to a result far
    below its terms (the Q8_0 workload's weights are O(1), not O(1/sqrt(K)))."""
    n = x.shape[-1] + 64
    u = 2.0 ** -24
    return n * u / (1 - n * u) * (np.abs(x) @ np.abs(W).T)


def run_ffn(cfg, nb, tag="ffn", garbage_seed=None):
    """Stage-wise: u against the oracle's conv of h; act against the oracle's
    gated MLP of the GPU's u; out against the oracle's down product of the
    GPU's act plus h, with the fp32 summation term of the down product.  End
    to end: out against the oracle chain (plus, for bf16 workloads,
    |act_gpu - act_ref| |Wd|^T, the propagation of the stage-checked act
    through the down product, and the same summation term)."""
    d, G, T, F = cfg.d, cfg.G, cfg.T, cfg.d_ff
    say(f"ffn {cfg.name} n_blocks={nb} B={cfg.B} d={d} d_ff={F} G={G} T={T} weight={cfg.weight}")
    w = synth.Workload(cfg)
    h = synth.normal(cfg.seed, f"{tag}.h.{nb}", (nb, cfg.B, d), 1.0, cfg.act)
    base, wd, wg, wu, wn = w.ffn_conv_base(), w.ffn_w_delta(), w.w_gate(), w.w_up(), w.w_down()
    dt = P.act_dtype(cfg.act)
    out = torch.empty((nb, cfg.B, d), dtype=dt, device="cuda")
    args = (nb, cfg.B, d, G, T, F)
    ws = D.workspace(D.dflash_ffn_block_workspace(*args))
    if garbage_seed is not None:
        garbage(ws, garbage_seed)
    D.dflash_ffn_block(dev(h, cfg.act), G, dev(base, cfg.act), wdev(wd), wdev(wg), wdev(wu), wdev(wn), out, ws)
    torch.cuda.synchronize()
    M = nb * cfg.B
    ug = f64(D.ws_view(ws, D.dflash_ffn_block_u_offset(*args), (M, d), dt))
    ag = f64(D.ws_view(ws, D.dflash_ffn_block_act_offset(*args), (M, F), dt))
    outg = f64(out).reshape(M, d)
    bp = cfg.act == "bf16"
    H = act_np(h, cfg.act)
    Wg, Wu, Wn = wnp(wg), wnp(wu), wnp(wn)
    c = O.conv(H, act_np(base, cfg.act), wnp(wd), G, bp)
    assert_close(ug, c["u"].reshape(M, d), cfg.act, f"{cfg.name} ffn u (n_blocks={nb})")
    f = O.ffn_hidden(ug, Wg, Wu, bp)
    assert_close(ag, f["act"], cfg.act, f"{cfg.name} ffn act from the GPU's u")
    H2 = H.reshape(M, d)
    sum_term = fp32_sum_term(ag, Wn)
    assert_close(outg, O.ffn_out(H2, ag, Wn, bp), cfg.act, f"{cfg.name} ffn out from the GPU's act",
                 term=sum_term)
    ref = O.ffn_block(H, act_np(base, cfg.act), wnp(wd), G, Wg, Wu, Wn, bp)
    term = sum_term + (np.abs(ag - ref["act"].reshape(M, F)) @ np.abs(Wn).T if bp else 0.0)
    assert_close(outg, ref["out"].reshape(M, d), cfg.act, f"{cfg.name} ffn out end to end", term=term)


@pytest.mark.parametrize("ci,nb", [(0, 1), (0, 3), (1, 1), (4, 1)])
def test_ffn_block(ci, nb):
    run_ffn(configs.get(ci), nb)


def test_ffn_block_many_rows():
    """1024 and 1040 rows (the tiled GEMMs, the second with a ragged tile) at
    a narrower width, bf16 and Q8_0 weights; 600 fp32 rows; 520 Q8_0 rows
    whose gate | up product runs without a k split."""
    run_ffn(cfg_small(1, d=1024, C=1024, d_ff=2048), 64, tag="ffnm")
    run_ffn(cfg_small(1, d=1024, C=1024, d_ff=2048, B=13), 80, tag="ffnr")
    run_ffn(cfg_small(4, d=1024, C=1024, d_ff=1536), 50, tag="ffnq")
    run_ffn(configs.get(0), 75, tag="ffnf")
    # Q8_0 gate | up over 1280 tiles of 128 x 128: the tile kernel without a k split;
    # the down product sums 16384 O(1)-weighted terms (the fp32 summation term)
    run_ffn(cfg_small(4, d=1024, C=1024, d_ff=16384), 65, tag="ffnqw")


def test_ffn_block_odd_shapes_and_garbage_workspace():
    """B = 5, T = 2, groups of 96 channels, d_ff = 64; random workspace bytes."""
    run_ffn(cfg_small(1, d=384, C=384, G=4, T=2, B=5, d_ff=64), 2, tag="ffno", garbage_seed=11)
    run_ffn(configs.get(0), 1, tag="ffng", garbage_seed=12)


# ---------------------------------------------------------------------------
# (3) block attention
# ---------------------------------------------------------------------------

def check_attn(cfg, U, X, wq, wk, wv, wo, CK, CV, n_ctx, scale, qkvg, og, outg, what, B):
    """Stage-wise: Q | Kb | Vb against the oracle's projections of u; O
    against the oracle's softmax over the GPU's Q, Kb, Vb (plus the bound for
    softmax weights rounded to bf16); out against the oracle's Wo product of
    the GPU's O.  End to end: out against the oracle chain (Q8_0 weights:
    plus |Wo| |O_gpu - O_ref|, the propagation of the stage-checked O)."""
    bp = cfg.act == "bf16"
    Wq, Wk, Wv, Wo = wnp(wq), wnp(wk), wnp(wv), wnp(wo)
    qd, kv = cfg.Hq * cfg.hd, cfg.Hkv * cfg.hd
    p = O.attn_qkv(U, Wq, Wk, Wv, bp)
    assert_close(qkvg[:, :qd], p["q"], cfg.act, f"{what} Q")
    assert_close(qkvg[:, qd:qd + kv], p["kb"], cfg.act, f"{what} Kb")
    assert_close(qkvg[:, qd + kv:], p["vb"], cfg.act, f"{what} Vb")
    c = O.attn_core(qkvg[:, :qd], qkvg[:, qd:qd + kv], qkvg[:, qd + kv:], CK, CV, n_ctx, cfg.Hq, scale, bp,
                    with_bound=True)
    assert_close(og, c["o"], cfg.act, f"{what} O from the GPU's Q, Kb, Vb",
                 term=c["o_bound"] if bp else None)
    assert_close(outg, O.attn_out(og, Wo, X, bp), cfg.act, f"{what} out from the GPU's O")
    ref = O.block_attn(U, X, Wq, Wk, Wv, Wo, CK, CV, n_ctx, cfg.Hq, scale, bp)
    if cfg.weight == "q8_0":
        assert_close(outg, ref["out"], cfg.act, f"{what} out end to end",
                     term=np.abs(og - ref["o"]) @ np.abs(Wo).T)
    else:
        assert_close(outg, ref["out"], cfg.act, f"{what} out end to end")
    return ref


def run_attn(cfg, n_ctx, cap=None, resid=True, B=None, poison=False, scale=0.0, garbage_seed=None):
    """poison: cache positions from n_ctx on hold NaN (the attention must not
    read them into the result, also where a tile ends inside a V panel)."""
    B = cfg.B if B is None else B
    cap = cap or -(-(n_ctx + 64) // 64) * 64   # the library wants a multiple of 64
    say(f"attn {cfg.name} B={B} n_ctx={n_ctx} cap={cap} scale={scale}")
    w = synth.Workload(cfg)
    shp = (cfg.Hkv, cap, cfg.hd)
    ck = synth.normal(cfg.seed, f"attn.ck.{cap}", shp, 1.0, cfg.act)
    cv = synth.normal(cfg.seed, f"attn.cv.{cap}", shp, 1.0, cfg.act)
    u = synth.normal(cfg.seed, "attn.u", (B, cfg.d), 1.0, cfg.act)
    x = synth.normal(cfg.seed, "attn.x", (B, cfg.d), 1.0, cfg.act)
    wq, wk, wv, wo = w.wq(), w.wk(), w.wv(), w.wo()
    ck_d, cv_d = dev(ck, cfg.act), dev(cv, cfg.act)
    if poison:
        ck_d[:, n_ctx:, :] = float("nan")
        cv_d[:, n_ctx:, :] = float("nan")
    cache = D.KVCache(ck_d, D.v_panels(cv_d))
    dt = P.act_dtype(cfg.act)
    out = torch.empty((B, cfg.d), dtype=dt, device="cuda")
    args = (B, cfg.d, cfg.Hq, cfg.Hkv, cfg.hd, n_ctx)
    ws = D.workspace(D.dflash_block_attn_workspace(*args))
    if garbage_seed is not None:
        garbage(ws, garbage_seed)
    xd = dev(x, cfg.act)
    D.dflash_block_attn(dev(u, cfg.act), xd if resid else None, cfg.Hq, wdev(wq), wdev(wk), wdev(wv),
                        wdev(wo), cache, n_ctx, scale, out, ws)
    torch.cuda.synchronize()
    qd, kv = cfg.Hq * cfg.hd, cfg.Hkv * cfg.hd
    qkvg = f64(D.ws_view(ws, D.dflash_block_attn_qkv_offset(*args), (B, qd + 2 * kv), dt))
    og = f64(D.ws_view(ws, D.dflash_block_attn_o_offset(*args), (B, qd), dt))
    check_attn(cfg, act_np(u, cfg.act), act_np(x, cfg.act) if resid else None, wq, wk, wv, wo,
               act_np(ck, cfg.act), act_np(cv, cfg.act), n_ctx, scale, qkvg, og, f64(out),
               f"{cfg.name} attn (n_ctx={n_ctx})", B)
    return out


@pytest.mark.parametrize("n_ctx", [64, 0, 1, 200, 777])
def test_attn_tiny_fp32(n_ctx):
    run_attn(configs.get(0), n_ctx)


def test_attn_tiny_no_residual_short_block():
    run_attn(configs.get(0), 64, resid=False, B=3)


@pytest.mark.parametrize("ci,n_ctx", [(1, 1024), (1, 1000), (2, 32768), (3, 65536 + 16), (4, 32768)])
def test_attn_full(ci, n_ctx):
    run_attn(configs.get(ci), n_ctx)


def test_attn_explicit_scale():
    """A caller-given softmax scale (scale != 0) instead of 1/sqrt(hd)."""
    run_attn(configs.get(0), 200, scale=0.05)
    run_attn(configs.get(1), 1000, scale=0.21)


def test_attn_garbage_workspace():
    """Random bytes in the workspace: the Q|Kb|Vb product of the small fp32
    layer runs on the counter path."""
    run_attn(configs.get(0), 200, garbage_seed=5)
    run_attn(configs.get(1), 1000, garbage_seed=6)


def test_attn_many_splits():
    """More than 64 splits per KV head (two KV heads over a long context): the
    combine kernel's multi-group path, with a partial last group."""
    run_attn(cfg_small(0, n_ctx=5000), 5000)                           # fp32, hd 64: 157 splits
    run_attn(cfg_small(1, Hq=8, Hkv=2, n_ctx=8000), 8000)              # bf16, hd 128: 250 splits


@pytest.mark.parametrize("ci,n_ctx", [(0, 77), (0, 200), (1, 1000), (1, 31), (4, 4133)])
def test_attn_cache_tail_not_finite(ci, n_ctx):
    """The context ends inside a 32-position V panel whose other positions
    hold NaN: they get zero weight and must not turn the output into NaN."""
    run_attn(configs.get(ci), n_ctx, poison=True)


def test_attn_deterministic():
    cfg = configs.get(1)
    a = run_attn(cfg, 1024)
    b = run_attn(cfg, 1024)
    assert torch.equal(a, b)


# ---------------------------------------------------------------------------
# Q8_0 KV cache: the quantising injection and the attention over codes
# ---------------------------------------------------------------------------

def q8_fill(cache, k_rows, v_rows, p0=0):
    """Oracle-quantised rows [Hkv][n][hd] (fp64) into a device Q8_0 cache at
    positions [p0, p0 + n), p0 and n multiples of 32; returns the values the
    attention must read (the oracle's dequantisation, reading R-KVQ)."""
    kc, ks = O.kv_quant_q8_0(k_rows)
    vc, vs = O.kv_quant_q8_0(v_rows)
    n = k_rows.shape[1]
    cache.k[:, p0:p0 + n] = torch.from_numpy(kc).cuda()
    cache.v[:, p0 // 32:(p0 + n) // 32] = D.v_panels(torch.from_numpy(vc).cuda())
    cache.k_scales[:, p0:p0 + n] = torch.from_numpy(ks).cuda()
    cache.v_scales[:, p0:p0 + n] = torch.from_numpy(vs).cuda()
    return O.kv_dequant_q8_0(kc, ks, True), O.kv_dequant_q8_0(vc, vs, True)


def q8_rows(cache, pos):
    """Codes and fp16 scales [Hkv][len(pos)][.] of K and V at positions `pos`."""
    p = torch.as_tensor(np.asarray(pos), device="cuda")
    return (cache.k[:, p].cpu().numpy(), cache.k_scales[:, p].cpu().numpy(),
            D.v_rows(cache.v)[:, p].cpu().numpy(), cache.v_scales[:, p].cpu().numpy())


def check_q8_rows(what, codes, scales, ref_codes, ref_scales):
    """Codes within one level and scales within one fp16 step of the oracle's
    quantisation of the same fp32 rows (the GPU forms 1 / scale and the
    products in fp32, the oracle in fp64, so a value on a rounding boundary
    may go either way); report how many are exactly equal."""
    dc = np.abs(codes.astype(np.int32) - ref_codes.astype(np.int32))
    sb = scales.view(np.int16).astype(np.int32) - ref_scales.view(np.int16).astype(np.int32)
    assert dc.max() <= 1, (what, "codes", int(dc.max()))
    assert np.abs(sb).max() <= 1, (what, "scales", int(np.abs(sb).max()))
    say(f"  {what}: {int((dc == 0).sum())}/{dc.size} codes and {int((sb == 0).sum())}/{sb.size} scales equal "
        f"to the oracle's, the rest one step off")


def run_inject_q8(cfg, n, pos0, cache=None, hid=None, tag=None):
    """Injection into a Q8_0 cache: the GPU's z against the oracle; the codes
    and scales against the oracle's quantisation of z_gpu . Wk^T / Wv^T (the
    unrounded projections).  Returns (cache, K values, V values) as the
    attention reads them (the oracle's dequantisation of the GPU's codes)."""
    say(f"inject q8_0 cache {cfg.name} n={n} pos0={pos0}")
    w = synth.Workload(cfg)
    if hid is None:
        hid = [w.hidden(l, n, tag=tag or f"injq{n}") for l in range(cfg.L_t)]
    fc, wk, wv = w.fc(), w.wk(), w.wv()
    if cache is None:
        cache = P.new_cache(cfg, kv="q8_0")
    ws = D.workspace(D.dflash_inject_workspace(cfg.L_t, n, cfg.d_t, cfg.d, cfg.kv, cfg.act))
    D.dflash_inject([dev(h, cfg.act) for h in hid], wdev(fc), None, cfg.eps, wdev(wk), wdev(wv), cache, pos0, ws)
    torch.cuda.synchronize()
    zoff = D.dflash_inject_z_offset(cfg.L_t, n, cfg.d_t, cfg.d, cfg.kv, cfg.act)
    zg = f64(D.ws_view(ws, zoff, (n, cfg.d), P.act_dtype(cfg.act)))
    enc = O.encode([act_np(h, cfg.act) for h in hid], wnp(fc), None, cfg.eps, True)
    assert_close(zg, enc["z"], cfg.act, f"{cfg.name} z (Q8_0 cache)")
    shp = lambda x: x.reshape(n, cfg.Hkv, cfg.hd).transpose(1, 0, 2)
    rk, rks = O.kv_quant_q8_0(shp(zg @ wnp(wk).T))
    rv, rvs = O.kv_quant_q8_0(shp(zg @ wnp(wv).T))
    kc, ks, vc, vs = q8_rows(cache, pos0 + np.arange(n))
    check_q8_rows(f"{cfg.name} K codes", kc, ks, rk, rks)
    check_q8_rows(f"{cfg.name} V codes", vc, vs, rv, rvs)
    return cache, O.kv_dequant_q8_0(kc, ks, True), O.kv_dequant_q8_0(vc, vs, True)


@pytest.mark.parametrize("n,pos0", [(16, 40), (5, 0), (200, 77)])
def test_inject_q8_0_cache(n, pos0):
    """The quantising store: decode rows (16, ragged 5, and a 200-row tile
    GEMM) at offsets inside and across V panels; positions around are
    untouched."""
    cfg = cfg_small(1, capacity=512)
    cache = P.new_cache(cfg, kv="q8_0")
    cache.k.fill_(3)
    cache.k_scales.fill_(1.5)
    run_inject_q8(cfg, n, pos0, cache=cache)
    k = cache.k.cpu()
    assert torch.all(k[:, :pos0] == 3) and torch.all(k[:, pos0 + n:] == 3)
    assert torch.all(cache.k_scales[:, pos0 + n:].cpu().float() == 1.5)


def run_attn_q8(cfg, n_ctx, poison=False, B=None):
    """Attention over a Q8_0 cache of seeded N(0,1) rows quantised by the
    oracle; stage-fed checks as for the bf16 cache, with the oracle reading
    the dequantised codes.  poison: scales past n_ctx are NaN."""
    B = cfg.B if B is None else B
    cap = -(-(n_ctx + 64) // 64) * 64
    say(f"attn q8_0 cache {cfg.name} B={B} n_ctx={n_ctx} cap={cap}")
    w = synth.Workload(cfg)
    shp = (cfg.Hkv, cap, cfg.hd)
    kr = synth.normal(cfg.seed, f"attnq.ck.{cap}", shp, 1.0, "f32").astype(np.float64)
    vr = synth.normal(cfg.seed, f"attnq.cv.{cap}", shp, 1.0, "f32").astype(np.float64)
    cache = P.new_cache(configs.shrink(cfg, capacity=cap), kv="q8_0")
    CK, CV = q8_fill(cache, kr, vr)
    if poison:
        cache.k_scales[:, n_ctx:] = float("nan")
        cache.v_scales[:, n_ctx:] = float("nan")
    u = synth.normal(cfg.seed, "attnq.u", (B, cfg.d), 1.0, cfg.act)
    x = synth.normal(cfg.seed, "attnq.x", (B, cfg.d), 1.0, cfg.act)
    wq, wk, wv, wo = w.wq(), w.wk(), w.wv(), w.wo()
    dt = P.act_dtype(cfg.act)
    out = torch.empty((B, cfg.d), dtype=dt, device="cuda")
    args = (B, cfg.d, cfg.Hq, cfg.Hkv, cfg.hd, n_ctx)
    ws = D.workspace(D.dflash_block_attn_workspace(*args))
    D.dflash_block_attn(dev(u, cfg.act), dev(x, cfg.act), cfg.Hq, wdev(wq), wdev(wk), wdev(wv), wdev(wo), cache,
                        n_ctx, 0.0, out, ws)
    torch.cuda.synchronize()
    qd, kv = cfg.Hq * cfg.hd, cfg.Hkv * cfg.hd
    qkvg = f64(D.ws_view(ws, D.dflash_block_attn_qkv_offset(*args), (B, qd + 2 * kv), dt))
    og = f64(D.ws_view(ws, D.dflash_block_attn_o_offset(*args), (B, qd), dt))
    check_attn(cfg, act_np(u, cfg.act), act_np(x, cfg.act), wq, wk, wv, wo, CK, CV, n_ctx, 0.0, qkvg, og, f64(out),
               f"{cfg.name} attn over a Q8_0 cache (n_ctx={n_ctx})", B)


@pytest.mark.parametrize("ci,n_ctx", [(1, 1000), (1, 31), (1, 0), (1, 1), (2, 32768), (3, 65552), (4, 32768),
                                      (4, 4133)])
def test_attn_q8_0_cache(ci, n_ctx):
    """Full-size contexts, ragged ends inside a panel, no or one context key;
    the Q8_0-weight workload at B = 8 (two column tiles per wave)."""
    run_attn_q8(configs.get(ci), n_ctx)


@pytest.mark.parametrize("ci,n_ctx", [(1, 77), (4, 1000)])
def test_attn_q8_0_cache_tail_not_finite(ci, n_ctx):
    run_attn_q8(configs.get(ci), n_ctx, poison=True)


def test_attn_q8_0_cache_small_groups():
    """Two query heads per KV head (waves 2-3 without a head), B = 5."""
    run_attn_q8(cfg_small(1, Hq=16, Hkv=8), 777, B=5)


def test_attn_q8_0_cache_eight_head_groups():
    """Eight query heads per KV head (two per wave) at B = 16: 128 query rows
    per KV head; a context that ends inside a tile."""
    run_attn_q8(cfg_small(1, Hq=64, Hkv=8), 3001)


# ---------------------------------------------------------------------------
# (4) LM head, top-K, unary
# ---------------------------------------------------------------------------

def run_topk(cfg, h=None, w_lm=None, tag="topk"):
    say(f"topk {cfg.name} V={cfg.V} K={cfg.K} B={cfg.B} weight={cfg.weight}")
    w = synth.Workload(cfg)
    if h is None:
        h = synth.normal(cfg.seed, tag + ".h", (cfg.B, cfg.d), 1.0, cfg.act)
    if w_lm is None:
        w_lm = w.w_lm()
    idx = torch.empty((cfg.B, cfg.K), dtype=torch.int32, device="cuda")
    un = torch.empty((cfg.B, cfg.K), dtype=torch.float32, device="cuda")
    ws = D.workspace(D.dflash_topk_unary_workspace(cfg.B, cfg.V, cfg.K))
    wl = wdev(w_lm)
    D.dflash_topk_unary(dev(h, cfg.act), wl, cfg.K, idx, un, ws)
    torch.cuda.synchronize()
    logits = O.lm_logits_stored(act_np(h, cfg.act), w_lm)
    gi, gu = idx.cpu().numpy(), un.cpu().numpy()
    check_topk(gi, gu, logits, cfg.K, cfg.act, f"{cfg.name} top-{cfg.K}")
    return gi, gu, logits


@pytest.mark.parametrize("ci", [0, 1, 4])
def test_topk_full(ci):
    run_topk(configs.get(ci))


@pytest.mark.parametrize("V,K,B", [(1007, 32, 5), (20, 20, 16), (16, 1, 1), (33, 7, 2), (5000, 16, 16)])
def test_topk_ragged_and_extremes(V, K, B):
    run_topk(cfg_small(0, V=V, K=K, B=B), tag=f"topk{V}.{K}")


@pytest.mark.parametrize("ci,V,K,B", [(1, 40009, 8, 16), (1, 32791, 32, 5), (4, 49157, 8, 8), (0, 70001, 3, 8)])
def test_topk_resident_path_ragged(ci, V, K, B):
    """Vocabularies with at least eight 16-row tiles per CU (one per wave of
    the 256 resident workgroups) take the LDS-resident path; ragged last tile,
    uneven tiles per wave, K up to 32, Q8_0, fp32."""
    run_topk(cfg_small(ci, V=V, K=K, B=B), tag=f"topkr{V}.{K}")


def test_topk_zero_hidden_ties():
    """h = 0: every logit is 0, so the answer is 0..K-1 with unary -ln V."""
    cfg = cfg_small(1, V=4099)
    h = np.zeros((cfg.B, cfg.d), dtype=np.uint16)
    gi, gu, _ = run_topk(cfg, h=h)
    assert np.array_equal(gi, np.tile(np.arange(cfg.K), (cfg.B, 1)))
    np.testing.assert_allclose(gu, -np.log(cfg.V), rtol=1e-5)


def test_topk_q8_0_scale_one_is_integer_exact():
    """Q8_0 with every scale 1 and small-integer activations: the logits are
    exact integers (bit-exact int8 matmul), so the top-K indices -- ties broken
    by the lower index -- must equal the oracle's exactly."""
    cfg = cfg_small(4, V=20000, B=8, K=8)
    q, _ = synth.q8_0(cfg.seed, "scale1", cfg.V, cfg.d)
    ones = np.ones((cfg.V, cfg.d // 32), dtype=np.float16)
    wl = {"dtype": "q8_0", "rows": cfg.V, "cols": cfg.d, "data": q, "scales": ones}
    hi = synth.integers(cfg.seed, "scale1.h", -2, 3, (cfg.B, cfg.d)).astype(np.float32)
    h = synth.f32_to_bf16_bits(hi)
    gi, gu, logits = run_topk(cfg, h=h, w_lm=wl)
    assert np.all(logits == np.round(logits))
    ref = O.topk_unary_from_logits(logits, cfg.K)
    assert np.array_equal(gi, ref["idx"])
    # doubling every scale doubles every logit exactly: same indices
    wl2 = dict(wl, scales=(ones * 2).astype(np.float16))
    gi2, _, _ = run_topk(cfg, h=h, w_lm=wl2)
    assert np.array_equal(gi2, gi)


def test_topk_deterministic():
    cfg = configs.get(1)
    a = run_topk(cfg)
    b = run_topk(cfg)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def run_topk_rows(x: np.ndarray, K: int):
    """dflash_topk_rows against the oracle's selection (value descending,
    equal values by ascending column): indices and values bit-exact."""
    say(f"topk_rows rows={x.shape[0]} cols={x.shape[1]} K={K}")
    xd = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    idx = torch.empty(x.shape[0], K, dtype=torch.int32, device="cuda")
    val = torch.empty(x.shape[0], K, dtype=torch.float32, device="cuda")
    ws = D.workspace(D.dflash_topk_rows_workspace(x.shape[0], x.shape[1], K))
    D.dflash_topk_rows(xd, K, idx, val, ws)
    torch.cuda.synchronize()
    ref = O.top_k_select(x.astype(np.float64), K)
    gi = idx.cpu().numpy()
    assert np.array_equal(gi, ref), f"first row differing: {np.where((gi != ref).any(1))[0][:3]}"
    assert np.array_equal(val.cpu().numpy(), np.take_along_axis(x.astype(np.float32), ref, axis=1))


@pytest.mark.parametrize("rows,cols,K", [(1, 1, 1), (3, 128, 64), (4096, 128, 64), (5, 1000, 1000),
                                         (64, 4096, 1024), (2, 200000, 64), (2, 200000, 1024),
                                         (7, 33333, 333)])
def test_topk_rows_random(rows, cols, K):
    rng = np.random.default_rng(rows * 7919 + cols + K)
    run_topk_rows(rng.standard_normal((rows, cols)).astype(np.float32), K)


@pytest.mark.parametrize("rows,cols,K", [(65535, 130, 7), (3, 200000, 1), (2, 16384, 64), (1, 8192, 1024)])
def test_topk_rows_limits(rows, cols, K):
    """The most rows a call takes (one grid row each), K = 1 from wide rows,
    widths that are whole segments, and the largest K on one segment."""
    rng = np.random.default_rng(rows + cols + K)
    run_topk_rows(rng.standard_normal((rows, cols)).astype(np.float32), K)


@pytest.mark.parametrize("rows,cols,K", [(3, 11284, 100), (2, 22548, 1000), (4, 81925, 1000)])
def test_topk_rows_short_last_list(rows, cols, K):
    """Widths whose last segment holds fewer than K scores: its candidate
    list is padded, and a later pass then sees a segment with more than K
    entries but fewer than K real keys.  Row 0 increases along the row, so
    its top K are exactly the keys in that segment; the other rows are
    random or decreasing."""
    rng = np.random.default_rng(cols + K)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x[0] = np.arange(cols, dtype=np.float32)
    x[-1] = -np.arange(cols, dtype=np.float32)
    run_topk_rows(x, K)


def test_topk_rows_ties_signed_zero_and_constant_rows():
    rng = np.random.default_rng(5)
    x = rng.integers(-3, 4, size=(6, 20000)).astype(np.float32)   # heavy ties
    x[1] = 0.0
    x[1, ::3] = -0.0                                              # -0.0 counts as +0.0
    x[2] = 1.5                                                    # one value everywhere
    x[3, 100:] = -3.0e38                                         # far below the rest
    run_topk_rows(x, 700)
    run_topk_rows(x[:, :900], 900)


# ---------------------------------------------------------------------------
# (5) selector edges + path, (6) accept length
# ---------------------------------------------------------------------------

def check_selector(ref, ge, gp, idx, what):
    """Edges element by element (fp32 arithmetic on exact inputs); the path
    exact where the best path beats the runner-up by more than GAP, else the
    GPU's path scores within GAP of the best."""
    assert_close(ge, ref["edges"], "f32", f"{what} edges")
    gap = ref["score"] - ref["runner_up"]
    if gap > GAP:
        assert np.array_equal(gp, ref["path"]), (gp, ref["path"])
    else:
        slots = [int(np.where(idx[i] == gp[i])[0][0]) for i in range(len(gp))]
        assert O.path_score(ref["edges"], slots) >= ref["score"] - GAP
    say(f"  {what}: path gap {gap:.3g}")
    return gap


def run_selector(cfg, anchor=None, tag="sel", garbage_seed=None):
    say(f"selector {cfg.name} B={cfg.B} K={cfg.K} r={cfg.r} V={cfg.V}")
    w = synth.Workload(cfg)
    h = synth.normal(cfg.seed, tag + ".h", (cfg.B, cfg.d), 1.0, cfg.act)
    idx = synth.distinct_indices(cfg.seed, tag + ".idx", cfg.B, cfg.K, cfg.V)
    un = -np.sort(np.abs(synth.normal(cfg.seed, tag + ".un", (cfg.B, cfg.K), 4.0, "f32")), axis=1)
    A, Bc = w.codebooks()
    Pw = w.sel_proj()
    anchor = int(w.anchor()[0]) if anchor is None else anchor
    edges = torch.empty((cfg.B, cfg.K, cfg.K), dtype=torch.float32, device="cuda")
    path = torch.empty((cfg.B,), dtype=torch.int32, device="cuda")
    ws = D.workspace(D.dflash_selector_edges_workspace(cfg.B, cfg.r, cfg.d, cfg.K))
    if garbage_seed is not None:
        garbage(ws, garbage_seed)
    ref = O.selector(act_np(h, cfg.act), wnp(Pw), act_np(A, cfg.act), act_np(Bc, cfg.act), idx,
                     un.astype(np.float32).astype(np.float64), anchor)
    # targets that agree with the oracle's path up to a seeded position: the
    # accept length computed in the selector's kernel
    tgt, m = synth.targets_with_mismatch(cfg.seed, tag + ".tgt", ref["path"][None, :], cfg.V)
    acc = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    D.dflash_selector_edges(dev(h, cfg.act), wdev(Pw), dev(A, cfg.act), dev(Bc, cfg.act),
                            torch.from_numpy(idx).cuda(), torch.from_numpy(un.astype(np.float32)).cuda(),
                            anchor, edges, path, ws, target=torch.from_numpy(tgt[0]).cuda(), accept=acc)
    torch.cuda.synchronize()
    gp = path.cpu().numpy()
    check_selector(ref, edges.cpu().numpy().astype(np.float64), gp, idx, cfg.name)
    assert int(acc.cpu()[0]) == int(O.accept_len(gp[None, :], tgt)[0])
    return gp, ref


@pytest.mark.parametrize("ci", [0, 1, 4])
def test_selector(ci):
    run_selector(configs.get(ci))


def test_selector_no_anchor_and_wide_k():
    run_selector(configs.get(0), anchor=-1)
    run_selector(cfg_small(1, K=32, B=16, r=256), tag="selK32")
    run_selector(cfg_small(1, K=1, B=1), tag="selK1")
    # one-workgroup path with more than 64 KB of LDS (K=32, r=256 above does
    # not fit in LDS and takes the two-kernel path)
    run_selector(cfg_small(1, K=16, B=16, r=64), tag="selK16")


def test_selector_one_launch_slices():
    """The one-launch selector's k-slices of the projection: d with a
    64-wide last piece (5184 = 40.5 pieces of 128), r = 48 (three P tiles of
    five waves each), d = 64 (one 64-wide piece, one workgroup), and fp32
    activations over several slices."""
    run_selector(cfg_small(1, d=5184), tag="sel1l1")
    run_selector(cfg_small(1, r=48, d=1024), tag="sel1l2")
    run_selector(cfg_small(1, d=64, r=16), tag="sel1l3")
    run_selector(cfg_small(0, d=2112), tag="sel1l4")


def test_selector_garbage_workspace():
    run_selector(configs.get(1), tag="selg", garbage_seed=9)


def run_topk_select(cfg, tag="tks", garbage_seed=None):
    """dflash_topk_select against dflash_topk_unary then dflash_selector_edges
    on the same inputs: idx, unary, edges, path and accept bit for bit; the
    top-K also against the oracle's logits."""
    say(f"topk_select {cfg.name} V={cfg.V} K={cfg.K} B={cfg.B} r={cfg.r} weight={cfg.weight}")
    w = synth.Workload(cfg)
    h = synth.normal(cfg.seed, tag + ".h", (cfg.B, cfg.d), 1.0, cfg.act)
    w_lm = w.w_lm()
    A, Bc = w.codebooks()
    hd, wl, pw = dev(h, cfg.act), wdev(w_lm), wdev(w.sel_proj())
    ad, bd = dev(A, cfg.act), dev(Bc, cfg.act)
    anchor = int(w.anchor()[0])
    B, K = cfg.B, cfg.K

    def outs():
        return (torch.empty((B, K), dtype=torch.int32, device="cuda"),
                torch.empty((B, K), dtype=torch.float32, device="cuda"),
                torch.empty((B, K, K), dtype=torch.float32, device="cuda"),
                torch.empty((B,), dtype=torch.int32, device="cuda"),
                torch.full((1,), -1, dtype=torch.int32, device="cuda"))

    i1, u1, e1, p1, a1 = outs()
    D.dflash_topk_unary(hd, wl, K, i1, u1, D.workspace(D.dflash_topk_unary_workspace(B, cfg.V, K)))
    # a target that leaves the first path at position min(5, B - 1)
    D.dflash_selector_edges(hd, pw, ad, bd, i1, u1, anchor, e1, p1,
                            D.workspace(D.dflash_selector_edges_workspace(B, cfg.r, cfg.d, K)))
    torch.cuda.synchronize()
    tgt = p1.clone()
    m = min(5, B - 1)
    tgt[m] = (tgt[m] + 1) % cfg.V
    D.dflash_selector_edges(hd, pw, ad, bd, i1, u1, anchor, e1, p1,
                            D.workspace(D.dflash_selector_edges_workspace(B, cfg.r, cfg.d, K)),
                            target=tgt, accept=a1)
    i2, u2, e2, p2, a2 = outs()
    ws = D.workspace(D.dflash_topk_select_workspace(B, cfg.V, K, cfg.r, cfg.d))
    if garbage_seed is not None:
        garbage(ws, garbage_seed)
    D.dflash_topk_select(hd, wl, K, pw, ad, bd, anchor, i2, u2, e2, p2, ws, target=tgt, accept=a2)
    torch.cuda.synchronize()
    for x, y, what in [(i1, i2, "idx"), (u1, u2, "unary"), (e1, e2, "edges"), (p1, p2, "path"),
                       (a1, a2, "accept")]:
        assert torch.equal(x, y), f"{cfg.name} {what} differs from the two calls"
    assert int(a2[0]) == m
    logits = O.lm_logits_stored(act_np(h, cfg.act), w_lm)
    check_topk(i2.cpu().numpy(), u2.cpu().numpy(), logits, K, cfg.act, f"{cfg.name} combined top-{K}")


@pytest.mark.parametrize("ci", [0, 1, 4])
def test_topk_select_matches_two_calls(ci):
    """c1 (bf16 head) and c4 (Q8_0 head, B = 8) take the one-kernel merge +
    selector; c0's small head takes the two calls' kernels."""
    run_topk_select(configs.get(ci))


def test_topk_select_shapes_and_garbage_workspace():
    """K < 8 and B < 16 on the one-kernel form (the merge and selector sized
    from B and K), r = 48, a garbage workspace (stale counters), fp32 with a
    resident head, and K = 16 (the two calls' kernels)."""
    run_topk_select(cfg_small(1, V=40009, K=5, B=7), tag="tks5", garbage_seed=21)
    run_topk_select(cfg_small(1, V=40009, r=48), tag="tks48")
    run_topk_select(cfg_small(0, V=70001, K=8, B=8), tag="tksf")
    run_topk_select(cfg_small(1, V=40009, K=16), tag="tks16")


def test_accept_len():
    rng_path = synth.integers(11, "acc.path", 0, 1000, (300, 16))
    tgt, m = synth.targets_with_mismatch(11, "acc.tgt", rng_path, 1000)
    acc = torch.empty((300,), dtype=torch.int32, device="cuda")
    D.dflash_accept_len(torch.from_numpy(rng_path).cuda(), torch.from_numpy(tgt).cuda(), acc)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), m)
    assert np.array_equal(O.accept_len(rng_path, tgt), m)


# ---------------------------------------------------------------------------
# the chained block step
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("ci", [0, 1])
def test_block_step_chain(ci):
    """inject(n_ctx) -> conv -> attention -> top-K -> selector -> accept on the
    GPU.  Each stage is checked against the oracle fed the GPU's previous
    outputs (the cache rows, u, h, idx / unary, path); the block output h is
    also checked against the oracle's own chain."""
    cfg = configs.get(ci)
    say(f"chain {cfg.name}")
    w = synth.Workload(cfg)
    W = P.DeviceWeights(w, drop_host=False)
    cache = P.new_cache(cfg)
    step = P.BlockStep(cfg, W, cache, inject_n=cfg.n_ctx)
    hid = [w.hidden(l) for l in range(cfg.L_t)]
    x = w.x()
    anchor = int(w.anchor()[0])
    bp = cfg.act == "bf16"
    a = lambda t: act_np(t, cfg.act)
    A, Bc = w.codebooks()
    # the oracle's own chain, for the end-to-end check of h
    inj = O.inject([a(h) for h in hid], wnp(w.fc()), None, cfg.eps, wnp(w.wk()), wnp(w.wv()), bp)
    ck = np.zeros((cfg.Hkv, cfg.cap, cfg.hd))
    cv = np.zeros_like(ck)
    O.cache_write(ck, cv, inj["k"], inj["v"], 0)
    ref = O.block_step(a(x)[0], a(w.conv_base()), wnp(w.w_delta()), cfg.G, wnp(w.wq()), wnp(w.wk()),
                       wnp(w.wv()), wnp(w.wo()), ck, cv, cfg.n_ctx, cfg.Hq, O.weight_to_f64(w.w_lm()),
                       cfg.K, wnp(w.sel_proj()), a(A), a(Bc), anchor, bp)
    tgt, m = synth.targets_with_mismatch(cfg.seed, "chain.tgt", ref["path"][None, :], cfg.V)
    step.run(dev(x, cfg.act), cfg.n_ctx, anchor, torch.from_numpy(tgt).cuda(),
             hidden=[dev(h, cfg.act) for h in hid], pos0=0)
    torch.cuda.synchronize()
    # stage by stage on the GPU's own intermediates
    gk, gv = rows_of_cache(cache, np.arange(cfg.n_ctx))
    assert_close(gk, inj["k"], cfg.act, f"{cfg.name} chain cache K")
    assert_close(gv, inj["v"], cfg.act, f"{cfg.name} chain cache V")
    CK = np.zeros((cfg.Hkv, cfg.cap, cfg.hd))
    CV = np.zeros_like(CK)
    O.cache_write(CK, CV, gk, gv, 0)
    c = O.conv(a(x), a(w.conv_base()), wnp(w.w_delta()), cfg.G, bp)
    ug = f64(step.u)
    assert_close(ug, c["u"], cfg.act, f"{cfg.name} chain u")
    gh = f64(step.h)
    at = O.block_attn(ug[0], a(x)[0], wnp(w.wq()), wnp(w.wk()), wnp(w.wv()), wnp(w.wo()), CK, CV, cfg.n_ctx,
                      cfg.Hq, 0.0, bp)
    assert_close(gh, at["out"], cfg.act, f"{cfg.name} chain h from the GPU's u and cache")
    logits = O.lm_logits_stored(gh, w.w_lm())
    gi, gu = step.idx.cpu().numpy(), step.unary.cpu().numpy()
    check_topk(gi, gu, logits, cfg.K, cfg.act, f"{cfg.name} chain top-K from the GPU's h")
    sel = O.selector(gh, wnp(w.sel_proj()), a(A), a(Bc), gi, gu.astype(np.float64), anchor)
    gp = step.path.cpu().numpy()[0]
    check_selector(sel, step.edges.cpu().numpy().astype(np.float64), gp, gi, f"{cfg.name} chain selector")
    # the accept length the selector's kernel formed against the targets
    assert int(step.accept.cpu()[0]) == int(O.accept_len(gp[None, :], tgt)[0])
    # end to end: the GPU's h against the oracle's own chain
    assert_close(gh, ref["attn"]["out"], cfg.act, f"{cfg.name} chain h end to end")


@pytest.mark.parametrize("ci", [1, 4])
def test_block_step_overlap_matches_serial(ci):
    """run() with the injection on its own stream (the attention waits for
    it before reading the cache) against the same steps in one stream: the
    cache, u, h, top-K, edges, path and accept length bit for bit, over three
    steps whose injected rows are the newest keys attended.  Before each
    injection its rows hold a constant, so an attention that read them early
    would differ."""
    cfg = configs.get(ci)
    say(f"overlap {cfg.name}")
    w = synth.Workload(cfg)
    W = P.DeviceWeights(w, drop_host=True)
    n, n0 = 16, 256
    anchor = int(w.anchor()[0])
    runs = []
    for overlap in (False, True):
        cache = P.new_cache(configs.shrink(cfg, capacity=n0 + 3 * n))
        cache.k[:, :n0].normal_(generator=torch.Generator(device="cuda").manual_seed(5))
        cache.v[:, :n0 // 32].normal_(generator=torch.Generator(device="cuda").manual_seed(6))
        step = P.BlockStep(cfg, W, cache, inject_n=n)
        outs = []
        for s in range(3):
            pos0 = n0 + n * s
            cache.k[:, pos0:pos0 + n].fill_(3.0)
            hid = [dev(synth.normal(cfg.seed, f"ovl.h{s}.{l}", (n, cfg.d_t), 1.0, cfg.act), cfg.act)
                   for l in range(cfg.L_t)]
            x = dev(synth.normal(cfg.seed, f"ovl.x{s}", (1, cfg.B, cfg.d), 1.0, cfg.act), cfg.act)
            tgt = torch.zeros((1, cfg.B), dtype=torch.int32, device="cuda")
            step.run(x, pos0 + n, anchor, tgt, hidden=hid, pos0=pos0, overlap=overlap)
            torch.cuda.synchronize()
            outs.append([t.clone() for t in (step.u, step.h, step.idx, step.unary, step.edges, step.path,
                                             step.accept)])
        outs.append([cache.k.clone(), cache.v.clone()])
        runs.append(outs)
    for s, (a, b) in enumerate(zip(*runs)):
        for x, y in zip(a, b):
            assert torch.equal(x, y), f"{cfg.name} step {s}: the overlapped step differs from the serial one"


@pytest.mark.parametrize("kv", ["bf16", "q8_0"])
def test_decode_64k_three_steps(kv):
    """The 64k decode workload as a sequence: the cache holds 65536 seeded
    rows; step s injects 16 rows at 65536 + 16 s (half a V panel each, so the
    steps alternate between starting a panel and finishing it) and then
    attends 65536 + 16 (s + 1) context keys plus the block.  Each step's rows
    and output are checked; the oracle's cache takes the GPU's injected rows
    once they have passed.  kv = q8_0: the same with a Q8_0 cache (seeded rows
    quantised by the oracle, injected rows quantised by the library)."""
    cfg = configs.get(3)
    w = synth.Workload(cfg)
    n0, n = cfg.prefill_kv, cfg.inject_per_step
    shp = (cfg.Hkv, n0, cfg.hd)
    CK = np.zeros((cfg.Hkv, cfg.cap, cfg.hd))
    CV = np.zeros_like(CK)
    if kv == "q8_0":
        cache = P.new_cache(cfg, kv="q8_0")
        kr = synth.normal(cfg.seed, "seqq.ck", shp, 1.0, "f32").astype(np.float64)
        vr = synth.normal(cfg.seed, "seqq.cv", shp, 1.0, "f32").astype(np.float64)
        CK[:, :n0], CV[:, :n0] = q8_fill(cache, kr, vr)
        del kr, vr
    else:
        ck0 = synth.normal(cfg.seed, "seq.ck", shp, 1.0, cfg.act)
        cv0 = synth.normal(cfg.seed, "seq.cv", shp, 1.0, cfg.act)
        cache = P.new_cache(cfg)
        cache.k[:, :n0] = dev(ck0, cfg.act)
        cache.v[:, :n0 // 32] = D.v_panels(dev(cv0, cfg.act))
        CK[:, :n0] = act_np(ck0, cfg.act)
        CV[:, :n0] = act_np(cv0, cfg.act)
        del ck0, cv0
    wq, wk, wv, wo = w.wq(), w.wk(), w.wv(), w.wo()
    dt = P.act_dtype(cfg.act)
    for s in range(3):
        pos0 = n0 + n * s
        hid = [synth.normal(cfg.seed, f"seq.h{s}.{l}", (n, cfg.d_t), 1.0, cfg.act) for l in range(cfg.L_t)]
        if kv == "q8_0":
            _, kvals, vvals = run_inject_q8(cfg, n, pos0, cache=cache, hid=hid)
            CK[:, pos0:pos0 + n], CV[:, pos0:pos0 + n] = kvals, vvals
        else:
            _, gk, gv = run_inject(cfg, n, pos0, cache=cache, hid=hid)
            O.cache_write(CK, CV, gk, gv, pos0)
        n_ctx = pos0 + n
        u = synth.normal(cfg.seed, f"seq.u{s}", (cfg.B, cfg.d), 1.0, cfg.act)
        x = synth.normal(cfg.seed, f"seq.x{s}", (cfg.B, cfg.d), 1.0, cfg.act)
        out = torch.empty((cfg.B, cfg.d), dtype=dt, device="cuda")
        args = (cfg.B, cfg.d, cfg.Hq, cfg.Hkv, cfg.hd, n_ctx)
        ws = D.workspace(D.dflash_block_attn_workspace(*args))
        say(f"attn step {s}: n_ctx={n_ctx} ({kv} cache)")
        D.dflash_block_attn(dev(u, cfg.act), dev(x, cfg.act), cfg.Hq, wdev(wq), wdev(wk), wdev(wv), wdev(wo),
                            cache, n_ctx, 0.0, out, ws)
        torch.cuda.synchronize()
        qd, kvd = cfg.Hq * cfg.hd, cfg.Hkv * cfg.hd
        qkvg = f64(D.ws_view(ws, D.dflash_block_attn_qkv_offset(*args), (cfg.B, qd + 2 * kvd), dt))
        og = f64(D.ws_view(ws, D.dflash_block_attn_o_offset(*args), (cfg.B, qd), dt))
        check_attn(cfg, act_np(u, cfg.act), act_np(x, cfg.act), wq, wk, wv, wo, CK, CV, n_ctx, 0.0, qkvg, og,
                   f64(out), f"64k step {s} attn (n_ctx={n_ctx}, {kv} cache)", cfg.B)
