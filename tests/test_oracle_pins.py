"""Pins of the CPU oracle against facts that do not come from the oracle itself:
closed forms, special cases that reduce to a library routine, invariants,
brute force on tiny inputs and the figures the pages print.

Each test states which plausible mistake it would catch.
"""
import itertools
import json
import os
import time

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O
from block_diffusion_drafter_step_amd import configs, synth, workmodel

GOLD = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


def randn(*shape, scale=1.0):
    return rng.standard_normal(shape) * scale


# --------------------------------------------------------------------------
# storage decoding
# --------------------------------------------------------------------------

def test_round_bf16_matches_torch():
    """The oracle's bf16 rounding equals torch's fp32 -> bf16 cast (RNE);
    catches truncation instead of rounding and wrong tie handling."""
    x = np.concatenate([randn(10000, scale=3.0), randn(1000, scale=1e-3), randn(1000, scale=1e4)])
    ref = torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_bf16(x), ref)
    # exact ties: 1 + 2^-8 -> 1 (even), 1 + 3*2^-8 -> 1 + 2^-6 (even)
    assert O.round_bf16(np.array([1 + 2 ** -8]))[0] == 1.0
    assert O.round_bf16(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6


def test_bf16_decode_matches_torch():
    bits = rng.integers(0, 1 << 16, size=5000).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]            # finite only
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.bf16_to_f64(bits), ref)


def test_q8_0_decode_matches_torch_and_scale_one():
    """value = bf16(fp32(scale) * q): torch computes the same product in fp32
    and casts; scale = 1 leaves the int8 codes exact.  Catches a dropped scale,
    a scale applied to the wrong block, or a missing rounding point."""
    q, s = synth.q8_0(7, "w", 6, 96)
    ref = (torch.from_numpy(q.astype(np.float32)).view(6, 3, 32)
           * torch.from_numpy(s).to(torch.float32)[:, :, None]).to(torch.bfloat16)
    np.testing.assert_array_equal(O.q8_0_to_f64(q, s), ref.reshape(6, 96).double().numpy())
    ones = np.ones_like(s)
    np.testing.assert_array_equal(O.q8_0_to_f64(q, ones), q.astype(np.float64))


def test_q8_0_int8_matmul_and_scale_doubling():
    """Scale 1 with small-integer activations equals an integer matmul exactly;
    doubling every scale doubles the output exactly."""
    q, s = synth.q8_0(3, "w", 16, 64)
    xi = rng.integers(-3, 4, size=(5, 64))
    w1 = O.q8_0_to_f64(q, np.ones_like(s))
    np.testing.assert_array_equal(xi @ w1.T, (xi.astype(np.int64) @ q.astype(np.int64).T).astype(np.float64))
    x = randn(5, 64)
    y1 = x @ O.q8_0_to_f64(q, s).T
    y2 = x @ O.q8_0_to_f64(q, (s.astype(np.float32) * 2).astype(np.float16)).T
    np.testing.assert_array_equal(y2, 2 * y1)


# --------------------------------------------------------------------------
# (1) injection
# --------------------------------------------------------------------------

def test_rmsnorm_unit_rms_closed_form():
    """With gamma = 1, rms(z) = sqrt(m / (m + eps)) where m = mean(y^2)."""
    y = randn(7, 300, scale=5.0)
    eps = 1e-6
    z = O.rmsnorm(y, None, eps)
    m = np.mean(y * y, axis=1)
    np.testing.assert_allclose(np.sqrt(np.mean(z * z, axis=1)), np.sqrt(m / (m + eps)), rtol=1e-14)


def test_rmsnorm_matches_torch():
    y = randn(9, 128)
    g = randn(128)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(y), (128,), torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(O.rmsnorm(y, g, 1e-6), ref, rtol=1e-12, atol=1e-12)


def test_rmsnorm_scale_invariant():
    y = randn(4, 64)
    np.testing.assert_allclose(O.rmsnorm(3.7 * y, None, 0.0), O.rmsnorm(y, None, 0.0), rtol=1e-13)


def test_inject_layer_order_and_identity():
    """Permuting the target layers together with fc's column blocks leaves y
    unchanged (catches concatenation along the wrong axis); a single layer with
    fc = I gives y = h."""
    n, dt, d, L = 5, 16, 8, 3
    hs = [randn(n, dt) for _ in range(L)]
    fc = randn(d, L * dt)
    wk, wv = randn(4, d), randn(4, d)
    r = O.inject(hs, fc, None, 1e-6, wk, wv, False)
    perm = [2, 0, 1]
    fcp = np.concatenate([fc[:, p * dt:(p + 1) * dt] for p in perm], axis=1)
    rp = O.inject([hs[p] for p in perm], fcp, None, 1e-6, wk, wv, False)
    np.testing.assert_allclose(rp["y"], r["y"], rtol=1e-12, atol=1e-12)
    r1 = O.inject([hs[0]], np.eye(dt), None, 1e-6, randn(4, dt), randn(4, dt), False)
    np.testing.assert_array_equal(r1["y"], hs[0])


def test_inject_chain_and_cache_write():
    """K = RMSNorm(h fc^T) Wk^T lands at cache[head][pos0 + t][dim]; rows
    outside [pos0, pos0 + n) are untouched."""
    n, dt, d, L, hkv, hd, cap = 3, 8, 8, 2, 2, 4, 10
    hs = [randn(n, dt) for _ in range(L)]
    fc, wk, wv = randn(d, L * dt), randn(hkv * hd, d), randn(hkv * hd, d)
    r = O.inject(hs, fc, None, 1e-6, wk, wv, False)
    y = np.hstack(hs) @ fc.T
    z = y / np.sqrt((y ** 2).mean(1, keepdims=True) + 1e-6)
    np.testing.assert_allclose(r["k"], z @ wk.T, rtol=1e-12)
    ck, cv = np.full((hkv, cap, hd), 7.0), np.full((hkv, cap, hd), 7.0)
    O.cache_write(ck, cv, r["k"], r["v"], 4)
    assert np.all(ck[:, :4] == 7.0) and np.all(ck[:, 7:] == 7.0)
    for t in range(n):
        for h in range(hkv):
            np.testing.assert_array_equal(ck[h, 4 + t], r["k"][t, h * hd:(h + 1) * hd])
    with pytest.raises(ValueError):
        O.cache_write(ck, cv, r["k"], r["v"], 8)


def test_encoder_flops_golden():
    """The work model reproduces the pages' ~69 GFLOP for the fc of a 512-token
    batch (32768 -> 2048)."""
    g = json.load(open(os.path.join(GOLD, "encoder_flops.json")))
    f = workmodel.fc_flops(g["tokens"], g["fc_in"], g["fc_out"]) / 1e9
    assert abs(f - g["gflop_quoted"]) <= g["quoted_precision"]
    # the full injection adds the two K/V projections on top of the fc term
    assert workmodel.inject_flops(512, 8, 4096, 2048, 0) == workmodel.fc_flops(512, 32768, 2048)


# --------------------------------------------------------------------------
# (2) conv
# --------------------------------------------------------------------------

def test_conv_static_equals_numpy_convolve():
    """W_delta = 0: a causal depthwise FIR per channel = numpy.convolve[:B]."""
    nb, B, C, G, T = 2, 8, 12, 3, 4
    x = randn(nb, B, C)
    base = randn(T, C)
    out = O.conv(x, base, np.zeros((T * G, C)), G, False)["u"]
    for b in range(nb):
        for c in range(C):
            np.testing.assert_allclose(out[b, :, c], np.convolve(x[b, :, c], base[:, c])[:B], rtol=1e-12, atol=1e-12)


def test_conv_single_tap_identity_and_causality():
    nb, B, C, G, T = 1, 6, 8, 2, 3
    x = randn(nb, B, C)
    base = np.zeros((T, C))
    base[0] = 1.0
    np.testing.assert_array_equal(O.conv(x, base, np.zeros((T * G, C)), G, False)["u"], x)
    # out[0] depends on x[0] only (zero padding before the block start)
    base = randn(T, C)
    wd = randn(T * G, C)
    x2 = x.copy()
    x2[:, 1:] = randn(nb, B - 1, C)
    a = O.conv(x, base, wd, G, False)["u"]
    b = O.conv(x2, base, wd, G, False)["u"]
    np.testing.assert_array_equal(a[:, 0], b[:, 0])


def test_conv_dynamic_tap_special_cases():
    """base = 0 and one tap: with G = C, out[i,c] = (x[i] . W_delta[c]) * x[i,c];
    with T = 2 and only tap-1 rows, out[i,c] = (x[i] . W_delta[G + c]) * x[i-1,c]
    (delta comes from the current position, index t*G + g)."""
    B, C = 5, 6
    x = randn(1, B, C)
    wd = randn(C, C)
    out = O.conv(x, np.zeros((1, C)), wd, C, False)["u"][0]
    np.testing.assert_allclose(out, (x[0] @ wd.T) * x[0], rtol=1e-12)
    wd2 = np.concatenate([np.zeros((C, C)), wd])
    out2 = O.conv(x, np.zeros((2, C)), wd2, C, False)["u"][0]
    ref2 = np.zeros((B, C))
    ref2[1:] = (x[0, 1:] @ wd.T) * x[0, :-1]
    np.testing.assert_allclose(out2, ref2, rtol=1e-12, atol=1e-14)


def test_conv_group_sharing():
    """G = 1: one delta for every channel, so with base = 0 and T = 1 the output
    is x scaled per position; equal x and base inside a group -> equal outputs."""
    B, C = 4, 10
    x = randn(1, B, C)
    wd = randn(1, C)
    out = O.conv(x, np.zeros((1, C)), wd, 1, False)["u"][0]
    np.testing.assert_allclose(out, (x[0] @ wd[0])[:, None] * x[0], rtol=1e-12)
    G, T = 2, 3
    x = randn(1, B, C)
    x[0, :, 1] = x[0, :, 0]                   # channels 0 and 1 share group 0
    base = randn(T, C)
    base[:, 1] = base[:, 0]
    u = O.conv(x, base, randn(T * G, C), G, False)["u"][0]
    np.testing.assert_array_equal(u[:, 0], u[:, 1])
    x[0, :, 6] = x[0, :, 0]                   # channel 6 is in group 1: differs
    base[:, 6] = base[:, 0]
    u = O.conv(x, base, randn(T * G, C), G, False)["u"][0]
    assert not np.allclose(u[:, 0], u[:, 6])


# --------------------------------------------------------------------------
# (3) attention
# --------------------------------------------------------------------------

def _attn_case(B=4, d=32, Hq=4, Hkv=2, hd=8, n_ctx=11, cap=16):
    return dict(u=randn(B, d), resid=randn(B, d), wq=randn(Hq * hd, d), wk=randn(Hkv * hd, d),
                wv=randn(Hkv * hd, d), wo=randn(d, Hq * hd), ck=randn(Hkv, cap, hd),
                cv=randn(Hkv, cap, hd), n_ctx=n_ctx, Hq=Hq)


def _run_attn(c, **over):
    c = dict(c, **over)
    return O.block_attn(c["u"], c["resid"], c["wq"], c["wk"], c["wv"], c["wo"], c["ck"], c["cv"],
                        c["n_ctx"], c["Hq"], 0.0, False)


def test_attention_identical_keys_give_mean_v():
    c = _attn_case()
    r = _run_attn(c, wk=np.zeros_like(c["wk"]), ck=np.zeros_like(c["ck"]))
    hd, n = 8, c["n_ctx"]
    for h in range(4):
        g = h // 2
        vals = np.concatenate([c["cv"][g, :n], r["vb"][:, g * hd:(g + 1) * hd]])
        np.testing.assert_allclose(r["o"][:, h * hd:(h + 1) * hd], np.tile(vals.mean(0), (4, 1)), rtol=1e-12)
    q0 = _run_attn(c, wq=np.zeros_like(c["wq"]))
    g = 0
    vals = np.concatenate([c["cv"][g, :n], q0["vb"][:, :hd]])
    np.testing.assert_allclose(q0["o"][:, :hd], np.tile(vals.mean(0), (4, 1)), rtol=1e-12)


def test_attention_single_key_returns_v():
    q = randn(3, 8)
    k, v = randn(1, 8), randn(1, 8)
    np.testing.assert_allclose(O.softmax_attend(q, k, v, 0.3)[0], np.tile(v, (3, 1)), rtol=1e-14)


def test_attention_matches_torch_sdpa_mha():
    """GQA with KV heads repeated to Hq equals torch's non-causal SDPA in fp64."""
    c = _attn_case()
    r = _run_attn(c)
    B, Hq, Hkv, hd, n = 4, 4, 2, 8, c["n_ctx"]
    q = torch.from_numpy(r["q"].reshape(B, Hq, hd)).permute(1, 0, 2)
    kb = r["kb"].reshape(B, Hkv, hd)
    vb = r["vb"].reshape(B, Hkv, hd)
    ks = torch.stack([torch.from_numpy(np.concatenate([c["ck"][h // 2, :n], kb[:, h // 2]])) for h in range(Hq)])
    vs = torch.stack([torch.from_numpy(np.concatenate([c["cv"][h // 2, :n], vb[:, h // 2]])) for h in range(Hq)])
    ref = torch.nn.functional.scaled_dot_product_attention(q, ks, vs, is_causal=False)
    ref = ref.permute(1, 0, 2).reshape(B, Hq * hd).numpy()
    np.testing.assert_allclose(r["o"], ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(r["out"], c["resid"] + ref @ c["wo"].T, rtol=1e-10, atol=1e-10)


def test_attention_context_permutation_invariant():
    c = _attn_case()
    r = _run_attn(c)
    perm = rng.permutation(c["n_ctx"])
    ck, cv = c["ck"].copy(), c["cv"].copy()
    ck[:, :c["n_ctx"]] = ck[:, perm]
    cv[:, :c["n_ctx"]] = cv[:, perm]
    rp = _run_attn(c, ck=ck, cv=cv)
    np.testing.assert_allclose(rp["out"], r["out"], rtol=1e-11, atol=1e-11)


def test_attention_ignores_rows_past_n_ctx():
    c = _attn_case()
    r = _run_attn(c)
    ck = c["ck"].copy()
    ck[:, c["n_ctx"]:] = 1e6
    np.testing.assert_array_equal(_run_attn(c, ck=ck)["out"], r["out"])


def test_attention_weight_rounding_bound_holds_and_is_needed():
    """The bound for softmax weights rounded to bf16 before they multiply V
    (the GPU's P.V operands): brute force emulates every way of rounding each
    weight up or down by at most one unit roundoff and never leaves the bound,
    and a single adversarial rounding comes within a few percent of it, so the
    bound is neither wrong nor vacuous.  Catches a dropped |V - out| (the
    bound would then not shrink for equal values) or a wrong roundoff."""
    q, keys, vals = randn(2, 8), randn(40, 8), randn(40, 8) * 3.0
    out, bound = O.softmax_attend(q, keys, vals, 0.4, O.U_BF16)
    assert np.all(bound > 0)
    s = (q @ keys.T) * 0.4
    w = np.exp(s - s.max(1, keepdims=True))
    w /= w.sum(1, keepdims=True)
    u = O.U_BF16
    for trial in range(200):
        e = rng.uniform(-u, u, size=w.shape)
        e[:, :trial % 3] = u                           # some weights at the extreme
        we = w * (1 + e)
        o2 = (we @ vals) / we.sum(1, keepdims=True)
        assert np.all(np.abs(o2 - out) <= bound * (1 + 1e-12))
    # the worst case for element (0, j): weights of values above out[0, j]
    # rounded up, below it rounded down
    j = 3
    e = np.where(vals[:, j] > out[0, j], u, -u)
    we = w[0] * (1 + e)
    o2 = (we @ vals[:, j]) / we.sum()
    assert abs(o2 - out[0, j]) >= 0.95 * bound[0, j]
    # equal values: rounding the weights cannot move the output
    _, b0 = O.softmax_attend(q, keys, np.ones((40, 8)), 0.4, O.U_BF16)
    np.testing.assert_allclose(b0, 0.0, atol=1e-15)
    _, bz = O.softmax_attend(q, keys, vals, 0.4)
    assert np.all(bz == 0)
    # bf16's unit roundoff: 8 significant bits, |bf16(x) - x| <= 2^-8 |x|
    xs = rng.uniform(0.5, 4.0, 20000)
    assert np.max(np.abs(O.round_bf16(xs) - xs) / xs) <= O.U_BF16
    assert np.max(np.abs(O.round_bf16(xs) - xs) / xs) > 0.9 * O.U_BF16


def test_attention_stages_compose():
    """attn_qkv -> attn_core -> attn_out is block_attn, and attn_core fed the
    projections reproduces the same O (the stage-fed GPU checks rely on it)."""
    c = _attn_case()
    r = _run_attn(c)
    p = O.attn_qkv(c["u"], c["wq"], c["wk"], c["wv"], False)
    co = O.attn_core(p["q"], p["kb"], p["vb"], c["ck"], c["cv"], c["n_ctx"], c["Hq"], 0.0, False)
    np.testing.assert_array_equal(co["o"], r["o"])
    np.testing.assert_array_equal(O.attn_out(co["o"], c["wo"], c["resid"], False), r["out"])


# --------------------------------------------------------------------------
# Q8_0 KV cache rows (quantisation, and the values attention reads)
# --------------------------------------------------------------------------

def test_kv_q8_0_exact_blocks_round_trip():
    """Blocks that are exactly a power-of-two scale times integers with one
    +-127 per block come back unchanged: codes, scale and values (bf16 and
    fp32).  Catches a 128 divisor, a scale over the wrong axis or a dropped
    scale."""
    r = np.random.default_rng(7)
    q = r.integers(-126, 127, size=(3, 4, 128))
    q[..., ::32] = 127 * np.where(r.random((3, 4, 4)) < 0.5, -1, 1)   # one +-127 per block
    x = q * 2.0 ** -6
    codes, scales = O.kv_quant_q8_0(x)
    assert np.array_equal(codes.astype(np.int64), q)
    assert np.all(scales.astype(np.float64) == 2.0 ** -6)
    assert np.array_equal(O.kv_dequant_q8_0(codes, scales, True), x)
    assert np.array_equal(O.kv_dequant_q8_0(codes, scales, False), x)


def test_kv_q8_0_ties_away_from_zero():
    """x / scale = k + 1/2 rounds away from zero (numpy's round-half-even would
    give 2, 0, 2 for 2.5, 0.5, 1.5).  Catches banker's rounding and
    truncation."""
    x = np.zeros(32)
    x[0] = 127.0
    x[1:7] = [2.5, -2.5, 0.5, -0.5, 1.5, -1.5]
    codes, scales = O.kv_quant_q8_0(x * 2.0 ** -4)
    assert float(scales[0]) == 2.0 ** -4
    assert list(codes[:7]) == [127, 3, -3, 1, -1, 2, -2]


def test_kv_q8_0_zero_block_sign_symmetry_and_block_order():
    """An all-zero block gives scale 0 and codes 0 (no NaN); negating x negates
    the codes and keeps the scales; block b's scale multiplies dims 32b ..
    32b+31 (catches a transposed scale index)."""
    r = np.random.default_rng(8)
    x = r.standard_normal((5, 128))
    x[2, 32:64] = 0.0
    c, s = O.kv_quant_q8_0(x)
    assert float(s[2, 1]) == 0.0 and not np.any(c[2, 32:64])
    assert np.all(np.isfinite(O.kv_dequant_q8_0(c, s, False)))
    cn, sn = O.kv_quant_q8_0(-x)
    assert np.array_equal(cn, -c) and np.array_equal(sn, s)
    ones = np.ones((1, 128), dtype=np.int8)
    sc = np.array([[1.0, 2.0, 4.0, 8.0]], dtype=np.float16)
    assert np.array_equal(O.kv_dequant_q8_0(ones, sc, True)[0], np.repeat([1.0, 2.0, 4.0, 8.0], 32))


def test_kv_q8_0_codes_are_the_nearest_level_by_brute_force():
    """On random blocks each code is the integer level in [-127, 127] nearest
    to x at the block's unrounded scale max|x|/127 (brute force over all 255
    levels), the largest |x| of a block takes +-127, and the value read back
    is within half a level plus the fp16 rounding of the scale."""
    r = np.random.default_rng(9)
    x = r.standard_normal((6, 64)) * r.uniform(0.01, 10.0, size=(6, 1))
    c, s = O.kv_quant_q8_0(x)
    blocks = x.reshape(6, 2, 32)
    exact = np.max(np.abs(blocks), axis=-1) / 127.0
    levels = np.arange(-127, 128)
    for i in range(6):
        for b in range(2):
            for e in range(32):
                v = blocks[i, b, e]
                dist = np.abs(v - exact[i, b] * levels)
                best = levels[np.argmin(dist)]
                assert c[i, 32 * b + e] == best, (i, b, e)
            assert np.max(np.abs(c[i, 32 * b:32 * b + 32])) == 127
    back = O.kv_dequant_q8_0(c, s, False).reshape(6, 2, 32)
    s16 = s.astype(np.float64)
    bound = exact / 2 + np.abs(s16 - exact) * 127 + 1e-12
    assert np.all(np.abs(back - blocks) <= bound[..., None])


# --------------------------------------------------------------------------
# (4) LM head
# --------------------------------------------------------------------------

def test_topk_zero_hidden():
    """h = 0: all logits equal, so idx = 0..K-1 (tie -> lower index) and
    unary = -ln V."""
    V, d, K = 50, 16, 5
    r = O.topk_unary(np.zeros((3, d)), randn(V, d), K)
    np.testing.assert_array_equal(r["idx"], np.tile(np.arange(K), (3, 1)))
    np.testing.assert_allclose(r["unary"], -np.log(V), rtol=1e-14)


def test_topk_matches_stable_argsort_and_lse():
    V, K = 300, 7
    logits = np.round(randn(6, V, scale=2.0), 1)        # rounding creates ties
    r = O.topk_unary_from_logits(logits, K)
    ref = np.argsort(-logits, axis=1, kind="stable")[:, :K]
    np.testing.assert_array_equal(r["idx"], ref)
    np.testing.assert_allclose(r["lse"], scipy.special.logsumexp(logits, axis=1), rtol=1e-14)
    u = r["unary"]
    assert np.all(np.diff(u, axis=1) <= 0)
    assert np.all(np.exp(u).sum(1) <= 1 + 1e-12)
    full = O.topk_unary_from_logits(logits, V)
    np.testing.assert_allclose(np.exp(full["unary"]).sum(1), 1.0, rtol=1e-12)


def test_topk_gap_values():
    logits = np.array([[5.0, 1.0, 4.0, 4.0005, 0.0]])
    g = O.topk_gaps(logits, 2)
    np.testing.assert_allclose(g["kth_gap"], [4.0005 - 4.0])
    np.testing.assert_allclose(g["adj_gap"], [[5.0 - 4.0005]])


# --------------------------------------------------------------------------
# (5) selector
# --------------------------------------------------------------------------

def _sel_case(B=5, K=3, V=40, r=6, d=12):
    idx = np.stack([rng.choice(V, K, replace=False) for _ in range(B)])
    unary = -np.abs(randn(B, K))
    return dict(h=randn(B, d), P=randn(r, d), A=randn(V, r), Bc=randn(V, r), idx=idx, unary=unary)


def test_selector_all_ones_codebooks():
    """A = B = 1: edge = sum(project(h)) + unary (for every predecessor)."""
    c = _sel_case()
    V, r = c["A"].shape
    e = O.selector_edges(c["h"], c["P"], np.ones((V, r)), np.ones((V, r)), c["idx"], c["unary"], 3)["edges"]
    proj = c["h"] @ c["P"].T
    ref = proj.sum(1)[:, None, None] + c["unary"][:, None, :]
    np.testing.assert_allclose(e[1:], np.broadcast_to(ref[1:], e[1:].shape), rtol=1e-12)
    np.testing.assert_allclose(e[0, 0], ref[0, 0], rtol=1e-12)
    assert np.all(np.isneginf(e[0, 1:]))


def test_selector_zero_predecessor_codebook_gives_top1_path():
    """A = 0: edge = unary, so the best path takes each position's best unary."""
    c = _sel_case()
    r = O.selector(c["h"], c["P"], np.zeros_like(c["A"]), c["Bc"], c["idx"], c["unary"], 2)
    best = np.argmax(c["unary"], axis=1)
    np.testing.assert_array_equal(r["path"], c["idx"][np.arange(5), best])


def test_selector_anchor_none_row0_is_unary():
    c = _sel_case()
    e = O.selector_edges(c["h"], c["P"], c["A"], c["Bc"], c["idx"], c["unary"], -1)["edges"]
    np.testing.assert_array_equal(e[0, 0], c["unary"][0])


def test_selector_edge_triple_product_elementwise():
    """One edge against the triple-product sum written over the rank index."""
    c = _sel_case()
    e = O.selector_edges(c["h"], c["P"], c["A"], c["Bc"], c["idx"], c["unary"], 7)["edges"]
    proj = c["h"] @ c["P"].T
    i, a, b = 3, 2, 1
    p, cc = c["idx"][i - 1, a], c["idx"][i, b]
    tp = sum(c["A"][p, k] * proj[i, k] * c["Bc"][cc, k] for k in range(proj.shape[1]))
    assert abs(e[i, a, b] - (tp + c["unary"][i, b])) < 1e-12
    p0 = sum(c["A"][7, k] * proj[0, k] * c["Bc"][c["idx"][0, b], k] for k in range(proj.shape[1]))
    assert abs(e[0, 0, b] - (p0 + c["unary"][0, b])) < 1e-12


@pytest.mark.parametrize("K,B", [(4, 8), (3, 6), (2, 1), (5, 2)])
def test_viterbi_matches_brute_force(K, B):
    """Best and runner-up path scores over all K^B paths (config 0: 4^8)."""
    e = np.round(randn(B, K, K), 2)
    e[0, 1:] = -np.inf
    v = O.viterbi(e)
    scores = []
    for slots in itertools.product(range(K), repeat=B):
        scores.append((O.path_score(e, slots), slots))
    scores.sort(key=lambda t: -t[0])
    assert abs(v["score"] - scores[0][0]) < 1e-12
    assert abs(O.path_score(e, v["slots"]) - scores[0][0]) < 1e-12
    finite = [s for s in scores if np.isfinite(s[0])]
    runner = finite[1][0] if len(finite) > 1 else -np.inf
    assert v["runner_up"] == pytest.approx(runner, abs=1e-12) if np.isfinite(runner) else np.isneginf(v["runner_up"])
    if scores[0][0] - runner > 1e-9:
        assert tuple(v["slots"]) == scores[0][1]


def test_viterbi_tie_goes_to_lower_slot():
    e = np.zeros((3, 2, 2))
    e[0, 1] = -np.inf
    v = O.viterbi(e)
    np.testing.assert_array_equal(v["slots"], [0, 0, 0])
    assert v["runner_up"] == v["score"]


def test_selector_param_counts_golden():
    g = json.load(open(os.path.join(GOLD, "selector_params.json")))
    for c in g["cases"]:
        if c["kind"] == "materialised":
            n = workmodel.selector_params(c["V"], c["r"])
        else:
            n = workmodel.selector_params_factorised(c["d"], c["r"])
        assert abs(n / 1e6 - c["quoted_millions"]) <= c["quoted_precision"], c


# --------------------------------------------------------------------------
# (6) accept length
# --------------------------------------------------------------------------

def test_accept_len_known_mismatch():
    path = rng.integers(0, 100, size=(64, 8)).astype(np.int32)
    tgt, m = synth.targets_with_mismatch(5, "tgt", path, 100)
    np.testing.assert_array_equal(O.accept_len(path, tgt), m)
    assert set(np.unique(m)) <= set(range(9))
    np.testing.assert_array_equal(O.accept_len(path, path), np.full(64, 8))


# --------------------------------------------------------------------------
# whole tiny step
# --------------------------------------------------------------------------

def test_tiny_config_step_runs_fast():
    cfg = configs.get(0)
    w = synth.Workload(cfg)
    t0 = time.time()
    f = lambda wt: O.weight_to_f64(wt)
    a = lambda x: O.act_to_f64(x, cfg.act)
    inj = O.inject([a(w.hidden(l)) for l in range(cfg.L_t)], f(w.fc()), None, cfg.eps, f(w.wk()), f(w.wv()), False)
    ck = np.zeros((cfg.Hkv, cfg.cap, cfg.hd))
    cv = np.zeros_like(ck)
    O.cache_write(ck, cv, inj["k"], inj["v"], 0)
    A, Bc = w.codebooks()
    r = O.block_step(a(w.x())[0], a(w.conv_base()), f(w.w_delta()), cfg.G, f(w.wq()), f(w.wk()),
                     f(w.wv()), f(w.wo()), ck, cv, cfg.n_ctx, cfg.Hq, f(w.w_lm()), cfg.K,
                     f(w.sel_proj()), a(A), a(Bc), int(w.anchor()[0]), False)
    assert time.time() - t0 < 1.0
    assert r["path"].shape == (cfg.B,)
    assert np.all(np.isfinite(r["attn"]["out"]))
    assert np.all((r["path"] >= 0) & (r["path"] < cfg.V))


def _step_inputs(cfg):
    w = synth.Workload(cfg)
    f = lambda wt: O.weight_to_f64(wt)
    a = lambda x: O.act_to_f64(x, cfg.act)
    inj = O.inject([a(w.hidden(l)) for l in range(cfg.L_t)], f(w.fc()), None, cfg.eps, f(w.wk()), f(w.wv()), False)
    ck = np.zeros((cfg.Hkv, cfg.cap, cfg.hd))
    cv = np.zeros_like(ck)
    O.cache_write(ck, cv, inj["k"], inj["v"], 0)
    A, Bc = w.codebooks()
    return dict(x=a(w.x())[0], base=a(w.conv_base()), w_delta=f(w.w_delta()), G=cfg.G, wq=f(w.wq()),
                wk=f(w.wk()), wv=f(w.wv()), wo=f(w.wo()), cache_k=ck, cache_v=cv, n_ctx=cfg.n_ctx,
                n_q_heads=cfg.Hq, w_lm=f(w.w_lm()), K=cfg.K, P=f(w.sel_proj()), A=a(A), Bc=a(Bc),
                anchor=int(w.anchor()[0]), bf16_points=False)


def test_block_step_wiring_residual_is_x():
    """Wo = 0 leaves the block output equal to the block input x exactly, so
    the residual is x (not the conv output u) and nothing else is added
    (reading R10); the LM head and selector then run on x."""
    cfg = configs.get(0)
    kw = _step_inputs(cfg)
    r = O.block_step(**dict(kw, wo=np.zeros_like(kw["wo"])))
    np.testing.assert_array_equal(r["attn"]["out"], kw["x"])
    np.testing.assert_allclose(r["topk"]["logits"], kw["x"] @ kw["w_lm"].T, rtol=1e-13, atol=1e-13)


def test_block_step_wiring_conv_feeds_attention():
    """base = the single tap e_0 with W_delta = 0 makes the conv the identity
    (reading R7), so the attention's Q / Kb / Vb are projections of x itself
    (the conv output feeds Q / K / V, reading R8); with a zero tap 0 instead,
    u = 0 and Q / Kb / Vb vanish."""
    cfg = configs.get(0)
    kw = _step_inputs(cfg)
    e0 = np.zeros_like(kw["base"])
    e0[0] = 1.0
    r = O.block_step(**dict(kw, base=e0, w_delta=np.zeros_like(kw["w_delta"])))
    np.testing.assert_array_equal(r["conv"]["u"][0], kw["x"])
    np.testing.assert_array_equal(r["attn"]["q"], kw["x"] @ kw["wq"].T)
    np.testing.assert_array_equal(r["attn"]["kb"], kw["x"] @ kw["wk"].T)
    r0 = O.block_step(**dict(kw, base=np.zeros_like(kw["base"]), w_delta=np.zeros_like(kw["w_delta"])))
    assert not np.any(r0["attn"]["q"]) and not np.any(r0["attn"]["vb"])


@pytest.mark.parametrize("kind", ["bf16", "q8_0"])
def test_lm_logits_stored_matches_a_direct_matmul(kind):
    """lm_logits_stored decodes the head a chunk of rows at a time; against
    torch's own decoding (bf16 -> fp64; Q8_0 codes times fp32 scales cast to
    bf16) and one fp64 matmul, across 16384-row chunk boundaries and a ragged
    last chunk.  Catches an off-by-one chunk edge, a chunk written to the
    wrong columns or a scale row misaligned with its codes."""
    V, d, B = 2 * 16384 + 1234, 64, 3
    h = randn(B, d)
    if kind == "bf16":
        wl = synth.weight(5, "lmpin", V, d, "bf16")
        wt = torch.from_numpy(wl["data"].view(np.int16)).view(torch.bfloat16).to(torch.float64)
    else:
        wl = synth.weight(5, "lmpin", V, d, "q8_0")
        q = torch.from_numpy(wl["data"].astype(np.float32)).view(V, d // 32, 32)
        sc = torch.from_numpy(wl["scales"]).to(torch.float32)[:, :, None]
        wt = (q * sc).to(torch.bfloat16).to(torch.float64).reshape(V, d)
    ref = (torch.from_numpy(h) @ wt.T).numpy()
    got = O.lm_logits_stored(h, wl)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-12)
    # the rows at the chunk edges are where they belong
    for v in (16383, 16384, 32767, 32768, V - 1):
        np.testing.assert_allclose(got[:, v], h @ wt[v].numpy(), rtol=1e-13, atol=1e-12)


# --------------------------------------------------------------------------
# feed-forward site (readings R19 - R21)
# --------------------------------------------------------------------------

def test_silu_is_x_times_the_logistic_function():
    """SiLU against scipy's logistic function expit, including large |x|
    where 1 + e^-x overflows; catches e^x for e^-x or a missing factor x."""
    x = np.concatenate([randn(20000, scale=4.0), [-800.0, -50.0, -1e-300, 0.0, 1e-300, 50.0, 800.0]])
    np.testing.assert_allclose(O.silu(x), x * scipy.special.expit(x), rtol=1e-14, atol=1e-300)
    assert O.silu(np.array([0.0]))[0] == 0.0


def test_silu_odd_part_is_the_identity():
    """silu(x) - silu(-x) = x (the logistic function satisfies s(x) + s(-x) = 1);
    catches a sign error in the exponent."""
    x = randn(5000, scale=6.0)
    np.testing.assert_allclose(O.silu(x) - O.silu(-x), x, rtol=1e-12, atol=1e-12)


def _ffn_inputs(d=64, d_ff=96, G=8, T=4, nb=3, B=5):
    return dict(h=randn(nb, B, d), base=randn(T, d, scale=0.7), w_delta=randn(T * G, d, scale=d ** -0.5),
                G=G, w_gate=randn(d_ff, d, scale=d ** -0.5), w_up=randn(d_ff, d, scale=d ** -0.5),
                w_down=randn(d, d_ff, scale=d_ff ** -0.5))


@pytest.mark.parametrize("bf16_points", [False, True])
def test_ffn_block_zero_down_projection_returns_the_input(bf16_points):
    """Wd = 0 leaves the block output equal to its input exactly: the residual
    is h itself (reading R21), not the conv output u, and nothing else is
    added (a bf16 h is unchanged by rounding)."""
    kw = _ffn_inputs()
    h = O.round_bf16(kw["h"]) if bf16_points else kw["h"]
    r = O.ffn_block(**dict(kw, h=h, w_down=np.zeros_like(kw["w_down"])), bf16_points=bf16_points)
    np.testing.assert_array_equal(r["out"], h)


def test_ffn_block_zero_conv_silences_the_mlp():
    """base = 0 and W_delta = 0 make u = 0, so gate, up and act vanish and the
    output is h: the MLP reads the conv output (R19), not h."""
    kw = _ffn_inputs()
    r = O.ffn_block(**dict(kw, base=np.zeros_like(kw["base"]), w_delta=np.zeros_like(kw["w_delta"])),
                    bf16_points=False)
    assert not np.any(r["u"]) and not np.any(r["act"])
    np.testing.assert_array_equal(r["out"], kw["h"])


def test_ffn_block_identity_weights_closed_form():
    """base = e_0 with W_delta = 0 makes the conv the identity (R7), and with
    d_ff = d, Wg = a I, Wu = I and Wd = I the block is elementwise:
    out = h + w a h^2 expit(a h) (scipy's logistic function), Wd = diag(w).
    Catches gate and up swapped (act would be a h^2 expit(h)) and a missing
    SiLU; the permutation below catches a transposed down projection."""
    d, a = 48, 1.7
    kw = _ffn_inputs(d=d, d_ff=d)
    h = kw["h"]
    e0 = np.zeros_like(kw["base"])
    e0[0] = 1.0
    w = randn(d)
    r = O.ffn_block(h=h, base=e0, w_delta=np.zeros_like(kw["w_delta"]), G=kw["G"], w_gate=a * np.eye(d),
                    w_up=np.eye(d), w_down=np.diag(w), bf16_points=False)
    np.testing.assert_allclose(r["out"], h + w * a * h ** 2 * scipy.special.expit(a * h), rtol=1e-12, atol=1e-12)
    # a permutation as the down projection: act column j lands in output row perm[j]
    perm = rng.permutation(d)
    wd = np.zeros((d, d))
    wd[perm, np.arange(d)] = 1.0
    r2 = O.ffn_block(h=h, base=e0, w_delta=np.zeros_like(kw["w_delta"]), G=kw["G"], w_gate=a * np.eye(d),
                     w_up=np.eye(d), w_down=wd, bf16_points=False)
    ref = h.copy()
    ref[..., perm] += (a * h ** 2 * scipy.special.expit(a * h))
    np.testing.assert_allclose(r2["out"], ref, rtol=1e-12, atol=1e-12)


def test_ffn_block_brute_force_tiny():
    """One output element by explicit sums over the pages' conv formula and the
    MLP, on a tiny case with dynamic taps (catches a wrong group, tap or
    position in the feed-forward site's conv and any index slip in the MLP)."""
    d, d_ff, G, T, B = 8, 6, 2, 3, 4
    kw = _ffn_inputs(d=d, d_ff=d_ff, G=G, T=T, nb=1, B=B)
    r = O.ffn_block(**kw, bf16_points=False)
    h, base, wd_, wg, wu, wdn = (kw["h"][0], kw["base"], kw["w_delta"], kw["w_gate"], kw["w_up"], kw["w_down"])
    cpg = d // G
    u = np.zeros((B, d))
    for i in range(B):
        for c in range(d):
            acc = 0.0
            for t in range(T):
                if i - t < 0:
                    continue
                delta = sum(h[i, k] * wd_[t * G + c // cpg, k] for k in range(d))
                acc += (base[t, c] + delta) * h[i - t, c]
            u[i, c] = acc
    for i in range(B):
        for c in range(d):
            tot = h[i, c]
            for j in range(d_ff):
                g = sum(u[i, k] * wg[j, k] for k in range(d))
                p = sum(u[i, k] * wu[j, k] for k in range(d))
                tot += g / (1.0 + np.exp(-g)) * p * wdn[c, j]
            assert abs(r["out"][0, i, c] - tot) <= 1e-12 * max(1.0, abs(tot))


# --------------------------------------------------------------------------
# generator
# --------------------------------------------------------------------------

def test_generator_rows_and_determinism():
    a = synth.normal(9, "t", (3000, 700), 1.0, "bf16")
    b = synth.normal(9, "t", (3000, 700), 1.0, "bf16")
    np.testing.assert_array_equal(a, b)
    rows = [0, 1497, 1498, 2999]
    np.testing.assert_array_equal(synth.normal_rows(9, "t", (3000, 700), 1.0, "bf16", rows), a[rows])
    ref = torch.from_numpy(synth.normal(9, "t", (3000, 700), 1.0, "f32")).to(torch.bfloat16)
    np.testing.assert_array_equal(a.view(np.int16), ref.view(torch.int16).numpy())
    s = synth.normal(1, "w", (4000, 512), 1.0 / 512, "f32")
    assert abs(s.var() * 512 - 1.0) < 0.01
