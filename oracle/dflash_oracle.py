"""fp64 CPU oracle of the DFlash / DFlash2 draft block step.

TEST INFRASTRUCTURE.  This is the correctness reference for the HIP library:
only tests, the smoke check and the benchmark's CPU-baseline timing may
import it.  It shares no code with the library (no kernels, headers, helpers,
tables or pre/post-processing) and reads its inputs in the storage formats
the seeded generator writes (fp32, bf16 bit patterns, Q8_0 codes + scales).

Sources (web pages, cited by title and section):
  [P1] "dflash: port #219 onto feature (rebased full CL)"
       - "DFlash Benchmark Sweep": every result table runs the draft with
         q8_0 K and V caches (the Cache K / Cache V columns).
       - "DFlash Prompt Processing Speed", Root Cause: the encoder is an fc
         matmul over the concatenated target-layer features plus a norm.
       - "Why We Can't Easily Fix It": the chain target features -> encode ->
         inject KV -> draft.
  [P2] "Turbo dflash"
       - Overview: a light draft model proposes a block of tokens from target
         hidden states and noise latents; it shares the target's output head.
       - "Deferred KV Injection Optimization", The Problem: injection is the
         K/V projections plus a write into the draft decoder's own KV cache,
         which the decoder reads when it drafts.
  [P3] "spec : add DFlash2 support (local convolution + candidate selector)"
       - Overview: the grouped dynamic depthwise convolution and the
         candidate-selector edge formula, whose unary term is the draft's
         log-softmax score of the candidate.
       - review of tensor names: attn_conv_base / attn_conv_proj and
         ffn_conv_base / ffn_conv_proj per layer, selector predecessor /
         successor / hidden tensors.
  [P4] "dflash: pass missing NVFP4 scales to attention operations"
       - Overview: every per-block weight scale of the K/V injection
         projections, the decoder's Q/K/V projections and both output
         projections must be applied.
       - merge log: the encoder (fc + norm) runs inline in the injection.

Readings where the pages are silent (each also listed in the design notes):
  R1 concat order: target layers in the given order, features [h_1 | .. | h_Lt].
  R2 no biases.
  R3 RMSNorm z = y / sqrt(mean(y^2) + eps) * gamma.
  R4 no rotary embedding / key norm.
  R5 contiguous conv groups g(c) = c // (C/G).
  R6 delta[i][t*G + g] = x[i] . W_delta[t*G + g]; no bias, no activation.
  R7 tap t = 0 is the current position; causal; zero before the block start.
  R8 the conv runs on the block input before the Q/K/V projections.
  R9 attention scale 1/sqrt(hd), GQA kv_head = h // (Hq/Hkv), no mask over
     [context | block]; block K/V are not written to the cache.
  R10 h_out = x + O . Wo^T; no FFN inside the block step (the feed-forward
      site is its own call, R19 - R21), no final norm; logit scale 1, no softcap.
  R11 top-K in descending logit order, equal logits -> lower vocab index;
      unary = logit - logsumexp(all logits).
  R12 predecessors of position 0: the anchor token only (anchor -1: none).
  R14 max-sum best path; ties -> lower slot.
  R15 accept length = longest common prefix with the target tokens.
  R-Q8 Q8_0 weight value = bf16_rne(fp32(scale) * q).
  R-RP in bf16 workloads the values the GPU stores as bf16 are rounded to
       bf16 here too: z, the cache rows, conv output u, Q/Kb/Vb, O and h_out.
  R19 the DFlash2 layer's second conv pair (ffn_conv_base / ffn_conv_proj)
      runs the same grouped dynamic conv on the feed-forward block's input,
      which is the attention block's output h_out.
  R20 the feed-forward block is a gated MLP with SiLU on the gate, no
      biases: act = silu(u Wg^T) * (u Wu^T), SiLU(x) = x / (1 + e^-x).
  R21 it adds its output to its input (residual); no norm is applied
      (the pages name none).  In bf16 workloads u, act and the block output
      are rounded to bf16 (R-RP); the gate and up products are not.
  R-KVQ a Q8_0 KV cache holds, per (KV head, position), blocks of 32 along
       the head dim: scale = max|x| / 127 stored as fp16, code = x / scale
       rounded to the nearest integer with ties away from zero (all codes 0
       when the block is all zero), x being the unrounded projection output;
       the attention reads value = bf16_rne(fp32(scale) * code) in bf16
       workloads (as R-Q8), fp32(scale) * code in fp32 ones.
"""
from __future__ import annotations

import numpy as np

QBLOCK = 32

# ---------------------------------------------------------------------------
# storage decoding (the oracle's own; no code shared with the library)
# ---------------------------------------------------------------------------


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact fp64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 (via fp32; round to nearest, ties to even)."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def round_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def q8_0_to_f64(q: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Q8_0 weight values (reading R-Q8): each block of 32 codes along the
    input dim shares one fp16 scale; value = bf16_rne(fp32(scale) * q).
    [P4] Overview: a missing per-block scale is the bug the page fixes, so
    every scale is applied here."""
    q = np.asarray(q, dtype=np.float64)
    rows, cols = q.shape
    s = np.asarray(scales, dtype=np.float16).astype(np.float32).astype(np.float64)
    if s.shape != (rows, cols // QBLOCK):
        raise ValueError("scale shape")
    prod = q.reshape(rows, cols // QBLOCK, QBLOCK) * s[:, :, None]   # exact in fp32
    return round_bf16(prod.reshape(rows, cols))


def act_to_f64(a: np.ndarray, act: str) -> np.ndarray:
    if act == "bf16":
        return bf16_to_f64(a)
    return np.asarray(a, dtype=np.float64)


def weight_to_f64(w: dict) -> np.ndarray:
    if w["dtype"] == "q8_0":
        return q8_0_to_f64(w["data"], w["scales"])
    return act_to_f64(w["data"], w["dtype"])


def _rp(x, bf16_points: bool):
    """A rounding point: bf16 in bf16 workloads, none in fp32 ones."""
    return round_bf16(x) if bf16_points else x


# ---------------------------------------------------------------------------
# (1) KV injection  [P1] Root Cause; [P2] The Problem; [P4] merge log
# ---------------------------------------------------------------------------


def rmsnorm(y: np.ndarray, gamma, eps: float) -> np.ndarray:
    """Reading R3: z = y / sqrt(mean(y^2) + eps) * gamma, per row."""
    ms = np.mean(y * y, axis=-1, keepdims=True)
    z = y / np.sqrt(ms + eps)
    if gamma is not None:
        z = z * gamma
    return z


def encode(hidden: list, fc: np.ndarray, gamma, eps: float, bf16_points: bool) -> dict:
    """The encoder of the injection: [P1] Root Cause, an fc matmul over the
    concatenated features of the chosen target layers followed by a norm.
      h = [h_1 | ... | h_Lt]  (R1)     y = h . fc^T      z = RMSNorm(y)  (R-RP: bf16)
    """
    h = np.concatenate(hidden, axis=1)
    y = h @ fc.T
    z = _rp(rmsnorm(y, gamma, eps), bf16_points)
    return {"y": y, "z": z}


def kv_project(z: np.ndarray, wk: np.ndarray, wv: np.ndarray, bf16_points: bool) -> dict:
    """[P2] The Problem: the injected rows' K and V are the Wk / Wv projections
    of the encoder output.  K = z . Wk^T, V = z . Wv^T  (R-RP: bf16)."""
    return {"k": _rp(z @ wk.T, bf16_points), "v": _rp(z @ wv.T, bf16_points)}


def inject(hidden: list, fc: np.ndarray, gamma, eps: float, wk: np.ndarray,
           wv: np.ndarray, bf16_points: bool) -> dict:
    """Encoder plus K/V projections for n injected tokens.

    [P1] Root Cause: the encoder is the fc matmul over the features of the
    chosen target layers, then a norm.  [P2] The Problem: injection is the
    Wk / Wv matmuls plus the cache write.  [P4] merge log: encoder and
    injection form one pass.  The two stages are encode() and kv_project().
    Returns the intermediates and the K / V rows [n][Hkv*hd] as stored.
    """
    e = encode(hidden, fc, gamma, eps, bf16_points)
    kv = kv_project(e["z"], wk, wv, bf16_points)
    return {"y": e["y"], "z": e["z"], "k": kv["k"], "v": kv["v"]}


def cache_write(cache_k: np.ndarray, cache_v: np.ndarray, k_rows: np.ndarray,
                v_rows: np.ndarray, pos0: int) -> None:
    """Write K / V rows [n][Hkv*hd] into the cache [Hkv][capacity][hd] at
    positions [pos0, pos0 + n); column c of a row is head c // hd, dim c % hd."""
    hkv, cap, hd = cache_k.shape
    n = k_rows.shape[0]
    if pos0 < 0 or pos0 + n > cap:
        raise ValueError("cache capacity")
    cache_k[:, pos0:pos0 + n, :] = k_rows.reshape(n, hkv, hd).transpose(1, 0, 2)
    cache_v[:, pos0:pos0 + n, :] = v_rows.reshape(n, hkv, hd).transpose(1, 0, 2)


def kv_quant_q8_0(x: np.ndarray):
    """Q8_0 cache rows (reading R-KVQ).  [P1] DFlash Benchmark Sweep: the
    draft's K and V caches are q8_0 in every measurement.  x [..., hd] with
    hd a multiple of 32 -> (codes int8 [..., hd], scales fp16 [..., hd/32])."""
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[-1]
    if hd % QBLOCK:
        raise ValueError("head dim not a multiple of 32")
    blocks = x.reshape(*x.shape[:-1], hd // QBLOCK, QBLOCK)
    scale = np.max(np.abs(blocks), axis=-1) / 127.0
    safe = np.where(scale > 0, scale, 1.0)
    t = np.where(scale[..., None] > 0, blocks / safe[..., None], 0.0)
    codes = np.sign(t) * np.floor(np.abs(t) + 0.5)          # ties away from zero
    return codes.astype(np.int8).reshape(x.shape), scale.astype(np.float16)


def kv_dequant_q8_0(codes: np.ndarray, scales: np.ndarray, bf16_points: bool) -> np.ndarray:
    """Values the attention reads from a Q8_0 cache (reading R-KVQ):
    fp32(scale) * code, rounded to bf16 in bf16 workloads (the product of an
    fp16 scale and an 8-bit code is exact in fp32)."""
    q = np.asarray(codes, dtype=np.float64)
    hd = q.shape[-1]
    s = np.asarray(scales, dtype=np.float16).astype(np.float32).astype(np.float64)
    if s.shape != q.shape[:-1] + (hd // QBLOCK,):
        raise ValueError("scale shape")
    v = (q.reshape(*q.shape[:-1], hd // QBLOCK, QBLOCK) * s[..., None]).reshape(q.shape)
    return _rp(v, bf16_points)


# ---------------------------------------------------------------------------
# (2) grouped dynamic depthwise convolution  [P3] Overview, first formula
# ---------------------------------------------------------------------------


def conv_delta(x: np.ndarray, w_delta: np.ndarray) -> np.ndarray:
    """Reading R6: the per-position kernel offsets, computed from the same
    input row, delta[..., i, t*G + g] = x[..., i, :] . W_delta[t*G + g, :]."""
    return x @ w_delta.T


def conv(x: np.ndarray, base: np.ndarray, w_delta: np.ndarray, G: int,
         bf16_points: bool) -> dict:
    """[P3] Overview: out[i,c] = sum_t (base[t,c] + delta[i,t,g(c)]) * x[i-t,c].

    x [n_blocks][B][C]; base [T][C]; W_delta [T*G][C].  delta is shared by the
    channels of one group (R5: contiguous groups); taps are causal inside the
    block and x before the block start is zero (R7).
    """
    nb, B, C = x.shape
    T = base.shape[0]
    if C % G or w_delta.shape != (T * G, C):
        raise ValueError("conv shapes")
    cpg = C // G
    delta = conv_delta(x, w_delta).reshape(nb, B, T, G)
    out = np.zeros_like(x)
    for t in range(T):
        # kernel value seen by (block, position i, channel c) for tap t
        kern = base[t][None, None, :] + np.repeat(delta[:, :, t, :], cpg, axis=2)
        shifted = np.zeros_like(x)
        if t < B:
            shifted[:, t:, :] = x[:, :B - t, :]
        out += kern * shifted
    return {"delta": delta.reshape(nb, B, T * G), "u": _rp(out, bf16_points)}


# ---------------------------------------------------------------------------
# (3) non-causal block attention  [P2] Overview / The Problem; [P4] Overview
# ---------------------------------------------------------------------------


# unit roundoff of bf16 (8 significant bits): |bf16_rne(x) - x| <= U_BF16 |x|
U_BF16 = 2.0 ** -8


def softmax_attend(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, scale: float,
                   weight_rounding: float = 0.0) -> tuple:
    """Softmax attention of queries [m][hd] over keys/values [S][hd], no mask.

    Returns (out, bound).  `weight_rounding` = u > 0 declares that an
    implementation may round each unnormalised softmax weight to a relative
    error of at most u before it multiplies V (and sums the rounded weights as
    the normaliser); then out_impl = sum_s w_s (1+e_s) V_s / sum_s w_s (1+e_s)
    with |e_s| <= u, so |out_impl - out| <= u / (1 - u) * sum_s w_s |V_s - out|
    per element, which is `bound` (zeros for u = 0)."""
    s = (q @ keys.T) * scale
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    out = p @ vals
    bound = np.zeros_like(out)
    if weight_rounding:
        for i in range(q.shape[0]):
            bound[i] = p[i] @ np.abs(vals - out[i][None, :])
        bound *= weight_rounding / (1.0 - weight_rounding)
    return out, bound


def attn_qkv(u: np.ndarray, wq: np.ndarray, wk: np.ndarray, wv: np.ndarray,
             bf16_points: bool) -> dict:
    """[P4] Overview: the decoder's Q, K and V projections of the block input.
    Q = u Wq^T, Kb = u Wk^T, Vb = u Wv^T  (R-RP: bf16), each [B][heads*hd]."""
    return {"q": _rp(u @ wq.T, bf16_points), "kb": _rp(u @ wk.T, bf16_points),
            "vb": _rp(u @ wv.T, bf16_points)}


def attn_core(q: np.ndarray, kb: np.ndarray, vb: np.ndarray, cache_k: np.ndarray,
              cache_v: np.ndarray, n_ctx: int, n_q_heads: int, scale: float,
              bf16_points: bool, with_bound: bool = False) -> dict:
    """[P2] Overview / The Problem: each query head attends the injected
    context and the whole block, no mask (block diffusion drafts the block at
    once).  Head h uses KV head h // (Hq/Hkv) (R9); scale 1/sqrt(hd) unless
    given; O is rounded to bf16 in bf16 workloads (R-RP).
    q [B][Hq*hd], kb / vb [B][Hkv*hd]; cache [Hkv][capacity][hd], n_ctx rows.
    "o_bound" (with_bound) is softmax_attend's bound for weights rounded to
    bf16 (the GPU's P.V operands), zeros in fp32 workloads."""
    B = q.shape[0]
    hkv, cap, hd = cache_k.shape
    if n_q_heads % hkv or n_ctx > cap:
        raise ValueError("attention shapes")
    grp = n_q_heads // hkv
    if not scale:
        scale = 1.0 / np.sqrt(hd)
    q = q.reshape(B, n_q_heads, hd)
    kb = kb.reshape(B, hkv, hd)
    vb = vb.reshape(B, hkv, hd)
    o = np.zeros((B, n_q_heads, hd))
    ob = np.zeros_like(o)
    u_w = U_BF16 if (bf16_points and with_bound) else 0.0
    for h in range(n_q_heads):
        g = h // grp
        keys = np.concatenate([cache_k[g, :n_ctx], kb[:, g]], axis=0)
        vals = np.concatenate([cache_v[g, :n_ctx], vb[:, g]], axis=0)
        o[:, h], ob[:, h] = softmax_attend(q[:, h], keys, vals, scale, u_w)
    o = o.reshape(B, n_q_heads * hd)
    return {"o_pre": o, "o": _rp(o, bf16_points), "o_bound": ob.reshape(B, n_q_heads * hd)}


def attn_out(o: np.ndarray, wo: np.ndarray, resid, bf16_points: bool) -> np.ndarray:
    """[P4] Overview: the output projection; R10: plus the residual.
    out = resid + O Wo^T  (R-RP: bf16)."""
    out = o @ wo.T
    if resid is not None:
        out = out + resid
    return _rp(out, bf16_points)


def block_attn(u: np.ndarray, resid, wq: np.ndarray, wk: np.ndarray, wv: np.ndarray,
               wo: np.ndarray, cache_k: np.ndarray, cache_v: np.ndarray, n_ctx: int,
               n_q_heads: int, scale: float, bf16_points: bool) -> dict:
    """B draft queries attend [injected context | block] keys, no mask:
    attn_qkv -> attn_core -> attn_out.

    [P2] Overview: the block is drafted at once (block diffusion), so the
    block's positions see each other; The Problem: the decoder reads the
    injected cache.  [P4] Overview: Q, K, V and output projections.
    u, resid [B][d]; cache [Hkv][capacity][hd] with n_ctx valid rows.
    """
    p = attn_qkv(u, wq, wk, wv, bf16_points)
    c = attn_core(p["q"], p["kb"], p["vb"], cache_k, cache_v, n_ctx, n_q_heads, scale, bf16_points)
    out = attn_out(c["o"], wo, resid, bf16_points)
    return {"q": p["q"], "kb": p["kb"], "vb": p["vb"], "o": c["o"], "out": out}


# ---------------------------------------------------------------------------
# (4) shared LM head, top-K candidates, log-softmax unary  [P2] Overview;
#     [P3] Overview (the unary term of an edge) and top-k review
# ---------------------------------------------------------------------------


def top_k_select(scores: np.ndarray, K: int) -> np.ndarray:
    """The K largest entries of each row, largest first; equal scores are
    taken in ascending index order (R11).  Plain repeated selection."""
    s = np.array(scores, dtype=np.float64, copy=True)
    rows, n = s.shape
    if K > n:
        raise ValueError("K > row length")
    out = np.empty((rows, K), dtype=np.int64)
    ar = np.arange(rows)
    for k in range(K):
        j = np.argmax(s, axis=1)          # first (lowest) index among equal maxima
        out[:, k] = j
        s[ar, j] = -np.inf
    return out


def logsumexp_rows(x: np.ndarray) -> np.ndarray:
    m = x.max(axis=1, keepdims=True)
    return (m + np.log(np.exp(x - m).sum(axis=1, keepdims=True)))[:, 0]


def lm_logits(h: np.ndarray, w_lm: np.ndarray, row_chunk: int = 32768) -> np.ndarray:
    """logits = h . W_lm^T in fp64, W_lm [V][d] (the target's output matrix)."""
    V = w_lm.shape[0]
    out = np.empty((h.shape[0], V))
    for r0 in range(0, V, row_chunk):
        out[:, r0:r0 + row_chunk] = h @ w_lm[r0:r0 + row_chunk].T
    return out


def lm_logits_stored(h: np.ndarray, w: dict, row_chunk: int = 16384) -> np.ndarray:
    """logits = h . W_lm^T with W_lm given in storage form (decoded a chunk
    of rows at a time, so a 1.5 GB head never exists in fp64 at once)."""
    V = w["rows"]
    out = np.empty((h.shape[0], V))
    for r0 in range(0, V, row_chunk):
        r1 = min(V, r0 + row_chunk)
        if w["dtype"] == "q8_0":
            blk = q8_0_to_f64(w["data"][r0:r1], w["scales"][r0:r1])
        else:
            blk = act_to_f64(w["data"][r0:r1], w["dtype"])
        out[:, r0:r1] = h @ blk.T
    return out


def topk_unary_from_logits(logits: np.ndarray, K: int) -> dict:
    idx = top_k_select(logits, K)
    lse = logsumexp_rows(logits)
    unary = np.take_along_axis(logits, idx, axis=1) - lse[:, None]
    return {"idx": idx.astype(np.int32), "unary": unary, "lse": lse}


def topk_unary(h: np.ndarray, w_lm: np.ndarray, K: int) -> dict:
    """idx = top-K of h . W_lm^T per row; unary = logit[idx] - logsumexp(logits)."""
    logits = lm_logits(h, w_lm)
    r = topk_unary_from_logits(logits, K)
    r["logits"] = logits
    return r


def topk_gaps(logits: np.ndarray, K: int) -> dict:
    """Score gaps used to decide which top-K results are unique:
    kth_gap[row] = l_(K) - l_(K+1) (inf when K = V); adj_gap[row][k] =
    l_(k) - l_(k+1) for k < K-1, in sorted order."""
    srt = -np.sort(-logits, axis=1)
    V = logits.shape[1]
    kth = srt[:, K - 1] - srt[:, K] if K < V else np.full(logits.shape[0], np.inf)
    adj = srt[:, :K - 1] - srt[:, 1:K]
    return {"kth_gap": kth, "adj_gap": adj}


# ---------------------------------------------------------------------------
# (5) candidate-selector edges and best path  [P3] Overview, second formula;
#     tensor names selector_predecessor / selector_successor / selector_hidden
# ---------------------------------------------------------------------------


def selector_edges(h: np.ndarray, P: np.ndarray, A: np.ndarray, Bc: np.ndarray,
                   idx: np.ndarray, unary: np.ndarray, anchor: int) -> dict:
    """edge(p -> c) = < A[p] (.) project(h), B[c] > + unary[c].

    [P3] Overview: A / B are the predecessor / candidate codebooks, project(h)
    maps this position's hidden state to the codebook rank, and unary[c] is
    the draft's log-softmax score of candidate c.  Candidates of position i are c_{i,b} = idx[i][b];
    predecessors are p_{i,a} = idx[i-1][a] for i >= 1 and the anchor token
    for i = 0 (R12).  Row 0 has one predecessor slot (a = 0); its other slots
    are -inf.  With anchor = -1 row 0 is the unary score alone.
    h [B][d]; P [r][d]; A, Bc [V][r]; idx [B][K]; unary [B][K].
    """
    B, K = idx.shape
    proj = h @ P.T                                            # [B][r]
    edges = np.full((B, K, K), -np.inf)
    for i in range(B):
        succ = Bc[idx[i]]                                     # [K][r]
        if i == 0:
            if anchor < 0:
                edges[0, 0, :] = unary[0]
            else:
                edges[0, 0, :] = (A[anchor] * proj[0]) @ succ.T + unary[0]
        else:
            pred = A[idx[i - 1]]                              # [K][r]
            edges[i] = (pred * proj[i][None, :]) @ succ.T + unary[i][None, :]
    return {"proj": proj, "edges": edges}


def viterbi(edges: np.ndarray) -> dict:
    """Max-sum best path over the K x K lattice (R14).
    s_0[b] = e[0][0][b];  s_i[b] = max_a s_{i-1}[a] + e[i][a][b]; ties -> lower a;
    final slot = argmax_b s_{B-1}[b], ties -> lower b.  Also returns the score
    of the best path that differs from it (runner-up), for the uniqueness gap."""
    B, K, _ = edges.shape
    s = edges[0, 0].copy()
    s2 = np.full(K, -np.inf)              # second-best distinct path ending at b
    back = np.zeros((B, K), dtype=np.int64)
    for i in range(1, B):
        cand = s[:, None] + edges[i]                       # [a][b]
        cand2 = s2[:, None] + edges[i]
        back[i] = np.argmax(cand, axis=0)                  # first max -> lower a
        best = cand[back[i], np.arange(K)]
        # runner-up at b: best over all (a, rank) pairs except the chosen one
        pool = np.concatenate([cand, cand2], axis=0)       # [2K][b]
        pool[back[i], np.arange(K)] = -np.inf
        s, s2 = best, pool.max(axis=0)
    b = int(np.argmax(s))
    best_score = s[b]
    others = np.concatenate([np.delete(s, b), s2])
    runner = others.max() if others.size else -np.inf
    slots = np.zeros(B, dtype=np.int64)
    slots[B - 1] = b
    for i in range(B - 1, 0, -1):
        slots[i - 1] = back[i, slots[i]]
    return {"slots": slots, "score": best_score, "runner_up": runner}


def path_score(edges: np.ndarray, slots) -> float:
    sc = edges[0, 0, slots[0]]
    for i in range(1, len(slots)):
        sc += edges[i, slots[i - 1], slots[i]]
    return float(sc)


def selector(h, P, A, Bc, idx, unary, anchor) -> dict:
    r = selector_edges(h, P, A, Bc, idx, unary, anchor)
    v = viterbi(r["edges"])
    r.update(v)
    r["path"] = idx[np.arange(idx.shape[0]), v["slots"]].astype(np.int32)
    return r


# ---------------------------------------------------------------------------
# (6) greedy accept length  [P1] benchmark sweep (greedy sampling);
#     [P3] Overview table (acceptance per block)
# ---------------------------------------------------------------------------


def accept_len(draft: np.ndarray, target: np.ndarray) -> np.ndarray:
    """Number of leading draft tokens equal to the target tokens (R15)."""
    draft = np.asarray(draft)
    target = np.asarray(target)
    n_seq, B = draft.shape
    out = np.zeros(n_seq, dtype=np.int32)
    for s in range(n_seq):
        m = 0
        while m < B and draft[s, m] == target[s, m]:
            m += 1
        out[s] = m
    return out


# ---------------------------------------------------------------------------
# (7) the DFlash2 layer's feed-forward site  [P3] review of tensor names
# ---------------------------------------------------------------------------


def silu(x: np.ndarray) -> np.ndarray:
    """R20: SiLU(x) = x / (1 + e^-x), the gate activation."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def ffn_hidden(u: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, bf16_points: bool) -> dict:
    """R20: gate = u Wg^T and up = u Wu^T (no rounding point), then
    act = silu(gate) * up (R21: bf16 in bf16 workloads)."""
    g = u @ w_gate.T
    p = u @ w_up.T
    return {"gate": g, "up": p, "act": _rp(silu(g) * p, bf16_points)}


def ffn_out(h: np.ndarray, act: np.ndarray, w_down: np.ndarray, bf16_points: bool) -> np.ndarray:
    """R21: out = h + act Wd^T (bf16 in bf16 workloads)."""
    return _rp(h + act @ w_down.T, bf16_points)


def ffn_block(h: np.ndarray, base: np.ndarray, w_delta: np.ndarray, G: int, w_gate: np.ndarray,
              w_up: np.ndarray, w_down: np.ndarray, bf16_points: bool) -> dict:
    """[P3] review of tensor names: besides the attention site's conv pair a
    layer holds ffn_conv_base / ffn_conv_proj.  R19: that conv runs on the
    feed-forward input h [n_blocks][B][d]; R20: the gated MLP follows; R21:
    with the residual.  u = conv(h); act = silu(u Wg^T) * (u Wu^T);
    out = h + act Wd^T."""
    c = conv(h, base, w_delta, G, bf16_points)
    f = ffn_hidden(c["u"], w_gate, w_up, bf16_points)
    out = ffn_out(h, f["act"], w_down, bf16_points)
    return {"delta": c["delta"], "u": c["u"], "gate": f["gate"], "up": f["up"], "act": f["act"],
            "out": out}


# ---------------------------------------------------------------------------
# the whole block step
# ---------------------------------------------------------------------------


def block_step(x, base, w_delta, G, wq, wk, wv, wo, cache_k, cache_v, n_ctx, n_q_heads,
               w_lm, K, P, A, Bc, anchor, bf16_points, scale=0.0) -> dict:
    """[P1] Why We Can't Easily Fix It: ... -> inject KV -> draft.  One block:
    conv (R8) -> block attention + residual (R10) -> LM head top-K + unary ->
    selector edges + best path.  x [B][d] is one block."""
    c = conv(x[None], base, w_delta, G, bf16_points)
    u = c["u"][0]
    a = block_attn(u, x, wq, wk, wv, wo, cache_k, cache_v, n_ctx, n_q_heads, scale, bf16_points)
    h = a["out"]
    t = topk_unary(h, w_lm, K)
    s = selector(h, P, A, Bc, t["idx"], t["unary"], anchor)
    return {"conv": c, "attn": a, "topk": t, "sel": s, "path": s["path"]}
