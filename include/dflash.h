/*
 * dflash.h - C ABI of libdflash, the DFlash / DFlash2 draft block step on
 * AMD Instinct MI355X (gfx950).
 *
 * The draft block step, as the pages describe it:
 *   "dflash: port #219 onto feature (rebased full CL)", Root Cause and "Why We
 *     Can't Easily Fix It": target features -> encode (fc matmul + norm) ->
 *     inject KV -> draft.
 *   "Turbo dflash", Overview: a light draft model proposes a block of tokens
 *     from target hidden states; "Deferred KV Injection Optimization", The
 *     Problem: injection is the Wk / Wv matmuls plus a write into the draft
 *     decoder's own KV cache, which the decoder reads when it drafts.
 *   "spec : add DFlash2 support (local convolution + candidate selector)",
 *     Overview: the grouped dynamic depthwise convolution and the candidate
 *     selector edge formula; review of tensor names: a conv pair at the
 *     attention site and one at the feed-forward site of each layer.
 *   "dflash: pass missing NVFP4 scales to attention operations", Overview:
 *     every per-block weight scale of the injection K/V, the decoder Q/K/V and
 *     both output projections must be applied.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Memory.  Every pointer argument is a device pointer unless the argument's
 *   comment says "host".  The caller allocates and owns everything, including
 *   the workspace; the library never allocates, frees or synchronises.
 * - Layout.  Activations are row-major [rows][features].  A weight is
 *   row-major [out][in] ("rows" x "cols").  The KV cache is
 *   [n_kv_heads][capacity][head_dim] for K and for V; column c of a K or V
 *   projection row belongs to head c / head_dim, dim c % head_dim.
 * - Types.  Activations, the KV cache, the conv base, W_delta, the selector
 *   projection and codebooks are either all fp32 or all bf16 (the "act" type).
 *   With fp32 activations every weight is fp32; with bf16 activations the fc,
 *   Wq, Wk, Wv, Wo, LM-head and feed-forward (gate, up, down) weights are bf16
 *   or Q8_0.  Arithmetic is fp32.
 * - Q8_0.  Blocks of 32 int8 codes along the input dim share one fp16 scale:
 *   data is int8 [rows][cols], scales is fp16 [rows][cols/32].  The value a
 *   kernel multiplies with is bf16_rne(fp32(scale) * code), i.e. the weight
 *   is dequantised to bf16 (round to nearest even) before the bf16 matrix
 *   multiply; every block's scale is applied.
 * - Rounding.  Values a call stores in the act type are rounded once from
 *   fp32 (bf16: round to nearest even).  fp32 outputs are not rounded.
 * - Streams.  `stream` is a hipStream_t passed as void* (NULL = the default
 *   stream).  A call only enqueues work; its outputs are valid when the stream
 *   reaches it, and every pointer must stay valid until then.
 * - Errors.  Every call checks its arguments before enqueueing anything: on
 *   an error it returns a non-OK status, writes nothing and launches nothing;
 *   dflash_last_error() then describes the problem (thread-local).  A kernel
 *   launch failure returns DFLASH_ERR_LAUNCH.  Nothing is thrown.
 * - Alignment.  Device pointers must be 16-byte aligned.
 * - Reentrancy.  The library holds no state between calls; calls on
 *   different streams with disjoint outputs and workspaces may overlap.
 * - Workspace.  A call that needs scratch device memory takes (ws, ws_bytes);
 *   the matching *_workspace() function returns the bytes it needs for the
 *   given shapes (0 for none).  A smaller workspace -> DFLASH_ERR_WORKSPACE.
 *   A workspace needs no initial contents and no clearing between calls: its
 *   first 64 KiB hold completion counters that each kernel launch stamps
 *   with a 48-bit value of its own, so whatever an earlier call (complete or
 *   not) or anything else left there is ignored.  Calls that share one
 *   workspace must be ordered (one stream, or events); overlapping calls on
 *   one workspace race.
 * - Intermediates.  After a call completes, its workspace holds the act-type
 *   intermediates named by the *_offset() queries until a later call reuses
 *   it (for stage-wise checking of each step against a reference).
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DFLASH_OK = 0,
  DFLASH_ERR_INVALID_ARG = 1,  /* null / misaligned pointer, bad shape or type mix */
  DFLASH_ERR_UNSUPPORTED = 2,  /* valid request outside what the kernels implement */
  DFLASH_ERR_CAPACITY = 3,     /* KV-cache rows out of range */
  DFLASH_ERR_WORKSPACE = 4,    /* workspace missing or too small */
  DFLASH_ERR_LAUNCH = 5        /* a kernel launch failed */
} dflash_status;

typedef enum { DFLASH_F32 = 0, DFLASH_BF16 = 1, DFLASH_Q8_0 = 2 } dflash_dtype;

/* A weight [rows][cols] (out x in).  data: fp32 / bf16 values or int8 Q8_0
 * codes; scales: fp16 [rows][cols/32] for Q8_0, else NULL. */
typedef struct {
  int32_t dtype;  /* dflash_dtype */
  int32_t reserved;
  int64_t rows;
  int64_t cols;
  const void *data;
  const void *scales;
} dflash_weight;

/* The draft decoder's KV cache.  K is [n_kv_heads][capacity][head_dim] (a
 * key is one contiguous row); V is stored in transposed panels of 32
 * positions, [n_kv_heads][capacity/32][head_dim][32]: element (h, pos, j) of
 * V sits at ((h*(capacity/32) + pos/32)*head_dim + j)*32 + pos%32.  32
 * positions of K and of V^T are then each one contiguous block for the
 * attention's streaming loads.  head_dim is 64 or 128; capacity is a
 * multiple of 64.
 * dtype is the act type, or DFLASH_Q8_0 with bf16 activations and head_dim
 * 128 ("dflash: port #219 onto feature", DFlash Benchmark Sweep: the draft's
 * K and V caches are q8_0): k and v then hold int8 codes in the same layouts,
 * and k_scales / v_scales fp16 [n_kv_heads][capacity][head_dim/32], one scale
 * per position and block of 32 consecutive head dims.  A row x (one position
 * of one head, the projection's fp32 output) is stored per block as
 * scale = fp16(max|x| / 127) and code = round-half-away(x / (max|x| / 127))
 * (0 for an all-zero block); the attention reads bf16_rne(fp32(scale) *
 * code).  k_scales / v_scales are NULL for other dtypes. */
typedef struct {
  int32_t dtype;  /* DFLASH_F32, DFLASH_BF16 or DFLASH_Q8_0 */
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t reserved;
  int64_t capacity;
  void *k;
  void *v;
  void *k_scales;
  void *v_scales;
} dflash_kv_cache;

/* Limits checked by every call. */
#define DFLASH_MAX_LAYERS 16   /* target layers concatenated by dflash_inject */
#define DFLASH_MAX_BLOCK 16    /* B: drafted tokens per block */
#define DFLASH_MAX_TOPK 32     /* K */

/* (1) KV injection.
 * "dflash: port #219 onto feature", Root Cause: the encoder is an fc matmul
 * over the chosen target layers' features plus a norm; "Turbo dflash", The
 * Problem: injection is the Wk / Wv projections plus the cache write; the
 * merge log on the NVFP4-scales page: encoder and injection run as one pass.
 *   h = [h_1 | ... | h_L]        concat along features, layers in the given order
 *   y = h . fc^T                 fc [d][L*d_t]                       (fp32)
 *   z = y / sqrt(mean(y^2) + eps) * gamma                            (act type)
 *   K = z . Wk^T, V = z . Wv^T   Wk, Wv [Hkv*hd][d]                  (act type)
 *   cache.k[h][pos0 + t][j] = K[t][h*hd + j], t < n_tokens
 *   V[t][h*hd + j] -> cache.v at position pos0 + t, head h, dim j
 *                     (transposed 32-position panels, see above)
 * A Q8_0 cache stores codes and scales of the fp32 K and V rows (not of
 * their bf16 roundings), as dflash_kv_cache describes.
 * layer_hidden: HOST array of n_layers device pointers, each [n_tokens][d_t]
 * in `act`.  gamma: [d] in `act`, or NULL for ones.  Requires
 * 0 <= pos0 && pos0 + n_tokens <= capacity (else DFLASH_ERR_CAPACITY),
 * d_t % 64 == 0, d % 64 == 0, n_tokens >= 1.  Cache positions outside
 * [pos0, pos0 + n_tokens) are not touched.  From 768 tokens on, the
 * workspace also holds bf16 copies of fc, Wk and Wv (2 bytes per weight,
 * reserved whatever their dtype): Q8_0 weights are expanded there once per
 * call, to the same bf16 values, bf16_rne(fp32(scale) * code), that the
 * products of fewer rows form as they read the codes. */
dflash_status dflash_inject(const void *const *layer_hidden, int32_t n_layers, int64_t n_tokens,
                            int32_t d_t, int32_t act, const dflash_weight *fc, const void *gamma,
                            float eps, const dflash_weight *wk, const dflash_weight *wv,
                            const dflash_kv_cache *cache, int64_t pos0, void *ws, size_t ws_bytes,
                            void *stream);
size_t dflash_inject_workspace(int32_t n_layers, int64_t n_tokens, int32_t d_t, int32_t d,
                               int32_t kv, int32_t act);
/* Byte offset into the injection's workspace of z [n_tokens][d] in `act`
 * (the RMSNorm output that Wk and Wv multiply), for the same arguments. */
size_t dflash_inject_z_offset(int32_t n_layers, int64_t n_tokens, int32_t d_t, int32_t d,
                              int32_t kv, int32_t act);

/* (2) DFlash2 grouped dynamic depthwise convolution.
 * "spec : add DFlash2 support", Overview:
 *   out[i,c] = sum_{t<T} (base[t,c] + delta[i,t,g(c)]) * x[i-t,c]
 * with delta[i][t*G + g] = x[i] . W_delta[t*G + g] (computed from the same
 * input row, shared by the channels of a group), contiguous groups g(c) = c / (C/G),
 * tap 0 = the current position, x before the block start = 0.
 * x, out: [n_blocks][B][C] in `act` (blocks are independent); base: [T][C]
 * in `act`; w_delta: [T*G][C] in `act`.  Requires C % G == 0, C % 64 == 0,
 * 1 <= T <= 16, 1 <= B <= DFLASH_MAX_BLOCK. */
dflash_status dflash_conv(const void *x, int32_t n_blocks, int32_t B, int32_t C, int32_t G,
                          int32_t T, int32_t act, const void *base, const dflash_weight *w_delta,
                          void *out, void *ws, size_t ws_bytes, void *stream);
size_t dflash_conv_workspace(int32_t n_blocks, int32_t B, int32_t C, int32_t G, int32_t T);

/* (2b) DFlash2 feed-forward site.  "spec : add DFlash2 support", review of
 * tensor names: each layer carries a second conv pair, ffn_conv_base /
 * ffn_conv_proj, beside the attention site's.  The pages name the tensors
 * only; this call takes the plainest reading of the site: the convolution of
 * (2) on the feed-forward input h, then a gated SiLU MLP and the residual,
 * with no biases and no norm:
 *   u   = conv(h)                         (as dflash_conv, act type)
 *   act = silu(u Wg^T) * (u Wu^T)         (products fp32, act in the act type)
 *   out = h + act Wd^T                    (act type)
 * silu(x) = x / (1 + e^-x).  h, out: [n_blocks][B][d] in `act`, not
 * overlapping; base [T][d] in `act`; w_delta [T*G][d] in `act`; w_gate,
 * w_up [d_ff][d] and w_down [d][d_ff] (bf16 / fp32 as `act`, or Q8_0 with
 * bf16 activations; w_gate and w_up share a dtype).  Requires d % 64 == 0,
 * d % G == 0, 1 <= T <= 16, 1 <= B <= DFLASH_MAX_BLOCK, d_ff % 64 == 0,
 * d_ff <= 2^20. */
dflash_status dflash_ffn_block(const void *h, int32_t n_blocks, int32_t B, int32_t d, int32_t G,
                               int32_t T, int32_t act, const void *base, const dflash_weight *w_delta,
                               const dflash_weight *w_gate, const dflash_weight *w_up,
                               const dflash_weight *w_down, void *out, void *ws, size_t ws_bytes,
                               void *stream);
size_t dflash_ffn_block_workspace(int32_t n_blocks, int32_t B, int32_t d, int32_t G, int32_t T,
                                  int32_t d_ff);
/* Byte offsets into that workspace, for the same arguments, of u
 * [n_blocks * B][d] and act [n_blocks * B][d_ff], both in `act`. */
size_t dflash_ffn_block_u_offset(int32_t n_blocks, int32_t B, int32_t d, int32_t G, int32_t T,
                                 int32_t d_ff);
size_t dflash_ffn_block_act_offset(int32_t n_blocks, int32_t B, int32_t d, int32_t G, int32_t T,
                                   int32_t d_ff);

/* (3) Non-causal block attention with the injected context.
 * "Turbo dflash", Overview (block diffusion drafting) and The Problem (the
 * decoder reads the injected cache); the NVFP4-scales page, Overview (Q, K, V
 * and output projections):
 *   Q = u Wq^T, Kb = u Wk^T, Vb = u Wv^T                               (act type)
 *   for query head h, KV head g = h / (Hq/Hkv):
 *     O_h = softmax(Q_h [Kctx_g | Kb_g]^T * scale) [Vctx_g | Vb_g]      (act type)
 *   out = residual + O Wo^T                                            (act type)
 * No mask: every block position sees all n_ctx context positions and all B
 * block rows.  Kctx / Vctx are cache positions [0, n_ctx) (V read from its
 * transposed panels).  The block's K/V are not written to the cache.
 * u, residual, out: [B][d] in `act` (residual NULL = none); Wq [Hq*hd][d],
 * Wk, Wv [Hkv*hd][d], Wo [d][Hq*hd]; scale 0 = 1/sqrt(hd).  Requires
 * 1 <= B <= DFLASH_MAX_BLOCK, Hq % Hkv == 0, 0 <= n_ctx <= capacity,
 * d % 64 == 0. */
dflash_status dflash_block_attn(const void *u, const void *residual, int32_t B, int32_t d,
                                int32_t n_q_heads, int32_t act, const dflash_weight *wq,
                                const dflash_weight *wk, const dflash_weight *wv,
                                const dflash_weight *wo, const dflash_kv_cache *cache,
                                int64_t n_ctx, float scale, void *out, void *ws, size_t ws_bytes,
                                void *stream);
/* (3) with the cache written on another stream: the same operation and
 * outputs, but `stream` waits for `cache_ready` (a hipEvent_t recorded
 * after the writes of cache positions [0, n_ctx), e.g. dflash_inject on a
 * second stream) once Q | Kb | Vb are enqueued and before the first kernel
 * that reads the cache.  "Turbo dflash", Deferred KV Injection
 * Optimization (the injection and the draft's own work are separate
 * steps): the projection of the block does not depend on the injection, so
 * the two can overlap.  cache_ready NULL -> DFLASH_ERR_INVALID_ARG (before
 * any HIP call); an event handle HIP rejects -> DFLASH_ERR_LAUNCH after the
 * projection was enqueued (only the workspace is written).  The workspace
 * is this call's alone while the event is pending: the injection that
 * overlaps it needs a workspace of its own. */
dflash_status dflash_block_attn_after(const void *u, const void *residual, int32_t B, int32_t d,
                                      int32_t n_q_heads, int32_t act, const dflash_weight *wq,
                                      const dflash_weight *wk, const dflash_weight *wv,
                                      const dflash_weight *wo, const dflash_kv_cache *cache,
                                      int64_t n_ctx, float scale, void *out, void *ws, size_t ws_bytes,
                                      void *stream, void *cache_ready);
size_t dflash_block_attn_workspace(int32_t B, int32_t d, int32_t n_q_heads, int32_t n_kv_heads,
                                   int32_t head_dim, int64_t n_ctx);
/* Byte offsets into the attention's workspace, for the same arguments, of
 * Q | Kb | Vb [B][(n_q_heads + 2 n_kv_heads) head_dim] and of
 * O [B][n_q_heads head_dim] (the softmax output before Wo), both in `act`. */
size_t dflash_block_attn_qkv_offset(int32_t B, int32_t d, int32_t n_q_heads, int32_t n_kv_heads,
                                    int32_t head_dim, int64_t n_ctx);
size_t dflash_block_attn_o_offset(int32_t B, int32_t d, int32_t n_q_heads, int32_t n_kv_heads,
                                  int32_t head_dim, int64_t n_ctx);

/* (4) Shared LM head, top-K candidates and log-softmax unary scores.
 * "Turbo dflash", Overview (the draft uses the target's output matrix);
 * "spec : add DFlash2 support", Overview (the unary term of an edge is the
 * draft's log-softmax score of the candidate) and the top-k review (small K over a wide vocabulary):
 *   l = h . W_lm^T  (fp32, never stored)
 *   idx[i] = the K largest l[i][.], largest first, equal logits -> lower index
 *   unary[i][k] = l[i][idx[i][k]] - log(sum_v exp(l[i][v]))
 * h: [B][d] in `act`, W_lm [V][d]; idx int32 [B][K]; unary fp32 [B][K].
 * Requires 1 <= B <= DFLASH_MAX_BLOCK, 1 <= K <= min(V, DFLASH_MAX_TOPK),
 * d % 64 == 0.  Deterministic: the same inputs give bitwise-equal outputs. */
dflash_status dflash_topk_unary(const void *h, int32_t B, int32_t act,
                                const dflash_weight *lm_head, int32_t K, int32_t *idx,
                                float *unary, void *ws, size_t ws_bytes, void *stream);
size_t dflash_topk_unary_workspace(int32_t B, int64_t V, int32_t K);

/* dflash_topk_unary without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments (minus ws), results, determinism and
 * errors as dflash_topk_unary; nothing is allocated.  Its scratch is a static
 * device array of DFLASH_TOPK_NOALLOC_SCRATCH_BYTES in the library, one per
 * GPU, held until the process ends; it serves any K <= DFLASH_MAX_TOPK for
 * vocabularies up to 2^20 rows, and a call that would need more returns
 * DFLASH_ERR_UNSUPPORTED before launching anything.  Calls on one GPU share
 * that array (it keeps the last call's contents, which no call reads):
 * calls that may overlap on one GPU (different streams without ordering)
 * race and must not be issued. */
#define DFLASH_TOPK_NOALLOC_SCRATCH_BYTES 4390912
dflash_status dflash_topk_unary_noalloc(const void *h, int32_t B, int32_t act,
                                        const dflash_weight *lm_head, int32_t K, int32_t *idx,
                                        float *unary, void *stream);

/* (5) Candidate-selector edges and the best path through them.
 * "spec : add DFlash2 support", Overview:
 *   edge(p -> c) = < A[p] (.) project(h), B[c] > + unary[c]
 * A = cb_pred, B = cb_succ [V][r] (the selector_predecessor / successor
 * codebooks), project(h) = h . P^T with P = proj [r][d] (selector_hidden).
 * Position i's candidates are c_{i,b} = idx[i][b]; its predecessors are
 * p_{i,a} = idx[i-1][a] for i >= 1 and the anchor token (the last accepted
 * token) for i = 0, so
 *   edges[i][a][b] = sum_rho A[p_{i,a}][rho] * proj[i][rho] * B[c_{i,b}][rho]
 *                    + unary[i][b]
 * Row 0 has one predecessor slot: edges[0][a >= 1][.] = -inf, and with
 * anchor = -1 edges[0][0][b] = unary[0][b].  The readout is the max-sum path:
 *   s_0[b] = edges[0][0][b];  s_i[b] = max_a s_{i-1}[a] + edges[i][a][b]
 * (ties -> lower a), final slot argmax_b s_{B-1}[b] (ties -> lower b), and
 * path[i] = idx[i][slot_i].
 * h: [B][d] in `act`; idx int32 [B][K] with values in [0, V); unary fp32
 * [B][K]; edges fp32 [B][K][K]; path int32 [B].  Requires
 * 1 <= B <= DFLASH_MAX_BLOCK, 1 <= K <= DFLASH_MAX_TOPK, r % 16 == 0,
 * r <= 256, -1 <= anchor < V, d % 64 == 0.  Indices in idx outside [0, V)
 * are clamped into range by the kernel (never read out of bounds).
 * target int32 [B] and accept int32 [1]: both NULL, or both given, and then
 * accept[0] = the greedy accept length of path against target, as
 * dflash_accept_len computes it for one sequence (in the same kernel). */
dflash_status dflash_selector_edges(const void *h, int32_t B, int32_t act,
                                    const dflash_weight *proj, const void *cb_pred,
                                    const void *cb_succ, int64_t V, const int32_t *idx,
                                    const float *unary, int32_t K, int32_t anchor, float *edges,
                                    int32_t *path, const int32_t *target, int32_t *accept, void *ws,
                                    size_t ws_bytes, void *stream);
size_t dflash_selector_edges_workspace(int32_t B, int32_t r, int32_t d, int32_t K);

/* (4) + (5) in one call: exactly the outputs of dflash_topk_unary followed
 * by dflash_selector_edges with V = lm_head->rows and the same h ("Turbo
 * dflash", Overview; "spec : add DFlash2 support", Overview).  Arguments
 * and requirements are those of the two calls; proj and lm_head share d.
 * Where the LM head keeps h resident in LDS, K <= 8 and the candidate rows
 * fit in LDS, the LM head's final merge and the whole selector (projection
 * included) run in one kernel after the LM head's kernel; otherwise the two
 * calls' kernels run in turn.  Either way idx, unary, edges, path (and
 * accept) are bit for bit those of the two calls.  ws:
 * dflash_topk_select_workspace(B, V, K, r, d) bytes (0 for invalid sizes). */
dflash_status dflash_topk_select(const void *h, int32_t B, int32_t act, const dflash_weight *lm_head,
                                 int32_t K, const dflash_weight *proj, const void *cb_pred,
                                 const void *cb_succ, int32_t anchor, int32_t *idx, float *unary,
                                 float *edges, int32_t *path, const int32_t *target, int32_t *accept,
                                 void *ws, size_t ws_bytes, void *stream);
size_t dflash_topk_select_workspace(int32_t B, int64_t V, int32_t K, int32_t r, int32_t d);

/* Row-wise top-K of a score matrix (a standalone form of the selection in
 * (4)).  "spec : add DFlash2 support", the top-k kernel review: a small K
 * chosen from very wide rows, measured against a full sort.
 *   idx[r][j] = column of the j-th largest x[r][*]: values descending, equal
 *               values in ascending column order (-0.0 counts as +0.0)
 *   val[r][j] = x[r][idx[r][j]]
 * x: fp32 [n_rows][n_cols] (device); idx int32 and val fp32 [n_rows][K].
 * Requires 1 <= n_rows <= 65535, 1 <= n_cols < 2^31, 1 <= K <=
 * min(n_cols, DFLASH_MAX_ROW_TOPK); x holds no NaN (the result is then
 * unspecified).  Results are exact (indices and copied values). */
#define DFLASH_MAX_ROW_TOPK 1024
dflash_status dflash_topk_rows(const float *x, int64_t n_rows, int64_t n_cols, int32_t K, int32_t *idx,
                               float *val, void *ws, size_t ws_bytes, void *stream);
size_t dflash_topk_rows_workspace(int64_t n_rows, int64_t n_cols, int32_t K);

/* (6) Greedy accept length.
 * "dflash: port #219 onto feature", benchmark sweep (greedy sampling) and
 * "spec : add DFlash2 support", Overview table (acceptance per block):
 *   accept[s] = max{ m : draft[s][j] == target[s][j] for all j < m }
 * draft, target int32 [n_seq][B]; accept int32 [n_seq].  Requires n_seq >= 1,
 * B >= 1. */
dflash_status dflash_accept_len(const int32_t *draft, const int32_t *target, int32_t n_seq,
                                int32_t B, int32_t *accept, void *stream);

/* Text of a status code (static storage). */
const char *dflash_status_string(int32_t status);
/* Detail of the last non-OK return on this thread ("" if none). */
const char *dflash_last_error(void);
/* Library version, major * 10000 + minor * 100 + patch. */
int32_t dflash_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH_H */
