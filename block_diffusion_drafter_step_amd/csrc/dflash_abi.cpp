// C-ABI entry points of libdflash (declared in include/dflash.h).
//
// Every call validates all of its arguments on the host before it touches
// the GPU, so an invalid call has no side effects and needs no device; only
// then does it carve the caller's workspace and enqueue the kernels on the
// caller's stream.  Nothing here allocates, frees or synchronises.
#include "dflash.h"

#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>

#include "kernels.h"

using namespace dfl;

namespace {

thread_local char g_err[512] = "";

dflash_status fail(dflash_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

#define TRY(expr)                              \
  do {                                         \
    const dflash_status s_ = (expr);           \
    if (s_ != DFLASH_OK) return s_;            \
  } while (0)

dflash_status launched(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(DFLASH_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  g_err[0] = 0;
  return DFLASH_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

dflash_status need_ptr(const void *p, const char *name) {
  if (!p) return fail(DFLASH_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(DFLASH_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return DFLASH_OK;
}

dflash_status check_act(int32_t act) {
  if (act != DFLASH_F32 && act != DFLASH_BF16)
    return fail(DFLASH_ERR_INVALID_ARG, "act must be DFLASH_F32 or DFLASH_BF16 (got %d)", act);
  return DFLASH_OK;
}

// A projection weight: shape [rows][cols]; fp32 with fp32 activations, bf16
// or Q8_0 with bf16 activations (`allow_q8` false: the act type only).
dflash_status check_weight(const dflash_weight *w, const char *name, int64_t rows, int64_t cols,
                           int32_t act, bool allow_q8) {
  if (!w) return fail(DFLASH_ERR_INVALID_ARG, "%s is NULL", name);
  if (w->rows != rows || w->cols != cols)
    return fail(DFLASH_ERR_INVALID_ARG, "%s is [%lld][%lld], expected [%lld][%lld]", name,
                (long long)w->rows, (long long)w->cols, (long long)rows, (long long)cols);
  if (w->dtype == DFLASH_Q8_0) {
    if (!allow_q8) return fail(DFLASH_ERR_UNSUPPORTED, "%s cannot be Q8_0", name);
    if (act != DFLASH_BF16)
      return fail(DFLASH_ERR_INVALID_ARG, "%s: Q8_0 weights need bf16 activations", name);
    if (cols % 32) return fail(DFLASH_ERR_INVALID_ARG, "%s: Q8_0 needs cols %% 32 == 0", name);
    TRY(need_ptr(w->scales, "Q8_0 scales"));
  } else if (w->dtype != act) {
    return fail(DFLASH_ERR_INVALID_ARG, "%s: dtype %d does not match the activation type %d", name,
                w->dtype, act);
  }
  TRY(need_ptr(w->data, name));
  return DFLASH_OK;
}

dflash_status check_ws(void *ws, size_t ws_bytes, size_t need) {
  if (need == 0) return DFLASH_OK;
  if (!ws) return fail(DFLASH_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (!aligned16(ws)) return fail(DFLASH_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  if (ws_bytes < need)
    return fail(DFLASH_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  return DFLASH_OK;
}

// bump allocator over the caller's workspace (256-byte aligned pieces); the
// completion counters always come first
struct Carve {
  char *base;
  size_t off = 0;
  unsigned long long *counters;
  explicit Carve(void *p) : base((char *)p) { counters = (unsigned long long *)take(kCounterBytes); }
  void *take(size_t bytes) {
    void *p = base ? base + off : nullptr;
    off += (bytes + 255) & ~(size_t)255;
    return p;
  }
};

int wkind_of(const dflash_weight *w) { return w->dtype == DFLASH_Q8_0 ? W_Q8_0 : W_SAME; }

WSet wset(std::initializer_list<const dflash_weight *> ws) {
  WSet s;
  memset(&s, 0, sizeof s);
  int n = 0, tot = 0;
  for (const dflash_weight *w : ws) {
    s.data[n] = w->data;
    s.scales[n] = w->scales;
    s.rows[n] = (int)w->rows;
    tot += (int)w->rows;
    s.K = (int)w->cols;
    ++n;
  }
  s.n_seg = n;
  s.n_total = tot;
  return s;
}

ASrc asrc1(const void *p, int k) {
  ASrc a;
  memset(&a, 0, sizeof a);
  a.ptr[0] = p;
  a.n_src = 1;
  a.k_per_src = k;
  return a;
}

OutSpec out_f32(void *p, long ld) {
  OutSpec o;
  memset(&o, 0, sizeof o);
  o.mode = OUT_F32;
  o.out = p;
  o.ld = ld;
  return o;
}

OutSpec out_act(void *p, long ld, const void *resid, long ld_resid) {
  OutSpec o = out_f32(p, ld);
  o.mode = OUT_ACT;
  o.resid = resid;
  o.ld_resid = ld_resid;
  return o;
}

hipError_t gemm(int act, int wkind, const ASrc &A, int M, const WSet &W, float *part,
                unsigned long long *cnt, const OutSpec &o, hipStream_t st) {
  if (M <= kSkinnyMaxM) return launch_skinny_gemm(act, wkind, A, M, W, part, cnt, o, st);
  return launch_tile_gemm(act, wkind, A, M, W, o, part, st);
}

size_t gemm_partial_bytes(int M, int N, int K) {
  return (M <= kSkinnyMaxM ? skinny_partial_floats(N, K) : tile_partial_floats(M, N, K)) * sizeof(float);
}

constexpr int64_t kMaxRows = (int64_t)1 << 26;

// LM head: h resident in LDS (1) or the streaming kernel only (0)
#ifndef DFL_TOPK_RESIDENT
#define DFL_TOPK_RESIDENT 1
#endif

// --- workspace sizes (buffers in the act type are sized for fp32) --------------

// `z_off`, when given, receives z's offset
size_t inject_ws(int32_t n_layers, int64_t n, int32_t d_t, int32_t d, int32_t kv, size_t *z_off = nullptr) {
  Carve c(nullptr);
  c.take(std::max(gemm_partial_bytes((int)n, d, n_layers * d_t), gemm_partial_bytes((int)n, 2 * kv, d)));
  c.take((size_t)n * std::max(d, 2 * kv) * 4);  // y, then the fp32 K | V rows of a Q8_0 cache
  if (z_off) *z_off = c.off;
  c.take((size_t)n * d * 4);  // z
  if (n >= kQ8ExpandMinM) {   // bf16 expansions of Q8_0 fc, Wk and Wv
    c.take((size_t)d * n_layers * d_t * 2);
    c.take((size_t)kv * d * 2);
    c.take((size_t)kv * d * 2);
  }
  return c.off;
}

// partial sums of the conv's delta product (either form)
size_t conv_part_bytes(int M, int C, int G, int T) {
  return std::max(gemm_partial_bytes(M, T * G, C), conv_fused_part_bytes(M, C, G, T));
}

// The conv of dflash_conv and of the feed-forward site: at most 16 rows in
// one launch (delta formed inside), otherwise the delta GEMM then the conv.
hipError_t run_conv(int32_t act, const void *x, int n_blocks, int B, int C, int G, int T, const void *base,
                    const dflash_weight *w_delta, void *out, float *part, float *delta,
                    unsigned long long *counters, hipStream_t st) {
  const int M = n_blocks * B;
  if (conv_fused_ok(M, C, G, T))
    return launch_conv_fused(act, x, n_blocks, B, C, G, T, base, w_delta->data, out, part, counters, st);
  hipError_t e = gemm(act, W_SAME, asrc1(x, C), M, wset({w_delta}), part, counters, out_f32(delta, T * G), st);
  if (e != hipSuccess) return e;
  return launch_conv(act, x, n_blocks, B, C, G, T, base, delta, out, st);
}

size_t conv_ws(int32_t n_blocks, int32_t B, int32_t C, int32_t G, int32_t T) {
  Carve c(nullptr);
  const int64_t M = (int64_t)n_blocks * B;
  c.take(conv_part_bytes((int)M, C, G, T));
  c.take((size_t)M * T * G * 4);  // delta
  return c.off;
}

// `u_off` / `act_off`, when given, receive the offsets of u and act
size_t ffn_ws(int32_t n_blocks, int32_t B, int32_t d, int32_t G, int32_t T, int32_t d_ff,
              size_t *u_off = nullptr, size_t *act_off = nullptr) {
  Carve c(nullptr);
  const int64_t M = (int64_t)n_blocks * B;
  c.take(std::max(std::max(conv_part_bytes((int)M, d, G, T), gemm_partial_bytes((int)M, 2 * d_ff, d)),
                  gemm_partial_bytes((int)M, d, d_ff)));
  c.take((size_t)M * T * G * 4);       // delta
  if (u_off) *u_off = c.off;
  c.take((size_t)M * d * 4);           // u
  c.take((size_t)M * 2 * d_ff * 4);    // gate | up, fp32
  if (act_off) *act_off = c.off;
  c.take((size_t)M * d_ff * 4);        // act
  return c.off;
}

// `qkv_off` / `o_off`, when given, receive the offsets of Q | Kb | Vb and O
size_t attn_ws(int32_t B, int32_t d, int32_t Hq, int32_t Hkv, int32_t hd, int64_t n_ctx,
               size_t *qkv_off = nullptr, size_t *o_off = nullptr) {
  Carve c(nullptr);
  const int qdim = Hq * hd, kv = Hkv * hd;
  c.take(std::max(gemm_partial_bytes(B, qdim + 2 * kv, d), gemm_partial_bytes(B, d, qdim)));
  if (qkv_off) *qkv_off = c.off;
  c.take((size_t)B * (qdim + 2 * kv) * 4);  // Q | Kb | Vb
  const int n_split = attn_max_splits(n_ctx, Hkv);   // >= the plan's split count
  c.take((size_t)Hq * B * n_split * hd * 4);  // partial O
  c.take((size_t)Hq * B * n_split * 2 * 4);   // partial (max, sum)
  if (o_off) *o_off = c.off;
  c.take((size_t)B * qdim * 4);               // O
  return c.off;
}

size_t topk_ws(int64_t V, int32_t K) {
  Carve c(nullptr);
  // sized for the largest plan: streaming (bf16/fp32 or Q8_0 weights) or one
  // resident workgroup per CU
  const int n_wg = std::max(std::max(topk_plan_wgs(V, W_SAME), topk_plan_wgs(V, W_Q8_0)), kMaxCUs);
  c.take((size_t)n_wg * 16 * K * 4);
  c.take((size_t)n_wg * 16 * K * 4);
  c.take((size_t)n_wg * 16 * 2 * 4);
  return c.off;
}

size_t sel_ws(int32_t B, int32_t r, int32_t d) {
  Carve c(nullptr);
  c.take(std::max(gemm_partial_bytes(B, r, d), selector_part_bytes(r, d)));
  c.take((size_t)B * r * 4);
  return c.off;
}

dflash_status check_cache(const dflash_kv_cache *cache, int32_t act) {
  if (!cache) return fail(DFLASH_ERR_INVALID_ARG, "cache is NULL");
  if (cache->dtype == DFLASH_Q8_0) {
    if (act != DFLASH_BF16) return fail(DFLASH_ERR_INVALID_ARG, "a Q8_0 cache needs bf16 activations");
    if (cache->head_dim != 128)
      return fail(DFLASH_ERR_UNSUPPORTED, "a Q8_0 cache needs head_dim 128 (got %d)", cache->head_dim);
    TRY(need_ptr(cache->k_scales, "cache.k_scales"));
    TRY(need_ptr(cache->v_scales, "cache.v_scales"));
  } else if (cache->dtype != act) {
    return fail(DFLASH_ERR_INVALID_ARG, "cache dtype %d does not match the activation type %d",
                cache->dtype, act);
  }
  if (cache->head_dim != 64 && cache->head_dim != 128)
    return fail(DFLASH_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", cache->head_dim);
  if (cache->n_kv_heads < 1) return fail(DFLASH_ERR_INVALID_ARG, "n_kv_heads must be >= 1");
  if (cache->capacity < 1 || cache->capacity > kMaxRows)
    return fail(DFLASH_ERR_INVALID_ARG, "cache capacity out of range");
  if (cache->capacity % 64)
    return fail(DFLASH_ERR_INVALID_ARG, "cache capacity must be a multiple of 64 (got %lld)",
                (long long)cache->capacity);
  TRY(need_ptr(cache->k, "cache.k"));
  TRY(need_ptr(cache->v, "cache.v"));
  return DFLASH_OK;
}

}  // namespace

extern "C" {

const char *dflash_status_string(int32_t s) {
  switch (s) {
    case DFLASH_OK: return "ok";
    case DFLASH_ERR_INVALID_ARG: return "invalid argument";
    case DFLASH_ERR_UNSUPPORTED: return "unsupported";
    case DFLASH_ERR_CAPACITY: return "KV-cache capacity exceeded";
    case DFLASH_ERR_WORKSPACE: return "workspace missing or too small";
    case DFLASH_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

const char *dflash_last_error(void) { return g_err; }

int32_t dflash_version(void) { return 100; }

size_t dflash_inject_workspace(int32_t n_layers, int64_t n_tokens, int32_t d_t, int32_t d,
                               int32_t kv, int32_t act) {
  (void)act;
  if (n_layers < 1 || n_tokens < 1 || d_t < 1 || d < 1 || kv < 1) return 0;
  return inject_ws(n_layers, n_tokens, d_t, d, kv);
}

size_t dflash_inject_z_offset(int32_t n_layers, int64_t n_tokens, int32_t d_t, int32_t d, int32_t kv,
                              int32_t act) {
  (void)act;
  if (n_layers < 1 || n_tokens < 1 || d_t < 1 || d < 1 || kv < 1) return 0;
  size_t z = 0;
  inject_ws(n_layers, n_tokens, d_t, d, kv, &z);
  return z;
}

size_t dflash_block_attn_qkv_offset(int32_t B, int32_t d, int32_t n_q_heads, int32_t n_kv_heads,
                                    int32_t head_dim, int64_t n_ctx) {
  if (B < 1 || d < 1 || n_q_heads < 1 || n_kv_heads < 1 || head_dim < 1 || n_ctx < 0) return 0;
  size_t q = 0;
  attn_ws(B, d, n_q_heads, n_kv_heads, head_dim, n_ctx, &q, nullptr);
  return q;
}

size_t dflash_block_attn_o_offset(int32_t B, int32_t d, int32_t n_q_heads, int32_t n_kv_heads,
                                  int32_t head_dim, int64_t n_ctx) {
  if (B < 1 || d < 1 || n_q_heads < 1 || n_kv_heads < 1 || head_dim < 1 || n_ctx < 0) return 0;
  size_t o = 0;
  attn_ws(B, d, n_q_heads, n_kv_heads, head_dim, n_ctx, nullptr, &o);
  return o;
}

size_t dflash_conv_workspace(int32_t n_blocks, int32_t B, int32_t C, int32_t G, int32_t T) {
  if (n_blocks < 1 || B < 1 || C < 1 || G < 1 || T < 1) return 0;
  return conv_ws(n_blocks, B, C, G, T);
}

static bool ffn_args_ok(int32_t n_blocks, int32_t B, int32_t d, int32_t G, int32_t T, int32_t d_ff) {
  return n_blocks >= 1 && B >= 1 && d >= 1 && G >= 1 && T >= 1 && d_ff >= 1 &&
         (int64_t)n_blocks * B <= kMaxRows;
}

size_t dflash_ffn_block_workspace(int32_t n_blocks, int32_t B, int32_t d, int32_t G, int32_t T,
                                  int32_t d_ff) {
  if (!ffn_args_ok(n_blocks, B, d, G, T, d_ff)) return 0;
  return ffn_ws(n_blocks, B, d, G, T, d_ff);
}

size_t dflash_ffn_block_u_offset(int32_t n_blocks, int32_t B, int32_t d, int32_t G, int32_t T,
                                 int32_t d_ff) {
  if (!ffn_args_ok(n_blocks, B, d, G, T, d_ff)) return 0;
  size_t o = 0;
  ffn_ws(n_blocks, B, d, G, T, d_ff, &o, nullptr);
  return o;
}

size_t dflash_ffn_block_act_offset(int32_t n_blocks, int32_t B, int32_t d, int32_t G, int32_t T,
                                   int32_t d_ff) {
  if (!ffn_args_ok(n_blocks, B, d, G, T, d_ff)) return 0;
  size_t o = 0;
  ffn_ws(n_blocks, B, d, G, T, d_ff, nullptr, &o);
  return o;
}

size_t dflash_block_attn_workspace(int32_t B, int32_t d, int32_t n_q_heads, int32_t n_kv_heads,
                                   int32_t head_dim, int64_t n_ctx) {
  if (B < 1 || d < 1 || n_q_heads < 1 || n_kv_heads < 1 || head_dim < 1 || n_ctx < 0) return 0;
  return attn_ws(B, d, n_q_heads, n_kv_heads, head_dim, n_ctx);
}

size_t dflash_topk_unary_workspace(int32_t B, int64_t V, int32_t K) {
  (void)B;
  if (V < 1 || K < 1) return 0;
  return topk_ws(V, K);
}

size_t dflash_selector_edges_workspace(int32_t B, int32_t r, int32_t d, int32_t K) {
  (void)K;
  if (B < 1 || r < 1 || d < 1) return 0;
  return sel_ws(B, r, d);
}

// ---------------------------------------------------------------------------

dflash_status dflash_inject(const void *const *layer_hidden, int32_t n_layers, int64_t n_tokens,
                            int32_t d_t, int32_t act, const dflash_weight *fc, const void *gamma,
                            float eps, const dflash_weight *wk, const dflash_weight *wv,
                            const dflash_kv_cache *cache, int64_t pos0, void *ws, size_t ws_bytes,
                            void *stream) {
  TRY(check_act(act));
  if (!layer_hidden) return fail(DFLASH_ERR_INVALID_ARG, "layer_hidden is NULL");
  if (n_layers < 1 || n_layers > DFLASH_MAX_LAYERS)
    return fail(DFLASH_ERR_INVALID_ARG, "n_layers must be in [1, %d]", DFLASH_MAX_LAYERS);
  if (n_tokens < 1 || n_tokens > kMaxRows) return fail(DFLASH_ERR_INVALID_ARG, "n_tokens out of range");
  if (d_t < 64 || d_t % 64) return fail(DFLASH_ERR_INVALID_ARG, "d_t must be a positive multiple of 64");
  for (int l = 0; l < n_layers; ++l) TRY(need_ptr(layer_hidden[l], "layer_hidden[l]"));
  if (!fc) return fail(DFLASH_ERR_INVALID_ARG, "fc is NULL");
  const int64_t d = fc->rows;
  if (d < 64 || d % 64) return fail(DFLASH_ERR_INVALID_ARG, "d (fc rows) must be a positive multiple of 64");
  TRY(check_weight(fc, "fc", d, (int64_t)n_layers * d_t, act, true));
  TRY(check_cache(cache, act));
  const int64_t kv = (int64_t)cache->n_kv_heads * cache->head_dim;
  TRY(check_weight(wk, "wk", kv, d, act, true));
  TRY(check_weight(wv, "wv", kv, d, act, true));
  if (wk->dtype != wv->dtype) return fail(DFLASH_ERR_UNSUPPORTED, "wk and wv must share a dtype");
  if (gamma) TRY(need_ptr(gamma, "gamma"));
  if (!(eps >= 0.f)) return fail(DFLASH_ERR_INVALID_ARG, "eps must be >= 0");
  if (pos0 < 0 || pos0 + n_tokens > cache->capacity)
    return fail(DFLASH_ERR_CAPACITY, "rows [%lld, %lld) exceed capacity %lld", (long long)pos0,
                (long long)(pos0 + n_tokens), (long long)cache->capacity);
  const size_t need = inject_ws(n_layers, n_tokens, d_t, (int)d, (int)kv);
  TRY(check_ws(ws, ws_bytes, need));

  hipStream_t st = (hipStream_t)stream;
  Carve c(ws);
  const int n = (int)n_tokens;
  float *part = (float *)c.take(std::max(gemm_partial_bytes(n, (int)d, n_layers * d_t),
                                         gemm_partial_bytes(n, 2 * (int)kv, (int)d)));
  float *y = (float *)c.take((size_t)n * std::max<int64_t>(d, 2 * kv) * 4);
  void *z = c.take((size_t)n * d * 4);

  // many rows: Q8_0 weights are expanded once to bf16 in the workspace
  dflash_weight fc_e = *fc, wk_e = *wk, wv_e = *wv;
  hipError_t e = hipSuccess;
  if (n >= kQ8ExpandMinM) {
    dflash_weight *ex[3] = {&fc_e, &wk_e, &wv_e};
    for (dflash_weight *w : ex) {
      void *buf = c.take((size_t)w->rows * w->cols * 2);
      if (w->dtype != DFLASH_Q8_0) continue;
      e = launch_expand_q8(w->data, w->scales, w->rows, (int)w->cols, buf, st);
      if (e != hipSuccess) return launched(e, "Q8_0 expansion");
      w->dtype = DFLASH_BF16;
      w->data = buf;
      w->scales = nullptr;
    }
  }

  ASrc A;
  memset(&A, 0, sizeof A);
  for (int l = 0; l < n_layers; ++l) A.ptr[l] = layer_hidden[l];
  A.n_src = n_layers;
  A.k_per_src = d_t;
  e = gemm(act, wkind_of(&fc_e), A, n, wset({&fc_e}), part, c.counters, out_f32(y, d), st);
  if (e != hipSuccess) return launched(e, "fc");
  e = launch_rmsnorm(act, y, n, (int)d, gamma, eps, z, st);
  if (e != hipSuccess) return launched(e, "rmsnorm");
  if (cache->dtype == DFLASH_Q8_0) {
    // fp32 K | V rows into y (free once z exists), then codes and scales
    e = gemm(act, wkind_of(&wk_e), asrc1(z, (int)d), n, wset({&wk_e, &wv_e}), part, c.counters,
             out_f32(y, 2 * kv), st);
    if (e != hipSuccess) return launched(e, "wk/wv");
    e = launch_kv_quant(y, n, cache->n_kv_heads, cache->head_dim, cache->capacity, pos0, cache->k, cache->v,
                        cache->k_scales, cache->v_scales, st);
    return launched(e, "kv quantisation");
  }
  OutSpec oc;
  memset(&oc, 0, sizeof oc);
  oc.mode = OUT_CACHE;
  oc.ck = cache->k;
  oc.cv = cache->v;
  oc.hd = cache->head_dim;
  oc.split = (int)kv;
  oc.cap = cache->capacity;
  oc.pos0 = pos0;
  e = gemm(act, wkind_of(&wk_e), asrc1(z, (int)d), n, wset({&wk_e, &wv_e}), part, c.counters, oc, st);
  return launched(e, "wk/wv");
}

dflash_status dflash_conv(const void *x, int32_t n_blocks, int32_t B, int32_t C, int32_t G,
                          int32_t T, int32_t act, const void *base, const dflash_weight *w_delta,
                          void *out, void *ws, size_t ws_bytes, void *stream) {
  TRY(check_act(act));
  TRY(need_ptr(x, "x"));
  TRY(need_ptr(base, "base"));
  TRY(need_ptr(out, "out"));
  if (n_blocks < 1 || B < 1 || (int64_t)n_blocks * B > kMaxRows)
    return fail(DFLASH_ERR_INVALID_ARG, "n_blocks and B must be >= 1");
  if (B > DFLASH_MAX_BLOCK)
    return fail(DFLASH_ERR_INVALID_ARG, "B must be in [1, %d]", DFLASH_MAX_BLOCK);
  if (C < 64 || C % 64) return fail(DFLASH_ERR_INVALID_ARG, "C must be a positive multiple of 64");
  if (G < 1 || C % G) return fail(DFLASH_ERR_INVALID_ARG, "G must divide C");
  if (T < 1 || T > 16) return fail(DFLASH_ERR_INVALID_ARG, "T must be in [1, 16]");
  TRY(check_weight(w_delta, "w_delta", (int64_t)T * G, C, act, false));
  const size_t need = conv_ws(n_blocks, B, C, G, T);
  TRY(check_ws(ws, ws_bytes, need));

  hipStream_t st = (hipStream_t)stream;
  Carve c(ws);
  const int M = n_blocks * B;
  float *part = (float *)c.take(conv_part_bytes(M, C, G, T));
  float *delta = (float *)c.take((size_t)M * T * G * 4);
  return launched(run_conv(act, x, n_blocks, B, C, G, T, base, w_delta, out, part, delta, c.counters, st),
                  "conv");
}

dflash_status dflash_ffn_block(const void *h, int32_t n_blocks, int32_t B, int32_t d, int32_t G,
                               int32_t T, int32_t act, const void *base, const dflash_weight *w_delta,
                               const dflash_weight *w_gate, const dflash_weight *w_up,
                               const dflash_weight *w_down, void *out, void *ws, size_t ws_bytes,
                               void *stream) {
  TRY(check_act(act));
  TRY(need_ptr(h, "h"));
  TRY(need_ptr(base, "base"));
  TRY(need_ptr(out, "out"));
  if (out == h) return fail(DFLASH_ERR_INVALID_ARG, "out must not overlap h");
  if (n_blocks < 1 || B < 1 || (int64_t)n_blocks * B > kMaxRows)
    return fail(DFLASH_ERR_INVALID_ARG, "n_blocks and B must be >= 1");
  if (B > DFLASH_MAX_BLOCK)
    return fail(DFLASH_ERR_INVALID_ARG, "B must be in [1, %d]", DFLASH_MAX_BLOCK);
  if (d < 64 || d % 64) return fail(DFLASH_ERR_INVALID_ARG, "d must be a positive multiple of 64");
  if (G < 1 || d % G) return fail(DFLASH_ERR_INVALID_ARG, "G must divide d");
  if (T < 1 || T > 16) return fail(DFLASH_ERR_INVALID_ARG, "T must be in [1, 16]");
  TRY(check_weight(w_delta, "w_delta", (int64_t)T * G, d, act, false));
  if (!w_gate) return fail(DFLASH_ERR_INVALID_ARG, "w_gate is NULL");
  const int64_t d_ff = w_gate->rows;
  if (d_ff < 64 || d_ff % 64 || d_ff > (1 << 20))
    return fail(DFLASH_ERR_INVALID_ARG, "d_ff (w_gate rows) must be a positive multiple of 64, at most 2^20");
  TRY(check_weight(w_gate, "w_gate", d_ff, d, act, true));
  TRY(check_weight(w_up, "w_up", d_ff, d, act, true));
  TRY(check_weight(w_down, "w_down", d, d_ff, act, true));
  if (w_gate->dtype != w_up->dtype) return fail(DFLASH_ERR_UNSUPPORTED, "w_gate and w_up must share a dtype");
  const size_t need = ffn_ws(n_blocks, B, d, G, T, (int)d_ff);
  TRY(check_ws(ws, ws_bytes, need));

  hipStream_t st = (hipStream_t)stream;
  Carve c(ws);
  const int M = n_blocks * B, F = (int)d_ff;
  float *part = (float *)c.take(std::max(std::max(conv_part_bytes(M, d, G, T), gemm_partial_bytes(M, 2 * F, d)),
                                         gemm_partial_bytes(M, d, F)));
  float *delta = (float *)c.take((size_t)M * T * G * 4);
  void *u = c.take((size_t)M * d * 4);
  float *gu = (float *)c.take((size_t)M * 2 * F * 4);
  void *av = c.take((size_t)M * F * 4);
  // the feed-forward site's conv: the same kernels as dflash_conv
  hipError_t e = run_conv(act, h, n_blocks, B, d, G, T, base, w_delta, u, part, delta, c.counters, st);
  if (e != hipSuccess) return launched(e, "ffn conv");
  e = gemm(act, wkind_of(w_gate), asrc1(u, d), M, wset({w_gate, w_up}), part, c.counters, out_f32(gu, 2 * F), st);
  if (e != hipSuccess) return launched(e, "gate/up");
  e = launch_silu_mul(act, gu, M, F, av, st);
  if (e != hipSuccess) return launched(e, "silu");
  e = gemm(act, wkind_of(w_down), asrc1(av, F), M, wset({w_down}), part, c.counters, out_act(out, d, h, d), st);
  return launched(e, "down");
}

}  // extern "C"

// The block attention; with `cache_ready`, the stream waits for that event
// after the Q | Kb | Vb projection, before the first kernel that reads the
// cache.
static dflash_status block_attn(const void *u, const void *residual, int32_t B, int32_t d, int32_t n_q_heads,
                                int32_t act, const dflash_weight *wq, const dflash_weight *wk,
                                const dflash_weight *wv, const dflash_weight *wo,
                                const dflash_kv_cache *cache, int64_t n_ctx, float scale, void *out, void *ws,
                                size_t ws_bytes, void *stream, hipEvent_t cache_ready) {
  TRY(check_act(act));
  TRY(need_ptr(u, "u"));
  if (residual) TRY(need_ptr(residual, "residual"));
  TRY(need_ptr(out, "out"));
  if (B < 1 || B > DFLASH_MAX_BLOCK)
    return fail(DFLASH_ERR_INVALID_ARG, "B must be in [1, %d]", DFLASH_MAX_BLOCK);
  if (d < 64 || d % 64) return fail(DFLASH_ERR_INVALID_ARG, "d must be a positive multiple of 64");
  TRY(check_cache(cache, act));
  const int Hkv = cache->n_kv_heads, hd = cache->head_dim;
  if (n_q_heads < 1 || n_q_heads % Hkv)
    return fail(DFLASH_ERR_INVALID_ARG, "n_q_heads must be a positive multiple of n_kv_heads");
  if (n_q_heads / Hkv > 8) return fail(DFLASH_ERR_UNSUPPORTED, "at most 8 query heads per KV head");
  const int kvq = cache->dtype == DFLASH_Q8_0;
  if (kvq && !attn_q8_ok(hd, n_q_heads / Hkv, B))
    return fail(DFLASH_ERR_UNSUPPORTED, "a Q8_0 cache needs head_dim 128");
  const int64_t qdim = (int64_t)n_q_heads * hd, kv = (int64_t)Hkv * hd;
  TRY(check_weight(wq, "wq", qdim, d, act, true));
  TRY(check_weight(wk, "wk", kv, d, act, true));
  TRY(check_weight(wv, "wv", kv, d, act, true));
  TRY(check_weight(wo, "wo", d, qdim, act, true));
  if (wq->dtype != wk->dtype || wq->dtype != wv->dtype)
    return fail(DFLASH_ERR_UNSUPPORTED, "wq, wk and wv must share a dtype");
  if (n_ctx < 0 || n_ctx > cache->capacity)
    return fail(DFLASH_ERR_CAPACITY, "n_ctx %lld outside [0, capacity %lld]", (long long)n_ctx,
                (long long)cache->capacity);
  if (!(scale >= 0.f)) return fail(DFLASH_ERR_INVALID_ARG, "scale must be >= 0");
  const size_t need = attn_ws(B, d, n_q_heads, Hkv, hd, n_ctx);
  TRY(check_ws(ws, ws_bytes, need));

  hipStream_t st = (hipStream_t)stream;
  Carve c(ws);
  const int nqkv = (int)(qdim + 2 * kv);
  float *part = (float *)c.take(std::max(gemm_partial_bytes(B, nqkv, d), gemm_partial_bytes(B, d, (int)qdim)));
  void *qkv = c.take((size_t)B * nqkv * 4);
  AttnArgs a;
  memset(&a, 0, sizeof a);
  attn_plan_call(act, hd, n_q_heads / Hkv, B, kvq, n_ctx, Hkv, &a.chunk, &a.n_split);
  const int ns_max = attn_max_splits(n_ctx, Hkv);
  a.part_o = (float *)c.take((size_t)n_q_heads * B * ns_max * hd * 4);
  a.part_ml = (float *)c.take((size_t)n_q_heads * B * ns_max * 2 * 4);
  void *o = c.take((size_t)B * qdim * 4);

  hipError_t e = gemm(act, wkind_of(wq), asrc1(u, d), B, wset({wq, wk, wv}), part, c.counters,
                      out_act(qkv, nqkv, nullptr, 0), st);
  if (e != hipSuccess) return launched(e, "qkv");
  if (cache_ready) {
    e = hipStreamWaitEvent(st, cache_ready, 0);
    if (e != hipSuccess) return launched(e, "wait for the cache");
  }
  a.qkv = qkv;
  a.ck = cache->k;
  a.cv = cache->v;
  a.cks = cache->k_scales;
  a.cvs = cache->v_scales;
  a.kvq = kvq;
  a.cap = cache->capacity;
  a.n_ctx = n_ctx;
  a.B = B;
  a.Hq = n_q_heads;
  a.Hkv = Hkv;
  a.hd = hd;
  a.scale = scale > 0.f ? scale : 1.0f / sqrtf((float)hd);
  a.o = o;
  e = launch_attention(act, a, st);
  if (e != hipSuccess) return launched(e, "attention");
  e = gemm(act, wkind_of(wo), asrc1(o, (int)qdim), B, wset({wo}), part, c.counters, out_act(out, d, residual, d), st);
  return launched(e, "wo");
}

extern "C" {

dflash_status dflash_block_attn(const void *u, const void *residual, int32_t B, int32_t d,
                                int32_t n_q_heads, int32_t act, const dflash_weight *wq,
                                const dflash_weight *wk, const dflash_weight *wv,
                                const dflash_weight *wo, const dflash_kv_cache *cache,
                                int64_t n_ctx, float scale, void *out, void *ws, size_t ws_bytes,
                                void *stream) {
  return block_attn(u, residual, B, d, n_q_heads, act, wq, wk, wv, wo, cache, n_ctx, scale, out, ws, ws_bytes,
                    stream, nullptr);
}

dflash_status dflash_block_attn_after(const void *u, const void *residual, int32_t B, int32_t d,
                                      int32_t n_q_heads, int32_t act, const dflash_weight *wq,
                                      const dflash_weight *wk, const dflash_weight *wv,
                                      const dflash_weight *wo, const dflash_kv_cache *cache,
                                      int64_t n_ctx, float scale, void *out, void *ws, size_t ws_bytes,
                                      void *stream, void *cache_ready) {
  if (!cache_ready) return fail(DFLASH_ERR_INVALID_ARG, "cache_ready is NULL");
  return block_attn(u, residual, B, d, n_q_heads, act, wq, wk, wv, wo, cache, n_ctx, scale, out, ws, ws_bytes,
                    stream, (hipEvent_t)cache_ready);
}

}  // extern "C"

namespace {

dflash_status topk_check(const void *h, int32_t B, int32_t act, const dflash_weight *lm_head, int32_t K,
                         int32_t *idx, float *unary) {
  TRY(check_act(act));
  TRY(need_ptr(h, "h"));
  TRY(need_ptr(idx, "idx"));
  TRY(need_ptr(unary, "unary"));
  if (B < 1 || B > DFLASH_MAX_BLOCK)
    return fail(DFLASH_ERR_INVALID_ARG, "B must be in [1, %d]", DFLASH_MAX_BLOCK);
  if (!lm_head) return fail(DFLASH_ERR_INVALID_ARG, "lm_head is NULL");
  const int64_t V = lm_head->rows, d = lm_head->cols;
  if (d < 64 || d % 64) return fail(DFLASH_ERR_INVALID_ARG, "d must be a positive multiple of 64");
  if (V < 1 || V >= ((int64_t)1 << 31)) return fail(DFLASH_ERR_INVALID_ARG, "V out of range");
  TRY(check_weight(lm_head, "lm_head", V, d, act, true));
  if (K < 1 || K > DFLASH_MAX_TOPK || K > V)
    return fail(DFLASH_ERR_INVALID_ARG, "K must be in [1, min(V, %d)]", DFLASH_MAX_TOPK);
  return DFLASH_OK;
}

// the LM head's arguments, its partial lists carved from `c`
TopkArgs topk_setup(const void *h, int32_t B, int32_t act, const dflash_weight *lm_head, int32_t K,
                    int32_t *idx, float *unary, Carve &c) {
  const int64_t V = lm_head->rows, d = lm_head->cols;
  TopkArgs a;
  memset(&a, 0, sizeof a);
  a.h = h;
  a.B = B;
  a.d = (int)d;
  a.w = lm_head->data;
  a.scales = lm_head->scales;
  a.V = V;
  a.K = K;
  const size_t lds = topk_lds_bytes(B, (int)d, act, K);
  const int cus = std::min(device_cu_count(), kMaxCUs);
  // resident path for bf16 / fp32 heads (measured faster there); Q8_0 heads
  // stream (their dequantisation favours more waves)
  if (DFL_TOPK_RESIDENT && lds <= kMaxLdsBytes && d % 128 == 0 &&
      (long)cus * topk_lds_waves() <= (V + 15) / 16) {
    a.lds_path = 1;
    a.lds_bytes = (int)lds;
    a.n_wg = cus;
    a.n_waves = cus * topk_lds_waves();
  } else {
    a.lds_path = 0;
    a.n_wg = topk_plan_wgs(V, wkind_of(lm_head));
    a.n_waves = topk_plan_waves(V, wkind_of(lm_head));
  }
  a.part_val = (float *)c.take((size_t)a.n_wg * 16 * K * 4);
  a.part_idx = (int *)c.take((size_t)a.n_wg * 16 * K * 4);
  a.part_ms = (float *)c.take((size_t)a.n_wg * 16 * 2 * 4);
  a.idx = idx;
  a.unary = unary;
  return a;
}

// carve `ws` (at least topk_ws(V, K) bytes) and enqueue the LM head + merge
dflash_status topk_enqueue(const void *h, int32_t B, int32_t act, const dflash_weight *lm_head, int32_t K,
                           int32_t *idx, float *unary, void *ws, void *stream) {
  Carve c(ws);
  const TopkArgs a = topk_setup(h, B, act, lm_head, K, idx, unary, c);
  return launched(launch_topk(act, wkind_of(lm_head), a, (hipStream_t)stream), "topk");
}

dflash_status sel_check(const void *h, int32_t B, int32_t act, const dflash_weight *proj, const void *cb_pred,
                        const void *cb_succ, int64_t V, const int32_t *idx, const float *unary, int32_t K,
                        int32_t anchor, float *edges, int32_t *path, const int32_t *target, int32_t *accept) {
  TRY(check_act(act));
  TRY(need_ptr(h, "h"));
  TRY(need_ptr(cb_pred, "cb_pred"));
  TRY(need_ptr(cb_succ, "cb_succ"));
  TRY(need_ptr(idx, "idx"));
  TRY(need_ptr(unary, "unary"));
  TRY(need_ptr(edges, "edges"));
  TRY(need_ptr(path, "path"));
  if ((target == nullptr) != (accept == nullptr))
    return fail(DFLASH_ERR_INVALID_ARG, "target and accept must be both given or both NULL");
  if (target) {
    TRY(need_ptr(target, "target"));
    TRY(need_ptr(accept, "accept"));
  }
  if (B < 1 || B > DFLASH_MAX_BLOCK)
    return fail(DFLASH_ERR_INVALID_ARG, "B must be in [1, %d]", DFLASH_MAX_BLOCK);
  if (K < 1 || K > DFLASH_MAX_TOPK)
    return fail(DFLASH_ERR_INVALID_ARG, "K must be in [1, %d]", DFLASH_MAX_TOPK);
  if (!proj) return fail(DFLASH_ERR_INVALID_ARG, "proj is NULL");
  const int64_t r = proj->rows, d = proj->cols;
  if (r < 16 || r % 16 || r > 256) return fail(DFLASH_ERR_INVALID_ARG, "r must be a multiple of 16 in [16, 256]");
  if (d < 64 || d % 64) return fail(DFLASH_ERR_INVALID_ARG, "d must be a positive multiple of 64");
  TRY(check_weight(proj, "proj", r, d, act, false));
  if (V < K || V >= ((int64_t)1 << 31)) return fail(DFLASH_ERR_INVALID_ARG, "V must be in [K, 2^31)");
  if (anchor < -1 || anchor >= V) return fail(DFLASH_ERR_INVALID_ARG, "anchor must be in [-1, V)");
  return DFLASH_OK;
}

// the selector's arguments, its buffers carved from `c` (sel_ws bytes)
SelArgs sel_setup(const void *h, int32_t B, const dflash_weight *proj, const void *cb_pred, const void *cb_succ,
                  int64_t V, const int32_t *idx, const float *unary, int32_t K, int32_t anchor, float *edges,
                  int32_t *path, const int32_t *target, int32_t *accept, Carve &c, float **pj) {
  const int64_t r = proj->rows, d = proj->cols;
  SelArgs a;
  memset(&a, 0, sizeof a);
  a.part = (float *)c.take(std::max(gemm_partial_bytes(B, (int)r, (int)d), selector_part_bytes((int)r, (int)d)));
  *pj = (float *)c.take((size_t)B * r * 4);
  a.cb_pred = cb_pred;
  a.cb_succ = cb_succ;
  a.V = V;
  a.r = (int)r;
  a.B = B;
  a.K = K;
  a.anchor = anchor;
  a.idx = idx;
  a.unary = unary;
  a.edges = edges;
  a.path = path;
  a.target = target;
  a.accept = accept;
  a.h = h;
  a.pw = proj->data;
  a.d = (int)d;
  a.cnt = c.counters;
  return a;
}

// the selector (projection, edges, path, accept) on arguments from sel_setup
dflash_status sel_enqueue(int32_t act, SelArgs a, const dflash_weight *proj, float *pj, hipStream_t st) {
  if (selector_fused_fits(act, a)) {
    // one launch: the projection is formed inside the selector kernel
    selector_fused_plan(a);
    a.fused = true;
    if (a.n_wg > 1) a.stamp = next_launch_stamp();
    return launched(launch_selector(act, a, st), "selector");
  }
  hipError_t e = gemm(act, W_SAME, asrc1(a.h, a.d), a.B, wset({proj}), a.part, a.cnt, out_f32(pj, a.r), st);
  if (e != hipSuccess) return launched(e, "project");
  a.proj = pj;
  return launched(launch_selector(act, a, st), "selector");
}

size_t topk_select_ws(int32_t B, int64_t V, int32_t K, int32_t r, int32_t d) {
  return topk_ws(V, K) + sel_ws(B, r, d);
}

static_assert(DFLASH_TOPK_NOALLOC_SCRATCH_BYTES == kTopkScratchBytes, "header and library agree");

}  // namespace

extern "C" {

dflash_status dflash_topk_unary(const void *h, int32_t B, int32_t act,
                                const dflash_weight *lm_head, int32_t K, int32_t *idx,
                                float *unary, void *ws, size_t ws_bytes, void *stream) {
  TRY(topk_check(h, B, act, lm_head, K, idx, unary));
  TRY(check_ws(ws, ws_bytes, topk_ws(lm_head->rows, K)));
  return topk_enqueue(h, B, act, lm_head, K, idx, unary, ws, stream);
}

dflash_status dflash_topk_unary_noalloc(const void *h, int32_t B, int32_t act,
                                        const dflash_weight *lm_head, int32_t K, int32_t *idx,
                                        float *unary, void *stream) {
  TRY(topk_check(h, B, act, lm_head, K, idx, unary));
  const size_t need = topk_ws(lm_head->rows, K);
  if (need > kTopkScratchBytes)
    return fail(DFLASH_ERR_UNSUPPORTED,
                "V = %lld, K = %d needs %zu bytes of scratch, more than the %zu of the static array",
                (long long)lm_head->rows, K, need, kTopkScratchBytes);
  void *ws = nullptr;
  const hipError_t e = topk_scratch_ptr(&ws);
  if (e != hipSuccess) return fail(DFLASH_ERR_LAUNCH, "static scratch: %s", hipGetErrorString(e));
  return topk_enqueue(h, B, act, lm_head, K, idx, unary, ws, stream);
}

dflash_status dflash_selector_edges(const void *h, int32_t B, int32_t act,
                                    const dflash_weight *proj, const void *cb_pred,
                                    const void *cb_succ, int64_t V, const int32_t *idx,
                                    const float *unary, int32_t K, int32_t anchor, float *edges,
                                    int32_t *path, const int32_t *target, int32_t *accept, void *ws,
                                    size_t ws_bytes, void *stream) {
  TRY(sel_check(h, B, act, proj, cb_pred, cb_succ, V, idx, unary, K, anchor, edges, path, target, accept));
  TRY(check_ws(ws, ws_bytes, sel_ws(B, (int)proj->rows, (int)proj->cols)));
  Carve c(ws);
  float *pj;
  const SelArgs a = sel_setup(h, B, proj, cb_pred, cb_succ, V, idx, unary, K, anchor, edges, path, target, accept,
                              c, &pj);
  return sel_enqueue(act, a, proj, pj, (hipStream_t)stream);
}

size_t dflash_topk_select_workspace(int32_t B, int64_t V, int32_t K, int32_t r, int32_t d) {
  if (B < 1 || B > DFLASH_MAX_BLOCK || V < 1 || V >= ((int64_t)1 << 31) || K < 1 || K > DFLASH_MAX_TOPK ||
      K > V || r < 16 || r % 16 || r > 256 || d < 64 || d % 64)
    return 0;
  return topk_select_ws(B, V, K, r, d);
}

dflash_status dflash_topk_select(const void *h, int32_t B, int32_t act, const dflash_weight *lm_head,
                                 int32_t K, const dflash_weight *proj, const void *cb_pred,
                                 const void *cb_succ, int32_t anchor, int32_t *idx, float *unary,
                                 float *edges, int32_t *path, const int32_t *target, int32_t *accept,
                                 void *ws, size_t ws_bytes, void *stream) {
  TRY(topk_check(h, B, act, lm_head, K, idx, unary));
  const int64_t V = lm_head->rows;
  TRY(sel_check(h, B, act, proj, cb_pred, cb_succ, V, idx, unary, K, anchor, edges, path, target, accept));
  if (proj->cols != lm_head->cols) return fail(DFLASH_ERR_INVALID_ARG, "proj and lm_head must share d");
  TRY(check_ws(ws, ws_bytes, topk_select_ws(B, V, K, (int)proj->rows, (int)proj->cols)));
  hipStream_t st = (hipStream_t)stream;
  Carve c(ws);
  const TopkArgs ta = topk_setup(h, B, act, lm_head, K, idx, unary, c);
  float *pj;
  SelArgs a = sel_setup(h, B, proj, cb_pred, cb_succ, V, idx, unary, K, anchor, edges, path, target, accept, c,
                        &pj);
  if (topk_select_ok(act, ta, a)) {
    // the LM head's partial lists, then its merge and the selector in one launch
    selector_fused_plan(a);
    a.fused = true;
    a.stamp = next_launch_stamp();
    hipError_t e = launch_topk_partials(act, wkind_of(lm_head), ta, st);
    if (e != hipSuccess) return launched(e, "topk");
    return launched(launch_topk_select(act, ta, a, st), "topk + selector");
  }
  TRY(launched(launch_topk(act, wkind_of(lm_head), ta, st), "topk"));
  return sel_enqueue(act, a, proj, pj, st);
}

size_t dflash_topk_rows_workspace(int64_t n_rows, int64_t n_cols, int32_t K) {
  if (n_rows < 1 || n_cols < 1 || K < 1 || K > DFLASH_MAX_ROW_TOPK || K > n_cols) return 0;
  size_t a, b;
  rowtopk_plan((long)n_rows, (long)n_cols, K, &a, &b);
  Carve c(nullptr);
  c.take(a);
  c.take(b);
  return c.off;
}

dflash_status dflash_topk_rows(const float *x, int64_t n_rows, int64_t n_cols, int32_t K, int32_t *idx,
                               float *val, void *ws, size_t ws_bytes, void *stream) {
  TRY(need_ptr(x, "x"));
  TRY(need_ptr(idx, "idx"));
  TRY(need_ptr(val, "val"));
  if (n_rows < 1 || n_rows > 65535) return fail(DFLASH_ERR_INVALID_ARG, "n_rows must be in [1, 65535]");
  if (n_cols < 1 || n_cols > INT32_MAX) return fail(DFLASH_ERR_INVALID_ARG, "n_cols must be in [1, 2^31)");
  if (K < 1 || K > DFLASH_MAX_ROW_TOPK || K > n_cols)
    return fail(DFLASH_ERR_INVALID_ARG, "K must be in [1, min(n_cols, %d)]", DFLASH_MAX_ROW_TOPK);
  size_t a, b;
  rowtopk_plan((long)n_rows, (long)n_cols, K, &a, &b);
  Carve probe(nullptr);
  probe.take(a);
  probe.take(b);
  TRY(check_ws(ws, ws_bytes, probe.off));
  Carve c(ws);
  void *buf_a = c.take(a);
  void *buf_b = c.take(b);
  return launched(launch_rowtopk(x, (long)n_rows, (long)n_cols, K, idx, val, buf_a, buf_b,
                                 (hipStream_t)stream),
                  "topk_rows");
}

dflash_status dflash_accept_len(const int32_t *draft, const int32_t *target, int32_t n_seq,
                                int32_t B, int32_t *accept, void *stream) {
  TRY(need_ptr(draft, "draft"));
  TRY(need_ptr(target, "target"));
  TRY(need_ptr(accept, "accept"));
  if (n_seq < 1 || B < 1) return fail(DFLASH_ERR_INVALID_ARG, "n_seq and B must be >= 1");
  return launched(launch_accept(draft, target, n_seq, B, accept, (hipStream_t)stream), "accept");
}

}  // extern "C"
