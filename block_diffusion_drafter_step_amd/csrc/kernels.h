// Host-side launchers of the libdflash kernels and the plain structs that
// describe their operands.  Included by the kernel sources and by the C-ABI
// layer; nothing here is exported.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dfl {

enum ActType { ACT_F32 = 0, ACT_BF16 = 1 };
enum WKind { W_SAME = 0, W_Q8_0 = 1 };  // weight stored in the act type, or Q8_0

constexpr int kMaxSrc = 16;  // K-concatenated activation sources
constexpr int kMaxSeg = 3;   // N-concatenated weights

// Activation operand [M][K] given as up to kMaxSrc arrays [M][k_per_src]
// side by side along K (the concatenation is never materialised).
struct ASrc {
  const void *ptr[kMaxSrc];
  int n_src;
  int k_per_src;  // columns of each array; K = n_src * k_per_src
};

// Up to kMaxSeg weights [rows_s][K] stacked along N (rows 0..rows_0-1 are
// weight 0, and so on).  All share K and the storage kind.
struct WSet {
  const void *data[kMaxSeg];
  const void *scales[kMaxSeg];  // Q8_0: fp16 [rows][K/32]
  int rows[kMaxSeg];
  int n_seg;
  int n_total;
  int K;
};

// Where a GEMM's fp32 result Y[t][n] goes.
enum OutMode {
  OUT_F32 = 0,    // float out[t * ld + col0 + n]
  OUT_ACT = 1,    // act out[t * ld + col0 + n] = round(Y + resid[t * ld_resid + n])
  OUT_CACHE = 2   // n < split -> K cache, else V cache; head n / hd, row pos0 + t
};

struct OutSpec {
  int mode;
  void *out;
  long ld;
  long col0;
  const void *resid;  // OUT_ACT: optional residual in the act type
  long ld_resid;
  void *ck;
  void *cv;
  int hd;
  int split;          // OUT_CACHE: columns that go to K
  long cap;
  long pos0;
};

// ---- GEMM family -----------------------------------------------------------

// Rows of the weight-streaming path: M <= 16 activation rows.
constexpr int kSkinnyMaxM = 16;

// Completion counters at the start of every workspace: 64-bit words stamped
// by the launch that uses them, so they need no initial value.
constexpr int kMaxCounters = 8192;
// stamp of the next launch that uses completion counters (48 bits, never 0)
unsigned long long next_launch_stamp();
constexpr size_t kCounterBytes = kMaxCounters * sizeof(unsigned long long);

// Workspace floats of the split-K partials of a skinny GEMM.
size_t skinny_partial_floats(int n_total, int K);
// Y = X . W^T for M <= 16 rows: split-K partials summed in a fixed order by
// the last workgroup of each tile group (counters `cnt`, kMaxCounters of
// them), or by a second kernel when there are more tile groups than
// counters.  `part` holds skinny_partial_floats() floats.
hipError_t launch_skinny_gemm(int act, int wkind, const ASrc &X, int M, const WSet &W, float *part,
                              unsigned long long *cnt, const OutSpec &out, hipStream_t st);
// Y = A . W^T for any M (tiled MFMA GEMMs, LDS-staged).  When the 128 x 128
// tile grid would leave CUs idle (few rows), the k-range is split and `part`
// (tile_partial_floats() floats) holds the fp32 partials; part == nullptr
// never splits.
hipError_t launch_tile_gemm(int act, int wkind, const ASrc &A, int M, const WSet &W,
                            const OutSpec &out, float *part, hipStream_t st);
size_t tile_partial_floats(int M, int N, int K);

// Products with at least this many activation rows expand a Q8_0 weight once
// into bf16 (the same values the in-kernel dequantisation produces) and run
// the bf16 direct-to-LDS GEMMs: every row tile would otherwise decode the
// whole weight again (measured break-even near 640 rows of the 32k Q8_0 layer).
#ifndef DFL_Q8_EXPAND_MIN_M
#define DFL_Q8_EXPAND_MIN_M 768
#endif
constexpr int kQ8ExpandMinM = DFL_Q8_EXPAND_MIN_M;
// out[r][c] = bf16_rne(fp32(scales[r][c/32]) * codes[r][c]), cols % 32 == 0
hipError_t launch_expand_q8(const void *codes, const void *scales, long rows, int cols, void *out,
                            hipStream_t st);

// ---- injection -----------------------------------------------------------------
// z[t] = round(y[t] / sqrt(mean(y[t]^2) + eps) * gamma), y fp32 [n][d].
hipError_t launch_rmsnorm(int act, const float *y, int n, int d, const void *gamma, float eps,
                          void *z, hipStream_t st);

// Q8_0 cache rows from fp32 K | V rows kv [n][2 * Hkv * hd] (K columns first):
// per (row, head, 32-dim block) scale = fp16(max|x| / 127), codes
// round-half-away(x / (max|x| / 127)); K codes [Hkv][cap][hd], V codes in
// transposed 32-position panels, scales [Hkv][cap][hd / 32].
hipError_t launch_kv_quant(const float *kv, int n, int Hkv, int hd, long cap, long pos0, void *ck,
                           void *cv, void *cks, void *cvs, hipStream_t st);

// ---- conv ------------------------------------------------------------------------
// out[b][i][c] = sum_t (base[t][c] + delta[b*B + i][t*G + g(c)]) * x[b][i - t][c]
// act [M][F] = silu(gu[:, :F]) * gu[:, F:] in the act type, gu fp32 [M][2F],
// F % 4 == 0.
hipError_t launch_silu_mul(int act, const float *gu, long M, int F, void *out, hipStream_t st);
hipError_t launch_conv(int act, const void *x, int n_blocks, int B, int C, int G, int T,
                       const void *base, const float *delta, void *out, hipStream_t st);
// The whole conv of at most 16 rows (n_blocks * B <= 16, (C / G) % 4 == 0)
// in one launch: delta = x . W_delta^T is formed per tile of groups and the
// last workgroup of a tile applies the taps to the tile's columns.
// conv_fused_ok says whether it applies, conv_fused_part_bytes the
// partial-sum space it needs.  wd: W_delta [T*G][C] in the act type; cnt:
// completion counters.
bool conv_fused_ok(int M, int C, int G, int T);
size_t conv_fused_part_bytes(int M, int C, int G, int T);
hipError_t launch_conv_fused(int act, const void *x, int n_blocks, int B, int C, int G, int T,
                             const void *base, const void *wd, void *out, float *part,
                             unsigned long long *cnt, hipStream_t st);

// ---- attention ---------------------------------------------------------------------
struct AttnArgs {
  const void *qkv;   // [B][Hq*hd + 2*Hkv*hd] in the act type: Q | Kb | Vb
  const void *ck;    // cache [Hkv][cap][hd]
  const void *cv;
  const void *cks;   // Q8_0 cache: fp16 scales [Hkv][cap][hd/32] of K and V
  const void *cvs;
  int kvq;           // 1: the cache holds Q8_0 codes
  long cap;
  long n_ctx;
  int B, Hq, Hkv, hd;
  float scale;
  int chunk;         // keys per split
  int n_split;
  float *part_o;     // [Hq][B][n_split][hd]
  float *part_ml;    // [Hq][B][n_split][2]
  void *o;           // [B][Hq*hd] in the act type
};
// keys per split workgroup and split count; `streams` from attn_streams()
void attn_plan(long n_keys, int Hkv, int streams, int *chunk, int *n_split);
int attn_streams(int act, int hd);
// the plan of the split kernel launch_attention picks for these shapes
void attn_plan_call(int act, int hd, int grp, int B, int kvq, long n_keys, int Hkv, int *chunk,
                    int *n_split);
// Q8_0 caches: head_dim 128 (and at most 8 query heads per KV head)
bool attn_q8_ok(int hd, int grp, int B);
int attn_max_splits(long n_keys, int Hkv);
hipError_t launch_attention(int act, const AttnArgs &a, hipStream_t st);

// ---- LM head top-K -------------------------------------------------------------------
struct TopkArgs {
  const void *h;      // [B][d] in the act type
  int B, d;
  const void *w;      // [V][d] codes or values
  const void *scales; // Q8_0 scales or null
  long V;
  int K;
  int n_wg;
  int n_waves;        // waves that own vocabulary tiles (<= 4 * n_wg)
  int lds_path;       // 1: h resident in LDS, one persistent workgroup per CU
  int lds_bytes;      // dynamic LDS of the resident path
  float *part_val;    // [16][K][n_wg]
  int *part_idx;      // [16][K][n_wg]
  float *part_ms;     // [16][2][n_wg]
  int *idx;           // [B][K]
  float *unary;       // [B][K]
};
int topk_plan_wgs(long V, int wkind);
// LDS bytes of the h-resident LM-head kernel (h block or merge arrays) and
// its waves per workgroup
size_t topk_lds_bytes(int B, int d, int act, int K);
int topk_lds_waves();
constexpr size_t kMaxLdsBytes = 160 * 1024;
// Allows `bytes` of dynamic LDS for kernel `k`.  An error -- the kernel's
// static LDS and `bytes` together over a CU's 160 KB, or the runtime's own --
// means the kernel must not be launched.
hipError_t allow_dynamic_lds(const void *k, size_t bytes);
constexpr int kMaxCUs = 1024;
int device_cu_count();
int topk_plan_waves(long V, int wkind);
hipError_t launch_topk(int act, int wkind, const TopkArgs &a, hipStream_t st);
// The no-allocation LM-head call's static scratch: its size (the workspace
// of K <= 32 for any vocabulary whose plan has at most kMaxCUs workgroups,
// i.e. V <= 2^20) and the current device's address of it.
constexpr size_t kTopkScratchBytes = 4390912;
hipError_t topk_scratch_ptr(void **out);

// ---- row-wise top-K of an fp32 matrix (K <= 1024) -----------------------------------
// bytes of the two candidate-key buffers the passes alternate between
void rowtopk_plan(long n_rows, long n_cols, int K, size_t *buf_a, size_t *buf_b);
hipError_t launch_rowtopk(const float *x, long n_rows, long n_cols, int K, int32_t *idx, float *val,
                          void *buf_a, void *buf_b, hipStream_t st);

// ---- selector ------------------------------------------------------------------------
struct SelArgs {
  const float *proj;  // [B][r] fp32 (two-kernel path: formed by a GEMM beforehand)
  const void *cb_pred, *cb_succ;  // [V][r] act type
  long V;
  int r, B, K, anchor;
  const int *idx;
  const float *unary;
  float *edges;       // [B][K][K]
  int *path;          // [B]
  const int *target;  // [B] or null: accept = length of the prefix where path == target
  int *accept;        // [1] or null
  // one-launch path: proj = h . P^T is formed inside the selector kernel
  bool fused;
  const void *h, *pw;  // [B][d], [r][d] act type
  int d, pieces, n_wg; // 128-wide k-pieces per wave; workgroups (k-slices)
  float *part;         // [n_wg][r/16][64] float4 partial projections
  unsigned long long *cnt, stamp;   // completion counter (n_wg > 1)
};
// Whether the one-launch selector (projection inside) fits in LDS; if so,
// selector_fused_plan fills pieces and n_wg from B, K, r and d.
bool selector_fused_fits(int act, const SelArgs &a);
void selector_fused_plan(SelArgs &a);
size_t selector_part_bytes(int r, int d);
hipError_t launch_selector(int act, const SelArgs &a, hipStream_t st);
// The LM head's partial lists only (the h-resident kernel, K <= 8); their
// merge is left to launch_topk_select.
hipError_t launch_topk_partials(int act, int wkind, const TopkArgs &a, hipStream_t st);
// The LM head's final merge and the one-launch selector in one kernel, after
// launch_topk_partials: applies when topk_select_ok; `a` planned by
// selector_fused_plan, with its counter and a fresh stamp.
bool topk_select_ok(int act, const TopkArgs &ta, const SelArgs &a);
hipError_t launch_topk_select(int act, const TopkArgs &ta, const SelArgs &a, hipStream_t st);

hipError_t launch_accept(const int *draft, const int *target, int n_seq, int B, int *accept,
                         hipStream_t st);

}  // namespace dfl
