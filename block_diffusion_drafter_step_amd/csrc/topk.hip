// Shared LM head with top-K candidates and log-softmax unary scores
// ("Turbo dflash", Overview: the draft uses the target's output matrix;
// "spec : add DFlash2 support", Overview: the unary term of an edge is the
// draft's log-softmax score of the candidate; and the top-k review: small K over a very wide row).
//
// The logits l = h . W_lm^T are never stored.  The LM head weight is by far
// the largest stream of the block step, so the first kernel streams it once:
// each wave owns a contiguous range of vocabulary rows, computes 32 rows x 16
// tokens per pass with 16x16x32 MFMAs (weight fragments straight from HBM into
// registers), and folds the 4 logits each lane receives into
//   * a per-lane running (max, sum of exp) for the log-sum-exp, and
//   * a per-lane sorted top-KM list (KM >= K), rows visited in increasing
//     order so a strict '>' keeps the lower index first on equal logits.
// The 16 lists of a token in a workgroup are merged in LDS and one partial
// (top-K, max, sum) per token per workgroup is written.  A second kernel
// merges the partials in a fixed order: deterministic, and the ordering is
// (logit descending, index ascending) throughout.
#include <mutex>

#include "common.h"
#include "kernels.h"
#include "stream.h"
#include "merge.h"

namespace dfl {


__device__ __forceinline__ bool better(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

// insert (x, r) into a list sorted by `better`; r is larger than every index
// already in the list, so equal values stay behind the earlier entries
template <int KM>
__device__ __forceinline__ void list_insert(float (&v)[KM], int (&ix)[KM], float x, int r) {
  if (x > v[KM - 1]) {
    v[KM - 1] = x;
    ix[KM - 1] = r;
#pragma unroll
    for (int j = KM - 1; j > 0; --j) {
      const bool sw = v[j] > v[j - 1];
      const float tv = v[j - 1];
      const int ti = ix[j - 1];
      v[j - 1] = sw ? v[j] : tv;
      ix[j - 1] = sw ? ix[j] : ti;
      v[j] = sw ? tv : v[j];
      ix[j] = sw ? ti : ix[j];
    }
  }
}

// Merge the 16 per-lane lists of each token in a workgroup (4 lane groups x
// 4 waves) and write the workgroup's partial (top-K, max, sum of exp) per token.
// Thread (token = tid / 16, list q = tid % 16) offers its list's head; a
// 16-lane argmax by (value desc, index asc) picks the next entry K times.
template <int KM, int NW = 4>
__device__ __forceinline__ void wg_merge_write(const float (&tv)[KM], const int (&ti)[KM], float m,
                                               float ssum, const TopkArgs &a, float *lv, int *li,
                                               float *lm, float *ls) {
  constexpr int LQ = 4 * NW;   // lists per token: 4 lane groups per wave
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    lv[tid * KM + j] = tv[j];
    li[tid * KM + j] = ti[j];
  }
  lm[tid] = m;
  ls[tid] = ssum;
  __syncthreads();
  const int tok = tid / LQ, q = tid % LQ;
  // list q of token tok was written by thread (q/4)*64 + (q%4)*16 + tok
  const int src = (q >> 2) * 64 + (q & 3) * 16 + tok;
  const float pm = lm[src];
  float M = pm;
#pragma unroll
  for (int o = 1; o < LQ; o <<= 1) M = fmaxf(M, shfl_xor(M, o));
  float ps = ls[src] > 0.f ? ls[src] * exp2f((pm - M) * kL2e) : 0.f;
#pragma unroll
  for (int o = 1; o < LQ; o <<= 1) ps += shfl_xor(ps, o);
  const int wg = blockIdx.x;
  if (q == 0) {
    a.part_ms[part_at(a, tok, 0, 2, wg)] = M;
    a.part_ms[part_at(a, tok, 1, 2, wg)] = ps;
  }
  int head = 0;
  for (int k = 0; k < a.K; ++k) {
    float bv = head < KM ? lv[src * KM + head] : -__builtin_inff();
    int bi = head < KM ? li[src * KM + head] : 0x7fffffff;
    int bq = q;
#pragma unroll
    for (int o = 1; o < LQ; o <<= 1) {
      const float ov = shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o, kWave);
      const int oq = __shfl_xor(bq, o, kWave);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
        bq = oq;
      }
    }
    if (bq == q) ++head;
    if (q == 0) {
      a.part_val[part_at(a, tok, k, a.K, wg)] = bv;
      a.part_idx[part_at(a, tok, k, a.K, wg)] = bi;
    }
  }
}

// Fold one 16-row tile's logits (lane: rows row0 + 4g + i of token r16) into
// the running (max, sum of exp) and the sorted top-KM list.
template <int KM>
__device__ __forceinline__ void fold_tile(const f32x4 &acc, long row0, long V, int g, float &m,
                                          float &ssum, float (&tv)[KM], int (&ti)[KM]) {
  float v[4];
  float tmax = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const long row = row0 + 4 * g + i;
    v[i] = row < V ? acc[i] : -__builtin_inff();
    tmax = fmaxf(tmax, v[i]);
  }
  if (tmax > m) {
    ssum *= exp2f((m - tmax) * kL2e);
    m = tmax;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (v[i] != -__builtin_inff()) ssum += exp2f((v[i] - m) * kL2e);
    list_insert<KM>(tv, ti, v[i], (int)(row0 + 4 * g + i));
  }
}

template <typename TA, int WK, int KM, int TPW>
__global__ __launch_bounds__(256) void lmhead_topk_kernel(TopkArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int d = a.d;
  const long V = a.V;
  const long ntiles = (V + 15) / 16;
  const long nw = a.n_waves;
  const long wid = (long)blockIdx.x * 4 + wave;
  // contiguous, balanced tile ranges: every wave owns floor or ceil of ntiles / nw
  const long t_beg = wid < nw ? wid * ntiles / nw : ntiles;
  const long t_end = wid < nw ? (wid + 1) * ntiles / nw : ntiles;
  const int cnt = (int)(t_end - t_beg);
  const bool tok_ok = r16 < a.B;
  const TA *hr = reinterpret_cast<const TA *>(a.h) + (long)min(r16, a.B - 1) * d;

  SRow<TA, WK> rows[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u)
    rows[u] = srow<TA, WK>(a.w, a.scales, min((t_beg + u) * 16 + r16, V - 1), d);
  f32x4 acc[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) acc[u] = zero4();
  if (cnt > 0) stream_k<TA, WK, TPW>(hr, rows, cnt, 0, d, g, tok_ok, acc);

  float tv[KM];
  int ti[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    tv[j] = -__builtin_inff();
    ti[j] = 0x7fffffff;
  }
  float m = -__builtin_inff(), ssum = 0.f;
  // fold: lane holds rows (t_beg+u)*16 + 4g + i of token r16, visited in increasing order
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    if (u < cnt) {
      float v[4];
      float tmax = -__builtin_inff();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const long row = (t_beg + u) * 16 + 4 * g + i;
        v[i] = row < V ? acc[u][i] : -__builtin_inff();
        tmax = fmaxf(tmax, v[i]);
      }
      if (tmax > m) {
        ssum *= exp2f((m - tmax) * kL2e);
        m = tmax;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (v[i] != -__builtin_inff()) ssum += exp2f((v[i] - m) * kL2e);
        list_insert<KM>(tv, ti, v[i], (int)((t_beg + u) * 16 + 4 * g + i));
      }
    }
  }

  __shared__ float lv[256 * KM];
  __shared__ int li[256 * KM];
  __shared__ float lm[256], ls[256];
  wg_merge_write<KM>(tv, ti, m, ssum, a, lv, li, lm, ls);
}

// ---------------------------------------------------------------------------
// LM head with the B x d activation block resident in LDS.  One persistent
// workgroup per CU stages h once (so h is fetched 256 times per launch, not
// once per wave per chunk); each wave then streams its contiguous range of
// 16-row tiles, one tile at a time, through a DEPTH-deep ring of 128-wide
// chunks that runs across tile boundaries, so DEPTH chunks of weight loads
// are always in flight.  h rows are stored with the fragment index (8
// elements) XORed by (token & 15): the 16 lanes reading one k-chunk of 16
// tokens hit 16 different bank groups.
// ---------------------------------------------------------------------------
#ifndef DFL_LMH_DEPTH
#define DFL_LMH_DEPTH 1      // chunks in flight per wave, bf16 / fp32 heads
#endif
#ifndef DFL_LMH_SCALE_X4
#define DFL_LMH_SCALE_X4 1   // Q8_0: one 8-byte scale load per chunk instead of two 2-byte ones
#endif
#ifndef DFL_LMH_DEPTH_Q8
#define DFL_LMH_DEPTH_Q8 2   // ... Q8_0 heads (half the bytes per chunk)
#endif

template <typename TA, int WK>
struct LmStage {
  Frag<TA> a[WK == W_Q8_0 ? 1 : 4];
  uint4 c[WK == W_Q8_0 ? 2 : 1];
  float sc[WK == W_Q8_0 ? 2 : 1];
};

// element k of token t's row, swizzled in units of one 8-element MFMA
// fragment (16 bytes of bf16, 32 of fp32), so a fragment stays contiguous
template <typename TA>
__device__ __forceinline__ int hsw(int t, int k, int d) {
  const int mask = ((d >> 3) & 15) == 0 ? 15 : 7;
  const int ch = k >> 3;
  return t * d + ((ch ^ (t & mask)) << 3) + (k & 7);
}

// A lane's weight row for the load cursor: values (or codes) and scales.
struct LmRow {
  const char *w;
  const uint16_t *s;
};

template <typename TA, int WK>
__device__ __forceinline__ LmRow lm_row(const void *w, const void *scales, long row, int d) {
  LmRow r;
  if constexpr (WK == W_Q8_0) {
    r.w = reinterpret_cast<const char *>(w) + row * d;
    r.s = reinterpret_cast<const uint16_t *>(scales) + row * (d >> 5);
  } else {
    r.w = reinterpret_cast<const char *>(w) + row * d * (long)sizeof(TA);
    r.s = nullptr;
  }
  return r;
}

// (d % 128 == 0 on this path: every chunk is whole, so no load is guarded)
template <typename TA, int WK>
__device__ __forceinline__ void lm_stage_load(LmStage<TA, WK> &s, const LmRow &r, int k, int g) {
  if constexpr (WK == W_Q8_0) {
#pragma unroll
    for (int m = 0; m < 2; ++m) s.c[m] = *reinterpret_cast<const uint4 *>(r.w + k + 64 * m + 16 * g);
#if DFL_LMH_SCALE_X4
    // the chunk's four block scales in one 8-byte load (a row's scales are
    // 8-byte aligned: d % 128 == 0); codes k + 64 m + 16 g use block 2 m + g / 2
    const uint2 q = *reinterpret_cast<const uint2 *>(r.s + (k >> 5));
    const uint32_t w0 = g < 2 ? q.x : q.x >> 16, w1 = g < 2 ? q.y : q.y >> 16;
    s.sc[0] = half_bits_to_f32((uint16_t)w0);
    s.sc[1] = half_bits_to_f32((uint16_t)w1);
#else
#pragma unroll
    for (int m = 0; m < 2; ++m) s.sc[m] = half_bits_to_f32(r.s[(k + 64 * m + 16 * g) >> 5]);
#endif
  } else {
    const TA *p = reinterpret_cast<const TA *>(r.w);
#pragma unroll
    for (int j = 0; j < 4; ++j) s.a[j] = load_frag(p + k + 32 * j + 8 * g);
  }
}

template <typename TA, int WK>
__device__ __forceinline__ void lm_stage_mma(const LmStage<TA, WK> &s, const TA *hrow, int d, int k,
                                             int g, int tok, f32x4 &acc) {
  if constexpr (WK == W_Q8_0) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int off = k + 64 * m + 16 * g;
      const Frag<bf16> b0 = load_frag(hrow + hsw<TA>(tok, off, d));
      const Frag<bf16> b1 = load_frag(hrow + hsw<TA>(tok, off + 8, d));
      mma(acc, dq8(s.c[m].x, s.c[m].y, s.sc[m]), b0);
      mma(acc, dq8(s.c[m].z, s.c[m].w, s.sc[m]), b1);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const Frag<TA> b = load_frag(hrow + hsw<TA>(tok, k + 32 * j + 8 * g, d));
      mma(acc, s.a[j], b);
    }
  }
}

template <typename TA, int WK, int KM, int NW>
__global__ __launch_bounds__(NW * 64) void lmhead_topk_lds_kernel(TopkArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  TA *hs = reinterpret_cast<TA *>(smem);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int d = a.d, B = a.B;
  const long V = a.V;
  constexpr int VEC = 16 / (int)sizeof(TA);
  // stage h (B rows) into LDS, swizzled; SB loads per thread in flight at a
  // time (a load-then-store loop would wait for every load in turn).
  // Chunks past the end re-read the last one and store it again (the same
  // bytes to the same place), so no load or store is conditional.
  const TA *hg = reinterpret_cast<const TA *>(a.h);
  {
    constexpr int SB = 8;
    const int nch = B * (d / VEC);
    for (int c0 = tid; c0 < nch; c0 += SB * NW * 64) {
      u32x4 v[SB];
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        const int c = min(c0 + u * NW * 64, nch - 1);
        const int t = c / (d / VEC), k = (c - t * (d / VEC)) * VEC;
        v[u] = *reinterpret_cast<const u32x4 *>(hg + (long)t * d + k);
      }
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        const int c = min(c0 + u * NW * 64, nch - 1);
        const int t = c / (d / VEC), k = (c - t * (d / VEC)) * VEC;
        *reinterpret_cast<u32x4 *>(hs + hsw<TA>(t, k, d)) = v[u];
      }
    }
  }
  __syncthreads();

  const long ntiles = (V + 15) / 16;
  const long nw = (long)gridDim.x * NW;
  const long wid = (long)blockIdx.x * NW + wave;
  const long t_beg = wid * ntiles / nw, t_end = (wid + 1) * ntiles / nw;
  const int nck = d / 128;
  const int total = (int)(t_end - t_beg) * nck;
  // tokens past B read token B-1's row (valid data); their columns are unused
  const int tok = min(r16, B - 1);

  float tv[KM];
  int ti[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    tv[j] = -__builtin_inff();
    ti[j] = 0x7fffffff;
  }
  float m = -__builtin_inff(), ssum = 0.f;

  constexpr int D = WK == W_Q8_0 ? DFL_LMH_DEPTH_Q8 : DFL_LMH_DEPTH;
  LmStage<TA, WK> st[D];
  // load cursor (tile lt, chunk lk); it stops at the wave's last chunk, so the
  // refills past the end re-read that chunk (a cache hit) instead of branching
  const long t_last = t_end > t_beg ? t_end - 1 : t_beg;
  long lt = t_beg;
  int lk = 0;
  // the cursor's row pointers change once per tile, not per chunk
  LmRow lrow = lm_row<TA, WK>(a.w, a.scales, min(lt * 16 + r16, V - 1), d);
  auto advance = [&]() {
    if (lk + 1 < nck) {
      ++lk;
    } else if (lt < t_last) {
      lk = 0;
      ++lt;
      lrow = lm_row<TA, WK>(a.w, a.scales, min(lt * 16 + r16, V - 1), d);
    }
  };
#pragma unroll
  for (int s = 0; s < D; ++s) {
    lm_stage_load(st[s], lrow, lk * 128, g);
    advance();
  }
  long ct = t_beg;
  int ck = 0;
  f32x4 acc = zero4();
  auto chunk = [&](LmStage<TA, WK> &sg) {
    lm_stage_mma(sg, hs, d, ck * 128, g, tok, acc);
    lm_stage_load(sg, lrow, lk * 128, g);
    advance();
    if (++ck == nck) {
      fold_tile<KM>(acc, ct * 16, V, g, m, ssum, tv, ti);
      acc = zero4();
      ck = 0;
      ++ct;
    }
  };
  // whole rings without guards (a guarded chunk would leave the compiler
  // unsure how many loads are in flight, and it would wait for all of them),
  // then the last total % D chunks
  int c = 0;
  for (; c + D <= total; c += D) {
#pragma unroll
    for (int s = 0; s < D; ++s) chunk(st[s]);
  }
#pragma unroll
  for (int s = 0; s < D - 1; ++s)
    if (c + s < total) chunk(st[s]);
  __syncthreads();   // every wave is done with hs: reuse the LDS for the merge
  float *lv = reinterpret_cast<float *>(smem);
  int *li = reinterpret_cast<int *>(lv + NW * 64 * KM);
  float *lm = reinterpret_cast<float *>(li + NW * 64 * KM);
  float *ls = lm + NW * 64;
  wg_merge_write<KM, NW>(tv, ti, m, ssum, a, lv, li, lm, ls);
}

// waves per workgroup of the h-resident LM head (4 or 8)
#ifndef DFL_LMH_WAVES
#define DFL_LMH_WAVES 8
#endif

int topk_lds_waves() { return DFL_LMH_WAVES; }

size_t topk_lds_bytes(int B, int d, int act, int K) {
  const int km = K <= 8 ? 8 : 32;
  const size_t h = (size_t)B * d * (act == ACT_F32 ? 4 : 2);
  const size_t nt = DFL_LMH_WAVES * 64;
  const size_t mg = nt * km * 8 + nt * 8;
  return h > mg ? h : mg;
}

// Final merge, one workgroup of 256 threads per token (merge_token).
template <int KM>
__global__ __launch_bounds__(256) void topk_merge_kernel(TopkArgs a) {
  merge_token<KM, 256>(a, blockIdx.x);
}

// about DFL_TOPK_WAVES waves, each owning at most TPW consecutive 16-row
// tiles of W_lm
// (Q8_0 weights: DFL_TOPK_WAVES_Q8, more waves with fewer tiles each, as the
// dequantisation needs more registers per tile)
#ifndef DFL_TOPK_WAVES
#define DFL_TOPK_WAVES 2048
#endif
#ifndef DFL_TOPK_WAVES_Q8
#define DFL_TOPK_WAVES_Q8 4096
#endif
static const int kTpwChoices[] = {1, 2, 4, 5, 6, 8, 12, 16};

static int topk_tpw(long V, int wkind) {
  const long ntiles = (V + 15) / 16;
  const long target = wkind == W_Q8_0 ? DFL_TOPK_WAVES_Q8 : DFL_TOPK_WAVES;
  const long need = (ntiles + target - 1) / target;
  for (int c : kTpwChoices)
    if (c >= need) return c;
  return 16;
}

int topk_plan_waves(long V, int wkind) {
  const long ntiles = (V + 15) / 16;
  const int tpw = topk_tpw(V, wkind);
  return (int)((ntiles + tpw - 1) / tpw);
}

int topk_plan_wgs(long V, int wkind) { return (topk_plan_waves(V, wkind) + 3) / 4; }

template <typename TA, int WK, int KM, int TPW>
static void topk_launch_t(const TopkArgs &a, hipStream_t st) {
  hipLaunchKernelGGL((lmhead_topk_kernel<TA, WK, KM, TPW>), dim3(a.n_wg), dim3(256), 0, st, a);
  hipLaunchKernelGGL((topk_merge_kernel<KM>), dim3(a.B), dim3(256), 0, st, a);
}

template <typename TA, int WK, int KM>
static void topk_launch_tpw(const TopkArgs &a, hipStream_t st) {
  switch (topk_tpw(a.V, WK)) {
    case 1: topk_launch_t<TA, WK, KM, 1>(a, st); break;
    case 2: topk_launch_t<TA, WK, KM, 2>(a, st); break;
    case 4: topk_launch_t<TA, WK, KM, 4>(a, st); break;
    case 5: topk_launch_t<TA, WK, KM, 5>(a, st); break;
    case 6: topk_launch_t<TA, WK, KM, 6>(a, st); break;
    case 8: topk_launch_t<TA, WK, KM, 8>(a, st); break;
    case 12: topk_launch_t<TA, WK, KM, 12>(a, st); break;
    default: topk_launch_t<TA, WK, KM, 16>(a, st); break;
  }
}

template <typename TA, int WK, int KM>
static hipError_t topk_launch_lds(const TopkArgs &a, hipStream_t st, bool merge = true) {
  auto *kern = &lmhead_topk_lds_kernel<TA, WK, KM, DFL_LMH_WAVES>;
  // more than 64 KB of dynamic LDS has to be allowed explicitly
  const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void *>(kern), (size_t)a.lds_bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(a.n_wg), dim3(DFL_LMH_WAVES * 64), (size_t)a.lds_bytes, st, a);
  if (merge) hipLaunchKernelGGL((topk_merge_kernel<KM>), dim3(a.B), dim3(256), 0, st, a);
  return hipSuccess;
}

hipError_t launch_topk_partials(int act, int wkind, const TopkArgs &a, hipStream_t st) {
  if (!a.lds_path || a.K > 8) return hipErrorInvalidValue;
  hipError_t e;
  if (act == ACT_F32) e = topk_launch_lds<float, W_SAME, 8>(a, st, false);
  else if (wkind == W_Q8_0) e = topk_launch_lds<bf16, W_Q8_0, 8>(a, st, false);
  else e = topk_launch_lds<bf16, W_SAME, 8>(a, st, false);
  return e != hipSuccess ? e : hipGetLastError();
}

template <typename TA, int WK>
static hipError_t topk_launch_k(const TopkArgs &a, hipStream_t st) {
  if (a.lds_path) return a.K <= 8 ? topk_launch_lds<TA, WK, 8>(a, st) : topk_launch_lds<TA, WK, 32>(a, st);
  if (a.K <= 8) topk_launch_tpw<TA, WK, 8>(a, st);
  else topk_launch_tpw<TA, WK, 32>(a, st);
  return hipSuccess;
}

hipError_t launch_topk(int act, int wkind, const TopkArgs &a, hipStream_t st) {
  hipError_t e;
  if (act == ACT_F32) e = topk_launch_k<float, W_SAME>(a, st);
  else if (wkind == W_Q8_0) e = topk_launch_k<bf16, W_Q8_0>(a, st);
  else e = topk_launch_k<bf16, W_SAME>(a, st);
  return e != hipSuccess ? e : hipGetLastError();
}

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// ---------------------------------------------------------------------------
// Scratch of the LM head's no-allocation entry point: a static device array
// (each GPU holds its own copy until the process ends).  In host code the
// array's name is not its device address, so it is never passed to a kernel
// or a copy: topk_scratch_ptr() looks the address up with
// hipGetSymbolAddress, once per device with that device current, and every
// later use takes that pointer.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[kTopkScratchBytes];

hipError_t topk_scratch_ptr(void **out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace dfl
