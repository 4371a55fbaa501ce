// GEMM kernels of libdflash: Y[t][n] = sum_k A[t][k] * W[n][k].
//
// Two shapes occur in the draft block step:
//  * skinny: at most 16 activation rows (a block of drafted tokens, or the
//    16 rows injected per decode step) against a large weight.  The weight
//    is streamed from HBM exactly once and that stream is the whole cost, so
//    each wave keeps its W fragments in registers straight from global memory
//    (no LDS), the 16 rows fill the N side of a 16x16x32 MFMA, and split-K
//    gives enough waves to keep HBM busy; partials are summed in a fixed order
//    by a second kernel (bitwise reproducible).
//  * tiled: many rows (a 32k-token prefill injection).  MFMA-bound; classic
//    LDS-staged tiles with double buffering and a register prefetch of the
//    next k-tile.  The activation operand may be several arrays side by side
//    along K (the concatenated target-layer features are never materialised).
#include "common.h"
#include "kernels.h"
#include "stream.h"

namespace dfl {

// ---------------------------------------------------------------------------
// shared epilogue
// ---------------------------------------------------------------------------

template <typename TA, int OM>
__device__ __forceinline__ void store_out_m(const OutSpec &o, long t, long n, float v) {
  if constexpr (OM == OUT_F32) {
    reinterpret_cast<float *>(o.out)[t * o.ld + o.col0 + n] = v;
  } else if constexpr (OM == OUT_ACT) {
    if (o.resid) v += to_f32(reinterpret_cast<const TA *>(o.resid)[t * o.ld_resid + n]);
    reinterpret_cast<TA *>(o.out)[t * o.ld + o.col0 + n] = from_f32<TA>(v);
  } else {
    TA *dst = reinterpret_cast<TA *>(n < o.split ? o.ck : o.cv);
    const long c = n < o.split ? n : n - o.split;
    const long head = c / o.hd, dim = c - head * o.hd;
    dst[(head * o.cap + o.pos0 + t) * o.hd + dim] = from_f32<TA>(v);
  }
}

template <typename TA>
__device__ __forceinline__ void store_out(const OutSpec &o, long t, long n, float v) {
  if (o.mode == OUT_F32) store_out_m<TA, OUT_F32>(o, t, n, v);
  else if (o.mode == OUT_ACT) store_out_m<TA, OUT_ACT>(o, t, n, v);
  else store_out_m<TA, OUT_CACHE>(o, t, n, v);
}

// row n of a stacked weight set -> (segment, local row)
__device__ __forceinline__ int seg_of(const WSet &W, int n, int *local) {
  int s = 0, base = 0;
#pragma unroll
  for (int j = 0; j < kMaxSeg - 1; ++j) {
    const int rs = pick(W.rows, s);
    if (s < W.n_seg - 1 && n >= base + rs) {
      base += rs;
      ++s;
    }
  }
  *local = n - base;
  return s;
}

// ---------------------------------------------------------------------------
// skinny (weight-streaming) GEMM
// ---------------------------------------------------------------------------

// Workgroup (x, y): 4 waves, each owning TPW consecutive 16-row tiles of the
// stacked weight, over k-range y.  Partials part[y][n][16] (fp32).
template <typename TA, int WK, int TPW>
__global__ __launch_bounds__(256) void skinny_gemm_kernel(ASrc X, int M, WSet W, int kchunk,
                                                          float *__restrict__ part) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int N = W.n_total, K = W.K;
  const int ntile = (N + 15) >> 4;
  const int tile0 = (blockIdx.x * 4 + wave) * TPW;
  const int cnt = min(TPW, ntile - tile0);
  if (cnt <= 0) return;
  const int k0 = blockIdx.y * kchunk;
  const int k1 = min(K, k0 + kchunk);

  SRow<TA, WK> rows[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    int lr;
    const int n = min((tile0 + u) * 16 + r16, N - 1);
    const int sg = seg_of(W, n, &lr);
    rows[u] = srow<TA, WK>(pick(W.data, sg), pick(W.scales, sg), lr, K);
  }
  const bool tok_ok = r16 < M;
  const int kps = X.k_per_src;
  const long trow = (long)min(r16, M - 1) * kps;

  f32x4 acc[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) acc[u] = zero4();
  // walk the k-range one activation source at a time
  for (int s = k0 / kps; s * kps < k1; ++s) {
    const int ka = max(k0, s * kps), kb = min(k1, (s + 1) * kps);
    const TA *xr = reinterpret_cast<const TA *>(pick(X.ptr, s)) + trow - (long)s * kps;
    stream_k<TA, WK, TPW>(xr, rows, cnt, ka, kb, g, tok_ok, acc);
  }
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    if (u < cnt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = (tile0 + u) * 16 + 4 * g + i;
        if (n < N) part[((long)blockIdx.y * N + n) * 16 + r16] = acc[u][i];
      }
    }
  }
}

// Y[t][n] = sum over k-ranges of the partials, in range order (bitwise
// reproducible); 8 ranges' loads are issued together to hide their latency.
template <typename TA>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ part,
                                                            int ksplit, int N, int M, OutSpec o) {
  const long id = (long)blockIdx.x * 256 + threadIdx.x;
  const long n = id >> 2;
  const int tg = (int)(id & 3);
  if (n >= N) return;
  const float *p = part + n * 16 + 4 * tg;
  const long stride = (long)N * 16;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  int ks = 0;
  for (; ks + 8 <= ksplit; ks += 8) {
    float4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = *reinterpret_cast<const float4 *>(p + (ks + j) * stride);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      s.x += v[j].x; s.y += v[j].y; s.z += v[j].z; s.w += v[j].w;
    }
  }
  for (; ks < ksplit; ++ks) {
    const float4 v = *reinterpret_cast<const float4 *>(p + ks * stride);
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  const float vals[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = 4 * tg + j;
    if (t < M) store_out<TA>(o, t, n, vals[j]);
  }
}

struct SkinnyPlan {
  int tpw, kchunk, ksplit, groups;
};

// about DFL_SKINNY_WAVES waves: TPW tiles per wave, the k-range split to match
#ifndef DFL_SKINNY_WAVES
#define DFL_SKINNY_WAVES 2048
#endif
// tiles per wave: 4 for long k-ranges (the injection fc), 2 otherwise
#ifndef DFL_SKINNY_TPW_LONGK
#define DFL_SKINNY_TPW_LONGK 4
#endif
#ifndef DFL_SKINNY_TPW
#define DFL_SKINNY_TPW 2
#endif
static SkinnyPlan skinny_plan(int N, int K) {
  SkinnyPlan p;
  const int ntile = (N + 15) / 16;
  p.tpw = ntile >= 256 ? (K >= 16384 ? DFL_SKINNY_TPW_LONGK : DFL_SKINNY_TPW) : 1;
  const int wave_groups = (ntile + p.tpw - 1) / p.tpw;
  p.groups = (wave_groups + 3) / 4;
  int ks = (DFL_SKINNY_WAVES + wave_groups - 1) / wave_groups;
  if (ks < 1) ks = 1;
  int kc = (K + ks - 1) / ks;
  kc = ((kc + 63) / 64) * 64;
  if (kc < 128) kc = 128;
  if (kc > K) kc = K;
  p.kchunk = kc;
  p.ksplit = (K + kc - 1) / kc;
  return p;
}

size_t skinny_partial_floats(int n_total, int K) {
  const SkinnyPlan p = skinny_plan(n_total, K);
  return (size_t)p.ksplit * (size_t)n_total * 16;
}

template <typename TA, int WK>
static hipError_t skinny_launch_t(const ASrc &X, int M, const WSet &W, float *part,
                                  const OutSpec &out, hipStream_t st) {
  const SkinnyPlan p = skinny_plan(W.n_total, W.K);
  dim3 grid(p.groups, p.ksplit);
  if (p.tpw == 4)
    hipLaunchKernelGGL((skinny_gemm_kernel<TA, WK, 4>), grid, dim3(256), 0, st, X, M, W, p.kchunk,
                       part);
  else if (p.tpw == 2)
    hipLaunchKernelGGL((skinny_gemm_kernel<TA, WK, 2>), grid, dim3(256), 0, st, X, M, W, p.kchunk,
                       part);
  else
    hipLaunchKernelGGL((skinny_gemm_kernel<TA, WK, 1>), grid, dim3(256), 0, st, X, M, W, p.kchunk,
                       part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long threads = (long)W.n_total * 4;
  hipLaunchKernelGGL((splitk_reduce_kernel<TA>), dim3((unsigned)((threads + 255) / 256)), dim3(256),
                     0, st, part, p.ksplit, W.n_total, M, out);
  return hipGetLastError();
}

hipError_t launch_skinny_gemm(int act, int wkind, const ASrc &X, int M, const WSet &W, float *part,
                              const OutSpec &out, hipStream_t st) {
  if (act == ACT_F32) return skinny_launch_t<float, W_SAME>(X, M, W, part, out, st);
  if (wkind == W_Q8_0) return skinny_launch_t<bf16, W_Q8_0>(X, M, W, part, out, st);
  return skinny_launch_t<bf16, W_SAME>(X, M, W, part, out, st);
}

// ---------------------------------------------------------------------------
// tiled GEMM (many rows)
// ---------------------------------------------------------------------------

constexpr int TBM = 128, TBN = 128;

template <typename TA>
struct TileCfg {
  static constexpr int BK = 128 / (int)sizeof(TA);   // one 128-byte row per k-tile
  static constexpr int PAD = 16 / (int)sizeof(TA);   // 16-byte row padding (bank spread)
  static constexpr int LD = BK + PAD;
  static constexpr int VEC = 16 / (int)sizeof(TA);   // elements per 16-byte chunk
  static constexpr int CPR = BK / VEC;               // chunks per row (8)
};

// one thread's share of a tile load: (BM * CPR) / 256 chunks of 16 bytes
template <typename TA, int WK>
struct TileLoader {
  using C = TileCfg<TA>;
  static constexpr int NA = TBM * C::CPR / 256;  // 4
  uint4 a[NA];
  uint4 w[NA];        // SAME: 16-byte chunks; Q8_0: half chunks (8 codes) in .x/.y
  float wscale[NA];

  __device__ __forceinline__ void load(const ASrc &A, int M, const WSet &W, int m0, int n0, int k0,
                                       int tid) {
    const int s = k0 / A.k_per_src;
    const int kl = k0 - s * A.k_per_src;
    const TA *src = reinterpret_cast<const TA *>(pick(A.ptr, s));
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const int c = tid + 256 * j;
      const int row = c / C::CPR, ch = c % C::CPR;
      const int m = min(m0 + row, M - 1);
      a[j] = *reinterpret_cast<const uint4 *>(src + (long)m * A.k_per_src + kl + ch * C::VEC);
      const int n = min(n0 + row, W.n_total - 1);
      int lr;
      const int sg = seg_of(W, n, &lr);
      if constexpr (WK == W_Q8_0) {
        const int8_t *q = reinterpret_cast<const int8_t *>(pick(W.data, sg)) + (long)lr * W.K + k0 + ch * 8;
        const uint2 v = *reinterpret_cast<const uint2 *>(q);
        w[j].x = v.x;
        w[j].y = v.y;
        const uint16_t *sc = reinterpret_cast<const uint16_t *>(pick(W.scales, sg)) + (long)lr * (W.K >> 5);
        wscale[j] = half_bits_to_f32(sc[(k0 + ch * 8) >> 5]);
      } else {
        w[j] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const TA *>(pick(W.data, sg)) +
                                                (long)lr * W.K + k0 + ch * C::VEC);
      }
    }
  }

  __device__ __forceinline__ void store(TA *As, TA *Ws, int tid) {
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const int c = tid + 256 * j;
      const int row = c / C::CPR, ch = c % C::CPR;
      *reinterpret_cast<uint4 *>(As + row * C::LD + ch * C::VEC) = a[j];
      if constexpr (WK == W_Q8_0) {
        // 8 codes -> 8 bf16 at k = ch*8 (the bf16 tile row holds BK = 64)
        const Frag<bf16> f = dequant8(make_uint2(w[j].x, w[j].y), wscale[j]);
        *reinterpret_cast<bf16x8 *>(Ws + row * C::LD + ch * 8) = f.v;
      } else {
        *reinterpret_cast<uint4 *>(Ws + row * C::LD + ch * C::VEC) = w[j];
      }
    }
  }
};

template <typename TA, int WK, int OM>
__global__ __launch_bounds__(256) void tile_gemm_kernel(ASrc A, int M, WSet W, OutSpec o) {
  using C = TileCfg<TA>;
  static_assert(WK == W_SAME || C::BK == 64, "Q8_0 tiles are bf16");
  // Q8_0 loads 8 codes per chunk, so a Q8_0 tile covers 8 * CPR = 64 k as well
  __shared__ __attribute__((aligned(16))) TA As[2][TBM * C::LD];
  __shared__ __attribute__((aligned(16))) TA Ws[2][TBN * C::LD];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * TBN, m0 = blockIdx.y * TBM;
  const int K = W.K;
  const int nk = K / C::BK;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = zero4();

  TileLoader<TA, WK> ld;
  ld.load(A, M, W, m0, n0, 0, tid);
  ld.store(As[0], Ws[0], tid);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    // prefetch the next k-tile (the last iteration re-reads its own tile, so
    // the loop body has no branches and the staging registers stay registers)
    ld.load(A, M, W, m0, n0, min(kt + 1, nk - 1) * C::BK, tid);
    const TA *as = As[cur];
    const TA *ws = Ws[cur];
#pragma unroll
    for (int kk = 0; kk < C::BK; kk += 32) {
      Frag<TA> fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[i] = load_frag(as + (wm * 64 + 16 * i + r16) * C::LD + kk + 8 * g);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        fb[j] = load_frag(ws + (wn * 64 + 16 * j + r16) * C::LD + kk + 8 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) mma(acc[i][j], fa[i], fb[j]);
    }
    ld.store(As[cur ^ 1], Ws[cur ^ 1], tid);
    __syncthreads();
  }

  // acc[i][j][v]: activation row m0 + wm*64 + 16i + 4g + v, weight row n0 + wn*64 + 16j + r16
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn * 64 + 16 * j + r16;
      if (n >= W.n_total) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + wm * 64 + 16 * i + 4 * g + v;
        if (m < M) store_out_m<TA, OM>(o, m, n, acc[i][j][v]);
      }
    }
}

template <typename TA, int WK>
static void tile_launch_t(const ASrc &A, int M, const WSet &W, const OutSpec &out, hipStream_t st) {
  dim3 grid((W.n_total + TBN - 1) / TBN, (M + TBM - 1) / TBM);
  if (out.mode == OUT_F32)
    hipLaunchKernelGGL((tile_gemm_kernel<TA, WK, OUT_F32>), grid, dim3(256), 0, st, A, M, W, out);
  else if (out.mode == OUT_ACT)
    hipLaunchKernelGGL((tile_gemm_kernel<TA, WK, OUT_ACT>), grid, dim3(256), 0, st, A, M, W, out);
  else
    hipLaunchKernelGGL((tile_gemm_kernel<TA, WK, OUT_CACHE>), grid, dim3(256), 0, st, A, M, W, out);
}

hipError_t launch_tile_gemm(int act, int wkind, const ASrc &A, int M, const WSet &W,
                            const OutSpec &out, hipStream_t st) {
  if (act == ACT_F32)
    tile_launch_t<float, W_SAME>(A, M, W, out, st);
  else if (wkind == W_Q8_0)
    tile_launch_t<bf16, W_Q8_0>(A, M, W, out, st);
  else
    tile_launch_t<bf16, W_SAME>(A, M, W, out, st);
  return hipGetLastError();
}

}  // namespace dfl
