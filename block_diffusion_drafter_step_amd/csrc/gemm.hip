// GEMM kernels of libdflash: Y[t][n] = sum_k A[t][k] * W[n][k].
//
// Two shapes occur in the draft block step:
//  * skinny: at most 16 activation rows (a block of drafted tokens, or the
//    16 rows injected per decode step) against a large weight.  The weight
//    is streamed from HBM exactly once and that stream is the whole cost, so
//    each wave keeps its W fragments in registers straight from global memory
//    (no LDS), the 16 rows fill the N side of a 16x16x32 MFMA, and split-K
//    gives enough waves to keep HBM busy; partial sums are always added in a
//    fixed order (bitwise reproducible), by a second kernel for large
//    weights, in LDS and by the last workgroup to finish for small ones.
//  * tiled: many rows (a 32k-token prefill injection).  MFMA-bound; classic
//    LDS-staged tiles with double buffering and a register prefetch of the
//    next k-tile.  The activation operand may be several arrays side by side
//    along K (the concatenated target-layer features are never materialised).
#include <algorithm>
#include <atomic>
#include <chrono>
#include <random>

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
  } else {   // K rows [head][pos][dim]; V in transposed 32-position panels [head][pos/32][dim][pos%32]
    if (n < o.split) {
      const long head = n / o.hd, dim = n - head * o.hd;
      reinterpret_cast<TA *>(o.ck)[(head * o.cap + o.pos0 + t) * o.hd + dim] = from_f32<TA>(v);
    } else {
      const long c = n - o.split;
      const long head = c / o.hd, dim = c - head * o.hd, pos = o.pos0 + t;
      reinterpret_cast<TA *>(o.cv)[((head * (o.cap >> 5) + (pos >> 5)) * o.hd + dim) * 32 + (pos & 31)] =
          from_f32<TA>(v);
    }
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

// Two arrangements of the waves of workgroup (x, y) over the tiles (TPW
// consecutive 16-row tiles of the stacked weight per wave) and the k-ranges:
//  * SPLIT_TILES: wave w owns tile group WPG x + w over k-range y and writes
//    its own partials part[y][tile][lane] (float4), summed in k-range order
//    by splitk_reduce_kernel.  Best for large weights: each wave streams
//    independently.
//  * otherwise: all waves own tile group x and stream the WPG consecutive
//    k-ranges (WPG y + wave) * kchunk of it; their accumulators are summed in
//    LDS in a fixed pairwise order.  With one k-group the workgroup writes
//    the outputs.  Otherwise it writes one partial per tile, and the last
//    workgroup of the tile group to finish -- found with the completion
//    counter cnt[x] (arrive_last) -- sums the partials in k-group order and
//    writes the outputs: one kernel, bitwise reproducible (the order never
//    depends on which workgroup finishes last), and no workgroup ever waits
//    for another.  Best for small weights, where a second launch would cost
//    more than the stream.  cnt == nullptr: partials only, as for SPLIT_TILES.
//
// Ordering of that hand-over (HIP's scoped memory model): partials are
// agent-scope atomic stores; each wave waits for its own stores, a
// workgroup barrier follows, then one thread counts the arrival with an
// agent-scope release CAS.  The thread that sees the last arrival issues an
// agent-scope acquire fence before a second barrier, so every partial
// happens-before the loads that sum them (on gfx950: buffer_wbl2 sc1 before
// each arrival, buffer_inv sc1 once per tile group, sc1 loads and stores).
// Q8_0 weights whose k-ranges all lie on 256-element boundaries (K,
// k_per_src and the k-chunks multiples of 256): chunks come in pairs, and the
// even chunk of a pair takes each tile's eight block scales (both chunks')
// in one 16-byte load, handing the odd chunk its two through registers, so a
// pair issues one scale load per tile instead of two.
template <typename TA, int TPW, bool EVEN>
__device__ __forceinline__ void chunk_load_q8p(Chunk<TA, W_Q8_0_S4, TPW, 4> &ch, float (&snext)[TPW][2],
                                               const TA *xr, const SRow<TA, W_Q8_0_S4> (&rows)[TPW], int cnt,
                                               int k, int g, bool tok_ok) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int off = k + 64 * (j >> 1) + 16 * g + 8 * (j & 1);
    ch.b[j] = tok_ok ? load_frag(reinterpret_cast<const bf16 *>(xr) + off) : frag_zero<bf16>();
  }
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    if (u < cnt) {
#pragma unroll
      for (int m = 0; m < 2; ++m)
        ch.c[u][m] = wload16(reinterpret_cast<const int8_t *>(rows[u].p) + k + 64 * m + 16 * g);
      if constexpr (EVEN) {
        // blocks k/32 + 0..7; codes k + 64 m + 16 g (+ 128 for the odd chunk) use block 2 m + g / 2
        const uint4 q = *reinterpret_cast<const uint4 *>(rows[u].s + (k >> 5));
        const int sh = g < 2 ? 0 : 16;
        ch.sc[u][0] = half_bits_to_f32((uint16_t)(q.x >> sh));
        ch.sc[u][1] = half_bits_to_f32((uint16_t)(q.y >> sh));
        snext[u][0] = half_bits_to_f32((uint16_t)(q.z >> sh));
        snext[u][1] = half_bits_to_f32((uint16_t)(q.w >> sh));
      } else {
        ch.sc[u][0] = snext[u][0];
        ch.sc[u][1] = snext[u][1];
      }
    }
  }
}

// stream_range_g for such weights: (kb - ka) a multiple of 256, so the
// double-buffered chunks alternate even (c0) and odd (c1) and no tail is left
template <typename TA, int TPW>
__device__ __forceinline__ void stream_range_q8p(const TA *xr, const SRow<TA, W_Q8_0_S4> (&rows)[TPW], int cnt,
                                                 int ka, int kb, int g, bool tok_ok, f32x4 (&acc)[TPW]) {
  const int n = (kb - ka) >> 7;
  if (n <= 0) return;
  int k = ka;
  Chunk<TA, W_Q8_0_S4, TPW, 4> c0, c1;
  float snext[TPW][2];
  chunk_load_q8p<TA, TPW, true>(c0, snext, xr, rows, cnt, k, g, tok_ok);
  for (int c = 0; c < n; c += 2) {
    chunk_load_q8p<TA, TPW, false>(c1, snext, xr, rows, cnt, k + 128, g, tok_ok);
    chunk_mma_g(c0, cnt, acc);
    k += 128;
    if (c + 2 < n) chunk_load_q8p<TA, TPW, true>(c0, snext, xr, rows, cnt, k + 128, g, tok_ok);
    chunk_mma_g(c1, cnt, acc);
    k += 128;
  }
}

template <typename TA, int WK, int TPW, int WPG, bool SPLIT_TILES, bool Q8P = false>
__global__ __launch_bounds__(WPG * 64, WPG >= 8 ? WPG / 4 : 2) void skinny_gemm_kernel(
    ASrc X, int M, WSet W, int kchunk, float *__restrict__ part,
    unsigned long long *__restrict__ cnt, unsigned long long stamp, OutSpec o) {
  const int tid = threadIdx.x, lane = tid & 63;
  // wave index as a scalar: tiles, k-range and loop bounds stay uniform
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int N = W.n_total, K = W.K;
  const int ntile = (N + 15) >> 4;
  const int tile0 = (SPLIT_TILES ? blockIdx.x * WPG + wave : blockIdx.x) * TPW;
  const int tcnt = min(TPW, ntile - tile0);
  // SPLIT_TILES: a wave past the last tile has nothing to do (no barrier
  // follows); otherwise never taken (the grid covers the tiles exactly)
  if (tcnt <= 0) return;
  const int k0 = (SPLIT_TILES ? blockIdx.y : blockIdx.y * WPG + wave) * kchunk;
  const int k1 = min(K, k0 + kchunk);

  f32x4 acc[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) acc[u] = zero4();
  if (k0 < k1) {
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
    // walk the k-range one activation source at a time
    for (int s = k0 / kps; s * kps < k1; ++s) {
      const int ka = max(k0, s * kps), kb = min(k1, (s + 1) * kps);
      const TA *xr = reinterpret_cast<const TA *>(pick(X.ptr, s)) + trow - (long)s * kps;
      if constexpr (Q8P && WK == W_Q8_0_S4)
        stream_range_q8p<TA, TPW>(xr, rows, tcnt, ka, kb, g, tok_ok, acc);
      else
        stream_k<TA, WK, TPW>(xr, rows, tcnt, ka, kb, g, tok_ok, acc);
    }
  }

  const int nky = gridDim.y;
  if constexpr (SPLIT_TILES) {
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      if (u < tcnt) {
        if (nky > 1) {
          reinterpret_cast<f32x4 *>(part)[((long)blockIdx.y * ntile + tile0 + u) * 64 + lane] = acc[u];
        } else if (r16 < M) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int n = (tile0 + u) * 16 + 4 * g + i;
            if (n < N) store_out<TA>(o, r16, n, acc[u][i]);
          }
        }
      }
    }
    return;
  } else {
    // sum the waves' accumulators: thread (u, l) owns lane l of tile u
    __shared__ f32x4 red[WPG][TPW][64];
    __shared__ unsigned last;
#pragma unroll
    for (int u = 0; u < TPW; ++u) red[wave][u][lane] = acc[u];
    __syncthreads();
    const int u = tid >> 6;   // tile of this thread (threads beyond TPW * 64 idle)
    const bool mine = u < tcnt;
    f32x4 v = zero4();
    if (mine) {
      f32x4 t[WPG];
#pragma unroll
      for (int w = 0; w < WPG; ++w) t[w] = red[w][u][lane];
#pragma unroll
      for (int h = WPG / 2; h >= 1; h /= 2)
#pragma unroll
        for (int w = 0; w < h; ++w)
#pragma unroll
          for (int i = 0; i < 4; ++i) t[w][i] += t[w + h][i];
      v = t[0];
    }
    if (nky > 1) {
      const long tstride = (long)ntile * 256;
      float *pp = part + (long)(tile0 + u) * 256 + lane * 4;
      if (mine) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          __hip_atomic_store(pp + blockIdx.y * tstride + i, v[i], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
      if (!cnt) return;
      // every wave's partial stores have completed before the arrival counts
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) {
        const bool l = arrive_last(&cnt[blockIdx.x], stamp, nky);
        if (l) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        last = l;
      }
      __syncthreads();
      if (!last || !mine) return;
      v = zero4();
      int ky = 0;
      for (; ky + 4 <= nky; ky += 4) {
        float t[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            t[j][i] = __hip_atomic_load(pp + (ky + j) * tstride + i, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] += t[j][i];
      }
      for (; ky < nky; ++ky)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          v[i] += __hip_atomic_load(pp + ky * tstride + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (mine && r16 < M) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = (tile0 + u) * 16 + 4 * g + i;
        if (n < N) store_out<TA>(o, r16, n, v[i]);
      }
    }
  }
}

// Outputs from the partials part[y][tile][lane] (float4) summed in k-group
// order, as the last workgroup of skinny_gemm_kernel does; 8 k-groups' loads
// are issued together to hide their latency (also in the last, partial
// group; 16 measured no faster in the step).  One thread per (tile, lane).
template <typename TA>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ part, int nky,
                                                            int N, int M, OutSpec o) {
  const int ntile = (N + 15) >> 4;
  const long id = (long)blockIdx.x * 256 + threadIdx.x;
  if (id >= (long)ntile * 64) return;
  const int tile = (int)(id >> 6), lane = (int)(id & 63);
  const int g = lane >> 4, r16 = lane & 15;
  const long tstride = (long)ntile * 64;
  const f32x4 *src = reinterpret_cast<const f32x4 *>(part) + id;
  f32x4 v = zero4();
  // groups past nky re-read the last one and are not added
  constexpr int NF = 8;
  for (int ky = 0; ky < nky; ky += NF) {
    f32x4 t[NF];
#pragma unroll
    for (int j = 0; j < NF; ++j) t[j] = src[(long)min(ky + j, nky - 1) * tstride];
#pragma unroll
    for (int j = 0; j < NF; ++j)
      if (ky + j < nky) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] += t[j][i];
      }
  }
  if (r16 >= M) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = tile * 16 + 4 * g + i;
    if (n < N) store_out<TA>(o, r16, n, v[i]);
  }
}

#ifndef DFL_Q8_SCALE_X4
#define DFL_Q8_SCALE_X4 1   // Q8_0 skinny GEMMs: 8-byte scale loads where k-ranges allow
#endif
#ifndef DFL_Q8_SCALE_X8
#define DFL_Q8_SCALE_X8 1   // ... and 16-byte ones per pair of chunks on split-tile plans
#endif

struct SkinnyPlan {
  int tpw, wpg, kchunk, kgroups, groups;
  bool split_tiles;
};

// About DFL_SKINNY_WAVES waves.  Weights of at least DFL_SKINNY_BIG_TILES
// tiles: SPLIT_TILES, 4 waves per workgroup, TPW tiles per wave (4 for long
// k-ranges such as the injection fc, 2 otherwise; fp32 activations at most
// 2, as 4 would not fit the registers), k-ranges of kchunk.  Smaller weights:
// DFL_SKINNY_WPG waves per workgroup on one tile each, the k-range cut into
// wpg * kgroups ranges.  k-ranges are multiples of 64, at least 128 wide.
#ifndef DFL_SKINNY_WAVES
#define DFL_SKINNY_WAVES 2048
#endif
#ifndef DFL_SKINNY_BIG_TILES
#define DFL_SKINNY_BIG_TILES 256
#endif
#ifndef DFL_SKINNY_WPG
#define DFL_SKINNY_WPG 8
#endif
// Smaller weights aim at fewer waves: for the Wk|Wv product into the cache
// (128 tiles, K = 5120) 8 waves per tile cover the whole k-range, so each
// tile's sum stays in its workgroup and no partials or arrivals are needed
// (2048 waves took two k-groups per tile and a last-arriver hand-over).
#ifndef DFL_SKINNY_SMALL_WAVES
#define DFL_SKINNY_SMALL_WAVES 1024
#endif
#ifndef DFL_SKINNY_TPW_LONGK
#define DFL_SKINNY_TPW_LONGK 4
#endif
#ifndef DFL_SKINNY_TPW
#define DFL_SKINNY_TPW 2
#endif
static SkinnyPlan skinny_plan(int N, int K, bool f32, int align = 64) {
  SkinnyPlan p;
  const int ntile = (N + 15) / 16;
  p.split_tiles = ntile >= DFL_SKINNY_BIG_TILES;
  if (p.split_tiles) {
    p.tpw = K >= 16384 ? DFL_SKINNY_TPW_LONGK : DFL_SKINNY_TPW;
    if (f32 && p.tpw > 2) p.tpw = 2;
    p.wpg = 4;
    const int wave_groups = (ntile + p.tpw - 1) / p.tpw;
    p.groups = (wave_groups + p.wpg - 1) / p.wpg;
    int ks = (DFL_SKINNY_WAVES + wave_groups - 1) / wave_groups;
    if (ks < 1) ks = 1;
    int kc = (K + ks - 1) / ks;
    kc = ((kc + align - 1) / align) * align;
    if (kc < 128) kc = 128;
    p.kchunk = kc;
    p.kgroups = (K + kc - 1) / kc;
  } else {
    p.tpw = 1;
    p.wpg = DFL_SKINNY_WPG;
    p.groups = ntile;
    int kw = (DFL_SKINNY_SMALL_WAVES + p.groups - 1) / p.groups;   // waves per tile
    const int kw_max = (K + 127) / 128;
    if (kw > kw_max) kw = kw_max;
    if (kw < p.wpg) kw = p.wpg;
    int kc = (K + kw - 1) / kw;
    kc = ((kc + align - 1) / align) * align;
    if (kc < 128) kc = 128;
    p.kchunk = kc;
    p.kgroups = (K + p.wpg * kc - 1) / (p.wpg * kc);
  }
  return p;
}

size_t skinny_partial_floats(int n_total, int K) {
  size_t most = 0;
  for (const bool f32 : {false, true})
    for (const int align : {64, 128, 256}) {
      const SkinnyPlan p = skinny_plan(n_total, K, f32, align);
      if (p.kgroups > 1) most = std::max(most, (size_t)p.kgroups * (size_t)((n_total + 15) / 16) * 256);
    }
  return most;
}

hipError_t allow_dynamic_lds(const void *k, size_t bytes) {
  hipFuncAttributes at;
  hipError_t e = hipFuncGetAttributes(&at, k);
  if (e != hipSuccess) return e;
  if (at.sharedSizeBytes + bytes > kMaxLdsBytes) return hipErrorInvalidValue;
  return hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

// Launch stamps of the completion counters: 48 bits, never 0 (a zeroed word
// then never matches), one per launch that uses counters.  The sequence
// starts at a per-process random point, so a counter word that another
// process left in reused device memory is as unlikely to carry a live stamp
// as one left by this process.
static unsigned long long stamp_seed() {
  std::random_device rd;
  const unsigned long long t =
      (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count();
  return (((unsigned long long)rd() << 32) ^ rd() ^ (t * 0x9E3779B97F4A7C15ull)) & 0xFFFFFFFFFFFFull;
}
static std::atomic<unsigned long long> g_stamp{stamp_seed()};
unsigned long long next_launch_stamp() {
  unsigned long long s;
  do {
    s = (g_stamp.fetch_add(1, std::memory_order_relaxed) + 1) & 0xFFFFFFFFFFFFull;
  } while (s == 0);
  return s;
}

template <typename TA, int WK>
static hipError_t skinny_launch_t(const ASrc &X, int M, const WSet &W, float *part,
                                  unsigned long long *cnt, const OutSpec &out, hipStream_t st) {
  // Q8_0 split-tile plans on 256 boundaries take the paired scale loads
  bool q8p = WK == W_Q8_0_S4 && DFL_Q8_SCALE_X8 && W.K % 256 == 0 && X.k_per_src % 256 == 0 &&
             (W.n_total + 15) / 16 >= DFL_SKINNY_BIG_TILES;
  for (int i = 0; q8p && i < W.n_seg; ++i) q8p = reinterpret_cast<uintptr_t>(W.scales[i]) % 16 == 0;
  const SkinnyPlan p = skinny_plan(W.n_total, W.K, sizeof(TA) == 4, q8p ? 256 : WK == W_Q8_0_S4 ? 128 : 64);
  const dim3 grid(p.groups, p.kgroups);
  unsigned long long *c = nullptr;
  unsigned long long stamp = 0;
  if (p.split_tiles) {
    if (q8p) {
      if constexpr (WK == W_Q8_0_S4) {
        if (p.tpw == 4)
          hipLaunchKernelGGL((skinny_gemm_kernel<TA, WK, 4, 4, true, true>), grid, dim3(256), 0, st, X, M, W,
                             p.kchunk, part, c, stamp, out);
        else
          hipLaunchKernelGGL((skinny_gemm_kernel<TA, WK, 2, 4, true, true>), grid, dim3(256), 0, st, X, M, W,
                             p.kchunk, part, c, stamp, out);
      }
    } else if (sizeof(TA) == 2 && p.tpw == 4)
      hipLaunchKernelGGL((skinny_gemm_kernel<TA, WK, sizeof(TA) == 2 ? 4 : 2, 4, true>), grid,
                         dim3(256), 0, st, X, M, W, p.kchunk, part, c, stamp, out);
    else if (p.tpw == 2)
      hipLaunchKernelGGL((skinny_gemm_kernel<TA, WK, 2, 4, true>), grid, dim3(256), 0, st, X, M, W,
                         p.kchunk, part, c, stamp, out);
    else
      hipLaunchKernelGGL((skinny_gemm_kernel<TA, WK, 1, 4, true>), grid, dim3(256), 0, st, X, M, W,
                         p.kchunk, part, c, stamp, out);
  } else {
    c = p.groups <= kMaxCounters && p.kgroups < (1 << 16) ? cnt : nullptr;
    if (c) stamp = next_launch_stamp();
    if (p.wpg == 4)
      hipLaunchKernelGGL((skinny_gemm_kernel<TA, WK, 1, 4, false>), grid, dim3(256), 0, st, X, M, W,
                         p.kchunk, part, c, stamp, out);
    else
      hipLaunchKernelGGL((skinny_gemm_kernel<TA, WK, 1, 8, false>), grid, dim3(512), 0, st, X, M, W,
                         p.kchunk, part, c, stamp, out);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || c || p.kgroups == 1) return e;
  const long threads = (long)((W.n_total + 15) / 16) * 64;
  hipLaunchKernelGGL((splitk_reduce_kernel<TA>), dim3((unsigned)((threads + 255) / 256)), dim3(256),
                     0, st, part, p.kgroups, W.n_total, M, out);
  return hipGetLastError();
}

hipError_t launch_skinny_gemm(int act, int wkind, const ASrc &X, int M, const WSet &W, float *part,
                              unsigned long long *cnt, const OutSpec &out, hipStream_t st) {
  if (act == ACT_F32) return skinny_launch_t<float, W_SAME>(X, M, W, part, cnt, out, st);
  // Q8_0 with every k-range on a 128 boundary (k-chunks rounded to 128):
  // one 8-byte scale load per 128-wide chunk
  if (wkind == W_Q8_0 && DFL_Q8_SCALE_X4 && W.K % 128 == 0 && X.k_per_src % 128 == 0)
    return skinny_launch_t<bf16, W_Q8_0_S4>(X, M, W, part, cnt, out, st);
  if (wkind == W_Q8_0) return skinny_launch_t<bf16, W_Q8_0>(X, M, W, part, cnt, out, st);
  return skinny_launch_t<bf16, W_SAME>(X, M, W, part, cnt, out, st);
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
  uint4 w[NA];

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
      w[j] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const TA *>(pick(W.data, sg)) + (long)lr * W.K +
                                              k0 + ch * C::VEC);
    }
  }

  __device__ __forceinline__ void store(TA *As, TA *Ws, int tid) {
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const int c = tid + 256 * j;
      const int row = c / C::CPR, ch = c % C::CPR;
      *reinterpret_cast<uint4 *>(As + row * C::LD + ch * C::VEC) = a[j];
      *reinterpret_cast<uint4 *>(Ws + row * C::LD + ch * C::VEC) = w[j];
    }
  }
};

// SPLIT: workgroup z covers k-tiles [z kc, (z + 1) kc) (kc in elements) and
// writes fp32 partials part[z][m][n] for tile_reduce_kernel instead of outputs.
template <typename TA, int WK, int OM, bool SPLIT>
__global__ __launch_bounds__(256) void tile_gemm_kernel(ASrc A, int M, WSet W, OutSpec o, int kc,
                                                        float *__restrict__ part) {
  using C = TileCfg<TA>;
  static_assert(WK == W_SAME, "Q8_0 weights take dma8q_gemm_kernel");
  __shared__ __attribute__((aligned(16))) TA As[2][TBM * C::LD];
  __shared__ __attribute__((aligned(16))) TA Ws[2][TBN * C::LD];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * TBN, m0 = blockIdx.y * TBM;
  const int K = W.K;
  int kt0 = 0, nk = K / C::BK;
  if constexpr (SPLIT) {
    kt0 = blockIdx.z * (kc / C::BK);
    nk = min(nk, kt0 + kc / C::BK);
  }

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = zero4();

  TileLoader<TA, WK> ld;
  ld.load(A, M, W, m0, n0, kt0 * C::BK, tid);
  ld.store(As[0], Ws[0], tid);
  __syncthreads();

  for (int kt = kt0; kt < nk; ++kt) {
    const int cur = (kt - kt0) & 1;
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
        if (m < M) {
          if constexpr (SPLIT)
            part[((long)blockIdx.z * M + m) * W.n_total + n] = acc[i][j][v];
          else
            store_out_m<TA, OM>(o, m, n, acc[i][j][v]);
        }
      }
    }
}

// out[m][n] from the partials of tile_gemm_kernel<SPLIT>, summed in k-piece
// order (bitwise reproducible); one thread per output element.
template <typename TA, int OM>
__global__ __launch_bounds__(256) void tile_reduce_kernel(const float *__restrict__ part, int S, int M,
                                                          int N, OutSpec o) {
  const long id = (long)blockIdx.x * 256 + threadIdx.x;
  const long mn = (long)M * N;
  if (id >= mn) return;
  // eight pieces' loads in flight at a time (a load-then-add loop waits for
  // each; sixteen slowed the larger sums); pieces past S re-read the last one
  // and are not added, so the sum is taken in piece order
  constexpr int NF = 8;
  float v = 0.f;
  for (int z = 0; z < S; z += NF) {
    float t[NF];
#pragma unroll
    for (int j = 0; j < NF; ++j) t[j] = part[(long)min(z + j, S - 1) * mn + id];
#pragma unroll
    for (int j = 0; j < NF; ++j)
      if (z + j < S) v += t[j];
  }
  const long m = id / N;
  store_out_m<TA, OM>(o, m, id - m * N, v);
}

// Split-K plan of the 128 x 128 tile GEMM.  With few rows (a batched
// injection of a few blocks) its grid covers a fraction of the CUs; below
// kTileSplitTarget workgroups the k-range is cut into S pieces of whole
// 64-wide k-steps (at least 4 each, at most 64 pieces).  Depends only on the
// shapes, so the workspace query and the launch agree.
constexpr int kTileSplitTarget = 512;
int tile_split_plan(int M, int N, int K, int *kc) {
  const long tiles = (long)((N + TBN - 1) / TBN) * ((M + TBM - 1) / TBM);
  const int nk = K / 64;
  int S = 1;
  if (tiles < kTileSplitTarget) S = (int)((kTileSplitTarget + tiles - 1) / tiles);
  S = std::min(S, std::max(1, nk / 4));
  S = std::min(S, 64);
  const int kc64 = (nk + S - 1) / S;
  S = (nk + kc64 - 1) / kc64;
  *kc = kc64 * 64;
  return S;
}

static int dma8s_plan(int M, int N, int K, int *kc);
static int dma8q_plan(int M, int N, int K, int *kc);

size_t tile_partial_floats(int M, int N, int K) {
  int kc;
  const int S = std::max(std::max(tile_split_plan(M, N, K, &kc), dma8s_plan(M, N, K, &kc)),
                         K % 64 == 0 ? dma8q_plan(M, N, K, &kc) : 1);
  return S > 1 ? (size_t)S * M * N : 0;
}

template <typename TA, int WK, int OM>
static void tile_go(const ASrc &A, int M, const WSet &W, const OutSpec &out, float *part, hipStream_t st) {
  int kc = 0;
  const int S = part && W.K % 64 == 0 ? tile_split_plan(M, W.n_total, W.K, &kc) : 1;
  if (S > 1) {
    dim3 grid((W.n_total + TBN - 1) / TBN, (M + TBM - 1) / TBM, S);
    hipLaunchKernelGGL((tile_gemm_kernel<TA, WK, OM, true>), grid, dim3(256), 0, st, A, M, W, out, kc, part);
    const long mn = (long)M * W.n_total;
    hipLaunchKernelGGL((tile_reduce_kernel<TA, OM>), dim3((unsigned)((mn + 255) / 256)), dim3(256), 0, st,
                       part, S, M, W.n_total, out);
  } else {
    dim3 grid((W.n_total + TBN - 1) / TBN, (M + TBM - 1) / TBM);
    hipLaunchKernelGGL((tile_gemm_kernel<TA, WK, OM, false>), grid, dim3(256), 0, st, A, M, W, out, 0,
                       part);
  }
}

template <typename TA, int WK>
static void tile_launch_t(const ASrc &A, int M, const WSet &W, const OutSpec &out, float *part,
                          hipStream_t st) {
  if (out.mode == OUT_F32) tile_go<TA, WK, OUT_F32>(A, M, W, out, part, st);
  else if (out.mode == OUT_ACT) tile_go<TA, WK, OUT_ACT>(A, M, W, out, part, st);
  else tile_go<TA, WK, OUT_CACHE>(A, M, W, out, part, st);
}

// workgroup id -> (m-tile, n-tile)
#ifndef DFL_TILE_GROUP_M
#define DFL_TILE_GROUP_M 4
#endif
__device__ __forceinline__ void big_tile_of(int L, int mt, int nt, int *tm, int *tn) {
  const int T = mt * nt;
  int j = L;
  if ((mt & 7) == 0) {                      // deal a contiguous band of m-tiles to each XCD
    const int per = T >> 3;
    j = (L & 7) * per + (L >> 3);
  }
  // groups of GM m-tiles x all n-tiles, m fastest inside a group
  const int GM = DFL_TILE_GROUP_M;
  const int grp = j / (GM * nt);
  const int rem = j - grp * GM * nt;
  const int gm = min(GM, mt - grp * GM);
  *tn = rem / gm;
  *tm = grp * GM + (rem - *tn * gm);
}

#ifndef DFL_BIG_GEMM_MIN_M
#define DFL_BIG_GEMM_MIN_M 1024
#endif

// ---------------------------------------------------------------------------
// prefill GEMM with direct-to-LDS loads (bf16 activations and weights): a
// 256-wide block tile along N, k-steps of 32.  Global memory is copied into
// LDS by global_load_lds_dwordx4 (no register staging) into a ring of
// stages, so several k-steps of loads are in flight while one is multiplied;
// one barrier per k-step.  A wave instruction writes 1 KB of LDS in lane
// order (16 rows x 64 bytes).
// ---------------------------------------------------------------------------
constexpr int DBN = 256, DBK = 32;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void dma16(const void *g, lds_void *l) {
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
}

// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// 16-byte chunk c of a 64-byte LDS row is stored at slot c ^ ((row >> 1) & 3):
// with this XOR the 16 rows x 4 chunks of one fragment read (ds_read_b128)
// measured free of bank conflicts on gfx950, while XORing with row bits
// 2-3 (or 0-1), or padding the rows, left 1.33 conflict cycles per read
__device__ __forceinline__ int dslot(int row, int c) { return c ^ ((row >> 1) & 3); }

// Workgroup barrier for the direct-to-LDS rings: the caller has waited for
// its own stage loads (vmcnt); this waits for the wave's LDS reads, then
// s_barrier.  Unlike __syncthreads, no workgroup release fence: that fence
// would also wait for every direct-to-LDS load still in flight (they are
// counted as vector-memory operations), draining the whole ring.  The empty
// asm statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((0x3F & 0xF) | ((0x3F >> 4) << 14) | (0x7 << 4) | (0x0 << 8));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 256 x 256 block tile on 8 waves (2 along M x 4 along N, 128 x 64 each):
// 128 accumulator registers per wave leave the fragments and addresses in
// VGPRs (a 128 x 128 wave tile fills the VGPR file with accumulators and the
// compiler shuttles operands through AGPRs), and two waves per SIMD hide each
// other's LDS and barrier stalls.  A 4-stage direct-to-LDS ring with the
// dslot swizzle; each wave issues 2 A and 2 W row blocks per stage from row
// pointers fixed before the loop, and the activation source
// advances without a division.  TBM = 128 halves the block along M (64 x 64
// wave tiles, one A row block per wave per stage) for products whose 256-row
// tiles would leave CUs idle, e.g. the conv's delta (N = T*G = 256).
#ifndef DFL_DMA8_STAGES
#define DFL_DMA8_STAGES 4
#endif
constexpr int D8STAGES = DFL_DMA8_STAGES;

template <int TBM>
constexpr int d8_stage_bytes() { return (TBM + DBN) * DBK * 2; }

// SPLIT: blockIdx.y takes k-steps [y kc, (y + 1) kc) (kc in elements, a
// multiple of 64) and writes fp32 partials part[y][m][n] for
// tile_reduce_kernel instead of outputs.
template <int OM, int TBM, bool SPLIT>
__global__ __launch_bounds__(512) void dma8_gemm_kernel(ASrc A, int M, WSet W, OutSpec o, int kc,
                                                        float *__restrict__ part) {
  static_assert(TBM == 256 || TBM == 128, "block rows");
  constexpr int NA = TBM / 128;        // A row blocks each wave issues per stage
  constexpr int MI = TBM / 32;         // 16-row fragments of a wave tile along M
  constexpr int LPS = NA + 2;          // loads per wave per stage
  constexpr int SB = d8_stage_bytes<TBM>();
  extern __shared__ __attribute__((aligned(1024))) char smem_dma8[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int wm = wave >> 2, wn = wave & 3;
  const int mt = (M + TBM - 1) / TBM, nt = (W.n_total + DBN - 1) / DBN;
  int tm, tn;
  big_tile_of(blockIdx.x, mt, nt, &tm, &tn);
  const int m0 = tm * TBM, n0 = tn * DBN;
  int kt0 = 0, nk = W.K / DBK;   // first k-step and k-step count of this workgroup
  if constexpr (SPLIT) {
    kt0 = blockIdx.y * (kc / DBK);
    nk = min(nk - kt0, kc / DBK);
  }
  const int kps = A.k_per_src;

  // this lane's DMA rows: A blocks NA*wave+j and W blocks 2*wave+j of 16
  // rows, row rl, 16-byte chunk c of the k-step (stored at slot lane & 3)
  const int rl = lane >> 2, slot = lane & 3;
  long a_off[NA];
  const bf16 *w_row[2];
#pragma unroll
  for (int j = 0; j < NA; ++j) {
    const int row = (NA * wave + j) * 16 + rl;
    a_off[j] = (long)min(m0 + row, M - 1) * kps + 8 * dslot(row, slot);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = (2 * wave + j) * 16 + rl;
    const int c = dslot(row, slot);
    int lr;
    const int n = min(n0 + row, W.n_total - 1);
    const int sg = seg_of(W, n, &lr);
    w_row[j] = reinterpret_cast<const bf16 *>(pick(W.data, sg)) + (long)lr * W.K + 8 * c + kt0 * DBK;
  }
  // next k-step to issue (counted from kt0) and its activation source
  int ki = 0, src_i = (kt0 * DBK) / kps, kl = kt0 * DBK - src_i * kps;
  const bf16 *src = reinterpret_cast<const bf16 *>(pick(A.ptr, src_i));
  // the loads of one stage (no branches, so they share a basic block with
  // the k-step's MFMAs and can be scheduled between them)
  auto issue_loads = [&](char *stage) {
#pragma unroll
    for (int j = 0; j < NA; ++j)
      dma16(src + kl + a_off[j], (lds_void *)(stage + (NA * wave + j) * 1024));
#pragma unroll
    for (int j = 0; j < 2; ++j)
      dma16(w_row[j] + ki * DBK, (lds_void *)(stage + TBM * DBK * 2 + (2 * wave + j) * 1024));
  };
  auto advance = [&]() {
    if (ki + 1 < nk) {   // past the last k-step the same one is issued again
      ++ki;
      kl += DBK;
      if (kl == kps) {
        kl = 0;
        ++src_i;
        src = reinterpret_cast<const bf16 *>(pick(A.ptr, src_i));
      }
    }
  };
  auto issue = [&](char *stage) {
    issue_loads(stage);
    advance();
  };

  f32x4 acc[MI][4];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = zero4();

#pragma unroll
  for (int s = 0; s < D8STAGES - 1; ++s) issue(smem_dma8 + s * SB);

  // The fragments of k-step kt+1 are read from LDS while the MFMAs of k-step
  // kt run: one barrier per k-step makes stages kt and kt+1 complete for
  // every wave, stage kt-1 (read a step ago) is then free for the next DMA.
  const int ar = wm * (TBM / 2) + r16, br = wn * 64 + r16;
  auto read_frags = [&](int kt, Frag<bf16> (&fa)[MI], Frag<bf16> (&fb)[4]) {
    const char *st = smem_dma8 + (kt % D8STAGES) * SB;
    const bf16 *as = reinterpret_cast<const bf16 *>(st);
    const bf16 *ws = reinterpret_cast<const bf16 *>(st + TBM * DBK * 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = br + 16 * j;
      fb[j] = load_frag(ws + row * DBK + 8 * dslot(row, g));
    }
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int row = ar + 16 * i;
      fa[i] = load_frag(as + row * DBK + 8 * dslot(row, g));
    }
  };
  auto mmas = [&](const Frag<bf16> (&fa)[MI], const Frag<bf16> (&fb)[4]) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) mma(acc[i][j], fa[i], fb[j]);
  };
  // one k-step: wait for stage kt+1, refill the ring, read kt+1, multiply kt
  auto step = [&](int kt, const Frag<bf16> (&fa)[MI], const Frag<bf16> (&fb)[4],
                  Frag<bf16> (&na)[MI], Frag<bf16> (&nb)[4]) {
    wait_vm<LPS * (D8STAGES - 3)>();   // this wave's loads of stage kt+1 have landed
    ring_barrier();                    // ... everyone's; stage kt-1 is no longer read
    // one basic block: the stage loads and the fragment reads of kt+1 (the
    // last k-step re-reads its own stage) issue between the MFMAs of kt,
    // so the matrix pipe is fed right after the barrier
    issue_loads(smem_dma8 + ((kt + D8STAGES - 1) % D8STAGES) * SB);
    read_frags(min(kt + 1, nk - 1), na, nb);
    mmas(fa, fb);
#pragma unroll
    for (int i = 0; i < LPS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one global load
    }
#pragma unroll
    for (int i = 0; i < MI + 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * MI - LPS - MI - 4, 0);
    advance();
  };
  Frag<bf16> fa0[MI], fb0[4], fa1[MI], fb1[4];
  wait_vm<LPS * (D8STAGES - 2)>();
  ring_barrier();
  read_frags(0, fa0, fb0);
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, fa0, fb0, fa1, fb1);
    if (kt + 1 < nk) step(kt + 1, fa1, fb1, fa0, fb0);
  }
  wait_vm<0>();
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn * 64 + 16 * j + r16;
      if (n >= W.n_total) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + wm * (TBM / 2) + 16 * i + 4 * g + v;
        if (m < M) {
          if constexpr (SPLIT)
            part[((long)blockIdx.y * M + m) * W.n_total + n] = acc[i][j][v];
          else
            store_out_m<bf16, OM>(o, m, n, acc[i][j][v]);
        }
      }
    }
}

template <int OM, int TBM>
static hipError_t dma8_go(const ASrc &A, int M, const WSet &W, const OutSpec &out, hipStream_t st) {
  const int mt = (M + TBM - 1) / TBM, nt = (W.n_total + DBN - 1) / DBN;
  const size_t lds = (size_t)D8STAGES * d8_stage_bytes<TBM>();
  const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void *>(&dma8_gemm_kernel<OM, TBM, false>), lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((dma8_gemm_kernel<OM, TBM, false>), dim3(mt * nt), dim3(512), lds, st, A, M, W, out,
                     0, nullptr);
  return hipSuccess;
}

template <int TBM>
static hipError_t dma8_launch(const ASrc &A, int M, const WSet &W, const OutSpec &out, hipStream_t st) {
  if (out.mode == OUT_F32) return dma8_go<OUT_F32, TBM>(A, M, W, out, st);
  if (out.mode == OUT_ACT) return dma8_go<OUT_ACT, TBM>(A, M, W, out, st);
  return dma8_go<OUT_CACHE, TBM>(A, M, W, out, st);
}

// k-split of the 128 x 256 direct-to-LDS tiles for products with few rows
// (the same rule as the 128 x 128 tile plan, over this kernel's tiles)
static int dma8s_plan(int M, int N, int K, int *kc) {
  const long tiles = (long)((N + DBN - 1) / DBN) * ((M + 127) / 128);
  const int nk = K / 64;
  int S = 1;
  if (tiles < kTileSplitTarget) S = (int)((kTileSplitTarget + tiles - 1) / tiles);
  S = std::min(S, std::max(1, nk / 4));
  S = std::min(S, 64);
  const int kc64 = (nk + S - 1) / S;
  S = (nk + kc64 - 1) / kc64;
  *kc = kc64 * 64;
  return S;
}

template <int OM>
static hipError_t dma8s_go(const ASrc &A, int M, const WSet &W, const OutSpec &out, float *part, int kc,
                           int S, hipStream_t st) {
  const int mt = (M + 127) / 128, nt = (W.n_total + DBN - 1) / DBN;
  const size_t lds = (size_t)D8STAGES * d8_stage_bytes<128>();
  const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void *>(&dma8_gemm_kernel<OM, 128, true>), lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((dma8_gemm_kernel<OM, 128, true>), dim3(mt * nt, S), dim3(512), lds, st, A, M, W, out,
                     kc, part);
  const long mn = (long)M * W.n_total;
  hipLaunchKernelGGL((tile_reduce_kernel<bf16, OM>), dim3((unsigned)((mn + 255) / 256)), dim3(256), 0, st,
                     part, S, M, W.n_total, out);
  return hipSuccess;
}

// bf16 products whose 128 x 256 tiles leave CUs idle: split k over the
// direct-to-LDS kernel (true when taken; *err then holds the launch's error)
static bool dma8_split_launch(const ASrc &A, int M, const WSet &W, const OutSpec &out, float *part,
                              hipStream_t st, hipError_t *err) {
  if (!part || W.K % 64 || A.k_per_src % 32) return false;
  int kc;
  const int S = dma8s_plan(M, W.n_total, W.K, &kc);
  if (S <= 1) return false;
  if (out.mode == OUT_F32) *err = dma8s_go<OUT_F32>(A, M, W, out, part, kc, S, st);
  else if (out.mode == OUT_ACT) *err = dma8s_go<OUT_ACT>(A, M, W, out, part, kc, S, st);
  else *err = dma8s_go<OUT_CACHE>(A, M, W, out, part, kc, S, st);
  return true;
}

// 128 x 256 direct-to-LDS tiles from this many rows, once their tiles cover
// 1 / DFL_HALF_GEMM_FILL of the CUs
#ifndef DFL_HALF_GEMM_MIN_M
#define DFL_HALF_GEMM_MIN_M 256
#endif
#ifndef DFL_HALF_GEMM_FILL
#define DFL_HALF_GEMM_FILL 2
#endif




// ---------------------------------------------------------------------------
// Q8_0 weights with few rows (a batched injection of up to kQ8ExpandMinM - 1
// rows): TBM x 256 direct-to-LDS tiles (TBM = 64 or 128) whose ring holds
// the weights' raw codes and scales.  A k-step is 64 wide (two Q8_0 blocks);
// a stage holds
//  * the activations as two 32-wide halves in the bf16 layout above (the
//    dslot swizzle, 16-row blocks),
//  * the codes as 256 rows of 64 bytes (the same 16-row x 64-byte DMA
//    geometry and swizzle, two blocks per wave),
//  * the scales as one dword per row (both blocks' fp16 scales), ordered so
//    that the rows a lane multiplies (16 apart) are one 16-byte read; the
//    dwords no lane reads repeat rows, so every wave issues the same loads.
// The 8 waves tile the block as (TBM / 64) x (8 / (TBM / 64)), 64 rows
// each: with 64-row tiles every code is dequantised by one wave only.
// Weight fragments are dequantised as they are read from LDS (dequant8, the
// products rounded to bf16 as on the other Q8_0 paths) and three k-steps of
// loads are in flight per CU.  Every LDS read is 16 bytes: narrower reads
// are paired by the compiler into instructions that lose their memory
// operands, after which it waits for all direct-to-LDS loads in flight
// before each k-step's reads.
// ---------------------------------------------------------------------------
constexpr int QBK = 64;                    // k per stage
constexpr int QSW = DBN * QBK;             // codes (16 KB)
constexpr int QSS = 8 * 64 * 4;            // scales: 64 dwords per wave (2 KB)
template <int TBM>
constexpr int q8_stage_bytes() { return 2 * TBM * 64 + QSW + QSS; }   // 34 KB or 26 KB
// ring stages (five or six for the 64-row tiles measured slower: 24 rows
// 72 -> 77 us)
template <int TBM>
constexpr int q8_stages() { return 4; }

// MI: 16-row activation fragments a wave multiplies (2 when a 64-row tile
// holds at most 32 rows: the other two would be padding)
template <int OM, int TBM, bool SPLIT, int MI>
__global__ __launch_bounds__(512) void dma8q_gemm_kernel(ASrc A, int M, WSet W, OutSpec o, int kc,
                                                         float *__restrict__ part) {
  static_assert(TBM == 128 || TBM == 64, "block rows");
  static_assert(MI == 4 || (MI == 2 && TBM == 64), "live fragments");
  constexpr int WNW = 8 / (TBM / 64);   // waves along N
  constexpr int CW = DBN / WNW;         // columns per wave (64 or 32)
  constexpr int NJ = CW / 16;           // weight fragments per wave and half
  constexpr int NAQ = TBM / 64;         // activation row blocks per wave per stage
  constexpr int BPH = TBM / 16;         // activation row blocks per half
  constexpr int QSA = TBM * 64;         // one activation half
  constexpr int QSB = q8_stage_bytes<TBM>();
  constexpr int QLPS = NAQ + 3;         // loads per wave per stage
  constexpr int Q8STAGES = q8_stages<TBM>();
  extern __shared__ __attribute__((aligned(1024))) char smem_q8[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int wm = wave / WNW, wn = wave % WNW;
  const int mt = (M + TBM - 1) / TBM, nt = (W.n_total + DBN - 1) / DBN;
  int tm, tn;
  big_tile_of(blockIdx.x, mt, nt, &tm, &tn);
  const int m0 = tm * TBM, n0 = tn * DBN;
  int kt0 = 0, nk = W.K / QBK;   // first k-step and k-step count of this workgroup
  if constexpr (SPLIT) {
    kt0 = blockIdx.y * (kc / QBK);
    nk = min(nk - kt0, kc / QBK);
  }
  const int kps = A.k_per_src;

  // this lane's DMA rows: activation blocks wave NAQ + q (half t / BPH, block
  // t % BPH), code blocks 2 wave + j (16-byte chunk dslot(row, slot) stored
  // at slot lane & 3), and the scales of the row read as dword d = 64 wave
  // + lane: p = d / 4 is the reading lane's wn 16 + r16, entry d % 4 its
  // fragment (entries past NJ repeat a row)
  const int rl = lane >> 2, slot = lane & 3;
  long a_off[NAQ];
  int a_dst[NAQ];
#pragma unroll
  for (int q = 0; q < NAQ; ++q) {
    const int t = wave * NAQ + q, h = t / BPH, row = (t % BPH) * 16 + rl;
    a_off[q] = (long)min(m0 + row, M - 1) * kps + 32 * h + 8 * dslot(row, slot);
    a_dst[q] = h * QSA + (t % BPH) * 1024;
  }
  const int8_t *w_row[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = (2 * wave + j) * 16 + rl;
    int lr;
    const int n = min(n0 + row, W.n_total - 1);
    const int sg = seg_of(W, n, &lr);
    w_row[j] = reinterpret_cast<const int8_t *>(pick(W.data, sg)) + (long)lr * W.K + 16 * dslot(row, slot) +
               (long)kt0 * QBK;
  }
  const uint16_t *s_row;
  {
    const int d = wave * 64 + lane, p = d >> 2;
    const int row = ((p >> 4) % WNW) * CW + (p & 15) + 16 * ((d & 3) % NJ);
    int lr;
    const int n = min(n0 + row, W.n_total - 1);
    const int sg = seg_of(W, n, &lr);
    s_row = reinterpret_cast<const uint16_t *>(pick(W.scales, sg)) + (long)lr * (W.K >> 5) + 2 * kt0;
  }
  // next k-step to issue (counted from kt0) and its activation source
  int ki = 0, src_i = (kt0 * QBK) / kps, kl = kt0 * QBK - src_i * kps;
  const bf16 *src = reinterpret_cast<const bf16 *>(pick(A.ptr, src_i));
  // the loads of one stage (no branches, so that they share a basic block
  // with the k-step's LDS reads: a branch between them makes the compiler
  // wait for every load in flight before the reads)
  auto issue_loads = [&](char *stage) {
#pragma unroll
    for (int q = 0; q < NAQ; ++q) dma16(src + kl + a_off[q], (lds_void *)(stage + a_dst[q]));
#pragma unroll
    for (int j = 0; j < 2; ++j)
      dma16(w_row[j] + (long)ki * QBK, (lds_void *)(stage + 2 * QSA + (2 * wave + j) * 1024));
    __builtin_amdgcn_global_load_lds(s_row + 2 * ki, (lds_void *)(stage + 2 * QSA + QSW + wave * 256), 4, 0, 0);
  };
  auto advance = [&]() {
    if (ki + 1 < nk) {   // past the last k-step the same one is issued again
      ++ki;
      kl += QBK;
      if (kl == kps) {
        kl = 0;
        ++src_i;
        src = reinterpret_cast<const bf16 *>(pick(A.ptr, src_i));
      }
    }
  };

  f32x4 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = zero4();

#pragma unroll
  for (int s = 0; s < Q8STAGES - 1; ++s) {
    issue_loads(smem_q8 + s * QSB);
    advance();
  }

  const int ar = wm * 64 + r16, br = wn * CW + r16;
  for (int kt = 0; kt < nk; ++kt) {
    wait_vm<QLPS * (Q8STAGES - 2)>();   // this wave's loads of stage kt have landed
    ring_barrier();                      // ... everyone's; stage kt-1 is no longer read
    issue_loads(smem_q8 + ((kt + Q8STAGES - 1) % Q8STAGES) * QSB);
    const char *st = smem_q8 + (kt % Q8STAGES) * QSB;
    const char *wq = st + 2 * QSA;
    // scales of rows br + 16 j: dwords 4 (wn 16 + r16) + j
    const u32x4 sv = *reinterpret_cast<const u32x4 *>(wq + QSW + (wn * 16 + r16) * 16);
    float sc[NJ][2];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      sc[j][0] = half_bits_to_f32((uint16_t)(sv[j] & 0xffffu));
      sc[j][1] = half_bits_to_f32((uint16_t)(sv[j] >> 16));
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bf16 *as = reinterpret_cast<const bf16 *>(st + h * QSA);
      Frag<bf16> fa[MI], fb[NJ];
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int row = ar + 16 * i;
        fa[i] = load_frag(as + row * 32 + 8 * dslot(row, g));
      }
      // codes 32 h + 8 g ... + 7 of the row: half g & 1 of chunk 2 h + g / 2
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int row = br + 16 * j;
        const u32x4 c = *reinterpret_cast<const u32x4 *>(wq + row * QBK + 16 * dslot(row, 2 * h + (g >> 1)));
        fb[j] = dequant8((g & 1) ? make_uint2(c[2], c[3]) : make_uint2(c[0], c[1]), sc[j][h]);
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) mma(acc[i][j], fa[i], fb[j]);
    }
    advance();
  }
  wait_vm<0>();
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int n = n0 + wn * CW + 16 * j + r16;
      if (n >= W.n_total) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + wm * 64 + 16 * i + 4 * g + v;
        if (m < M) {
          if constexpr (SPLIT)
            part[((long)blockIdx.y * M + m) * W.n_total + n] = acc[i][j][v];
          else
            store_out_m<bf16, OM>(o, m, n, acc[i][j][v]);
        }
      }
    }
}

// One workgroup per CU (the ring takes 104 or 136 KB of LDS), so the grid is
// sized to one pass over kQ8Wgs CUs.  64-row tiles (each code dequantised by
// one wave) while they still leave a k-split of at least two over those CUs
// (measured on the Q8_0 workload's fc: 24 rows 103 -> 73 us, 192 rows
// 177 -> 147 us; at 512 rows the 168 unsplit 64-row tiles took 413 us
// against 306 for 128-row tiles split three ways).
constexpr int kQ8Wgs = 256;
static int q8_tbm(int M, int N) {
  const long nt = (N + DBN - 1) / DBN;
  return (long)((M + 63) / 64) * nt * 2 <= kQ8Wgs ? 64 : 128;
}

// k-split of the Q8_0 tiles
static int dma8q_plan(int M, int N, int K, int *kc) {
  const int tbm = q8_tbm(M, N);
  const long tiles = (long)((N + DBN - 1) / DBN) * ((M + tbm - 1) / tbm);
  const int nk = K / QBK;
  int S = (int)std::max(1L, kQ8Wgs / tiles);
  S = std::min(S, std::max(1, nk / 4));
  S = std::min(S, 64);
  const int kcq = (nk + S - 1) / S;
  S = (nk + kcq - 1) / kcq;
  *kc = kcq * QBK;
  return S;
}

template <int OM, int TBM, bool SPLIT, int MI>
static hipError_t dma8q_go1(const ASrc &A, int M, const WSet &W, const OutSpec &out, float *part, int kc,
                            int S, hipStream_t st) {
  const int mt = (M + TBM - 1) / TBM, nt = (W.n_total + DBN - 1) / DBN;
  const size_t lds = (size_t)q8_stages<TBM>() * q8_stage_bytes<TBM>();
  auto *k = &dma8q_gemm_kernel<OM, TBM, SPLIT, MI>;
  const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void *>(k), lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3(mt * nt, S), dim3(512), lds, st, A, M, W, out, kc, part);
  if (SPLIT) {
    const long mn = (long)M * W.n_total;
    hipLaunchKernelGGL((tile_reduce_kernel<bf16, OM>), dim3((unsigned)((mn + 255) / 256)), dim3(256), 0, st,
                       part, S, M, W.n_total, out);
  }
  return hipSuccess;
}

template <int OM, int TBM, int MI>
static hipError_t dma8q_go_t(const ASrc &A, int M, const WSet &W, const OutSpec &out, float *part,
                             hipStream_t st) {
  int kc = 0;
  const int S = part ? dma8q_plan(M, W.n_total, W.K, &kc) : 1;
  return S > 1 ? dma8q_go1<OM, TBM, true, MI>(A, M, W, out, part, kc, S, st)
               : dma8q_go1<OM, TBM, false, MI>(A, M, W, out, nullptr, 0, 1, st);
}

template <int OM>
static hipError_t dma8q_go(const ASrc &A, int M, const WSet &W, const OutSpec &out, float *part,
                           hipStream_t st) {
  if (q8_tbm(M, W.n_total) == 128) return dma8q_go_t<OM, 128, 4>(A, M, W, out, part, st);
  return M <= 32 ? dma8q_go_t<OM, 64, 2>(A, M, W, out, part, st) : dma8q_go_t<OM, 64, 4>(A, M, W, out, part, st);
}

// Q8_0 weights through the ring above: bf16 activations, k-ranges of whole
// 64-wide steps that never straddle two activation sources
static bool dma8q_ok(int act, int wkind, const ASrc &A, const WSet &W) {
  return act == ACT_BF16 && wkind == W_Q8_0 && W.K % QBK == 0 && A.k_per_src % QBK == 0;
}

// Q8_0 -> bf16 expansion: one thread per 32-code block (two 16-byte code
// loads, one scale, four 16-byte stores), consecutive threads on consecutive
// blocks of a row, so reads and writes are both contiguous.
__global__ __launch_bounds__(256) void expand_q8_kernel(const int8_t *__restrict__ codes,
                                                        const uint16_t *__restrict__ scales,
                                                        long n_blocks, bf16 *__restrict__ out) {
  const long b = (long)blockIdx.x * 256 + threadIdx.x;
  if (b >= n_blocks) return;
  const uint4 *src = reinterpret_cast<const uint4 *>(codes + 32 * b);
  const uint4 c0 = src[0], c1 = src[1];
  const float s = half_bits_to_f32(scales[b]);
  bf16x8 *dst = reinterpret_cast<bf16x8 *>(out + 32 * b);
  dst[0] = dequant8(make_uint2(c0.x, c0.y), s).v;
  dst[1] = dequant8(make_uint2(c0.z, c0.w), s).v;
  dst[2] = dequant8(make_uint2(c1.x, c1.y), s).v;
  dst[3] = dequant8(make_uint2(c1.z, c1.w), s).v;
}

hipError_t launch_expand_q8(const void *codes, const void *scales, long rows, int cols, void *out,
                            hipStream_t st) {
  // blocks run along a row and rows are contiguous, so block b of the whole
  // weight has its codes at 32 b and its scale at index b of [rows][cols/32]
  const long nb = rows * (long)(cols / 32);
  if (nb > 0)
    hipLaunchKernelGGL(expand_q8_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, st,
                       static_cast<const int8_t *>(codes), static_cast<const uint16_t *>(scales), nb,
                       static_cast<bf16 *>(out));
  return hipGetLastError();
}

hipError_t launch_tile_gemm(int act, int wkind, const ASrc &A, int M, const WSet &W,
                            const OutSpec &out, float *part, hipStream_t st) {
  // 256 x 256 tiles while they give every CU two workgroups; a narrow
  // product (the batched conv's delta, N = 256) takes 128 x 256 tiles while
  // those still cover the CUs, and the 128 x 128 tile kernel below that
  const long cus = device_cu_count();
  const long tiles256 = (long)((M + 255) / 256) * ((W.n_total + 255) / 256);
  const long tiles128 = (long)((M + 127) / 128) * ((W.n_total + 255) / 256);
  const bool big = M >= DFL_BIG_GEMM_MIN_M && tiles256 >= 2 * cus;
  const bool half = M >= DFL_HALF_GEMM_MIN_M && !big && tiles128 * DFL_HALF_GEMM_FILL >= cus;
  // the last wave of 128 x 256 tiles less than three quarters full: split k
  const long tail = tiles128 % cus;
  const bool ragged = tail != 0 && tail * 4 < cus * 3;
  hipError_t e = hipSuccess;
  if (act == ACT_F32)
    tile_launch_t<float, W_SAME>(A, M, W, out, part, st);
  else if (dma8q_ok(act, wkind, A, W)) {   // fewer rows than kQ8ExpandMinM: codes in the ring
    if (out.mode == OUT_F32) e = dma8q_go<OUT_F32>(A, M, W, out, part, st);
    else if (out.mode == OUT_ACT) e = dma8q_go<OUT_ACT>(A, M, W, out, part, st);
    else e = dma8q_go<OUT_CACHE>(A, M, W, out, part, st);
  } else if (wkind == W_Q8_0)   // the callers keep K and the sources to multiples of 64
    return hipErrorInvalidValue;
  else if (!big && (!half || ragged) && dma8_split_launch(A, M, W, out, part, st, &e))
    return e != hipSuccess ? e : hipGetLastError();
  else if (big)
    e = dma8_launch<256>(A, M, W, out, st);
  else if (half)
    e = dma8_launch<128>(A, M, W, out, st);
  else
    tile_launch_t<bf16, W_SAME>(A, M, W, out, part, st);
  return e != hipSuccess ? e : hipGetLastError();
}

}  // namespace dfl
