// The small kernels of the draft block step: the injection RMSNorm, the
// DFlash2 grouped dynamic depthwise convolution, the candidate-selector
// edges with their best-path readout, and the greedy accept length.
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "merge.h"
#include "stream.h"

namespace dfl {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor(v, m);
  return v;
}

// ---------------------------------------------------------------------------
// RMSNorm (encoder norm, "dflash: port #219 onto feature", Root Cause):
// z = y / sqrt(mean(y^2) + eps) * gamma, one workgroup per row, fixed-order sum.
// ---------------------------------------------------------------------------
template <typename TA>
__device__ __forceinline__ void rmsnorm_store4(TA *zr, int c, f32x4 v, float inv, const TA *gamma) {
  float o[4] = {v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv};
  if (gamma) {
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] *= to_f32(gamma[c + j]);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) zr[c + j] = from_f32<TA>(o[j]);
}

// Rows up to kRmsHeld float4 per thread (8192 wide) are read once into
// registers, every load issued before the first is used; wider rows are
// read twice (the second time from the cache).
constexpr int kRmsHeld = 8;

template <typename TA>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float *__restrict__ y, int d,
                                                      const TA *__restrict__ gamma, float eps,
                                                      TA *__restrict__ z) {
  const long row = blockIdx.x;
  const int tid = threadIdx.x;
  const float *yr = y + row * d;
  const f32x4 *yv = reinterpret_cast<const f32x4 *>(yr);
  const int nv = d / 4;
  const bool held = nv <= kRmsHeld * 256;
  f32x4 v[kRmsHeld];
  float ss = 0.f;
  if (held) {
#pragma unroll
    for (int j = 0; j < kRmsHeld; ++j)
      if (j * 256 < nv) v[j] = yv[min(tid + j * 256, nv - 1)];
#pragma unroll
    for (int j = 0; j < kRmsHeld; ++j)
      if (j * 256 < nv && tid + j * 256 < nv)
        ss += v[j][0] * v[j][0] + v[j][1] * v[j][1] + v[j][2] * v[j][2] + v[j][3] * v[j][3];
  } else {
    for (int c = tid; c < nv; c += 256) {
      const f32x4 t = yv[c];
      ss += t[0] * t[0] + t[1] * t[1] + t[2] * t[2] + t[3] * t[3];
    }
  }
  __shared__ float red[4];
  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float inv = 1.0f / sqrtf(tot / (float)d + eps);
  TA *zr = z + row * d;
  if (held) {
#pragma unroll
    for (int j = 0; j < kRmsHeld; ++j)
      if (j * 256 < nv && tid + j * 256 < nv) rmsnorm_store4<TA>(zr, 4 * (tid + j * 256), v[j], inv, gamma);
  } else {
    for (int c = tid; c < nv; c += 256) rmsnorm_store4<TA>(zr, 4 * c, yv[c], inv, gamma);
  }
}

hipError_t launch_rmsnorm(int act, const float *y, int n, int d, const void *gamma, float eps,
                          void *z, hipStream_t st) {
  if (act == ACT_F32)
    hipLaunchKernelGGL((rmsnorm_kernel<float>), dim3(n), dim3(256), 0, st, y, d,
                       reinterpret_cast<const float *>(gamma), eps, reinterpret_cast<float *>(z));
  else
    hipLaunchKernelGGL((rmsnorm_kernel<bf16>), dim3(n), dim3(256), 0, st, y, d,
                       reinterpret_cast<const bf16 *>(gamma), eps, reinterpret_cast<bf16 *>(z));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Q8_0 KV-cache rows ("dflash: port #219 onto feature", DFlash Benchmark
// Sweep: q8_0 K and V caches).  One thread per (row, K or V, head, block of 32
// head dims): scale d = max|x| / 127 of the fp32 projection output, stored as
// fp16; codes round-half-away(x / d) (x * (1 / d) in fp32), all 0 for a zero
// block.  K codes land as 32 contiguous bytes of the key's row, V codes in
// the transposed 32-position panels (one byte per dim row).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kv_quant_kernel(const float *__restrict__ kv, int n, int Hkv,
                                                       int hd, long cap, long pos0,
                                                       int8_t *__restrict__ ck, int8_t *__restrict__ cv,
                                                       _Float16 *__restrict__ cks,
                                                       _Float16 *__restrict__ cvs) {
  const int nb = hd >> 5, per_row = 2 * Hkv * nb;
  const long id = (long)blockIdx.x * 256 + threadIdx.x;
  if (id >= (long)n * per_row) return;
  const int t = (int)(id / per_row);
  const int r = (int)(id - (long)t * per_row);
  const int isv = r / (Hkv * nb), hb = r - isv * Hkv * nb;
  const int h = hb / nb, b = hb - h * nb;
  const f32x4 *src = reinterpret_cast<const f32x4 *>(kv + (long)t * 2 * Hkv * hd + (long)isv * Hkv * hd +
                                                     (long)h * hd + 32 * b);
  f32x4 x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = src[j];
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(x[j][i]));
  const float d = amax / 127.f;
  const float inv = d != 0.f ? 1.f / d : 0.f;
  int8_t q[32];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float c = fminf(fmaxf(roundf(x[j][i] * inv), -127.f), 127.f);
      q[4 * j + i] = (int8_t)(int)c;
    }
  const long pos = pos0 + t;
  const long srow = ((long)h * cap + pos) * nb + b;
  if (!isv) {
    uint4 w[2];
    __builtin_memcpy(w, q, 32);
    uint4 *dst = reinterpret_cast<uint4 *>(ck + ((long)h * cap + pos) * hd + 32 * b);
    dst[0] = w[0];
    dst[1] = w[1];
    cks[srow] = (_Float16)d;
  } else {
    int8_t *panel = cv + ((long)h * (cap >> 5) + (pos >> 5)) * hd * 32 + (pos & 31);
#pragma unroll
    for (int j = 0; j < 32; ++j) panel[(long)(32 * b + j) * 32] = q[j];
    cvs[srow] = (_Float16)d;
  }
}

hipError_t launch_kv_quant(const float *kv, int n, int Hkv, int hd, long cap, long pos0, void *ck,
                           void *cv, void *cks, void *cvs, hipStream_t st) {
  const long threads = (long)n * 2 * Hkv * (hd / 32);
  hipLaunchKernelGGL(kv_quant_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, kv, n, Hkv,
                     hd, cap, pos0, static_cast<int8_t *>(ck), static_cast<int8_t *>(cv),
                     static_cast<_Float16 *>(cks), static_cast<_Float16 *>(cvs));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Gated MLP activation of the feed-forward site: act[m][j] = silu(g) * p with
// g = gu[m][j], p = gu[m][F + j] (the stacked gate | up product, fp32),
// SiLU(x) = x / (1 + e^-x), rounded once to the activation type.  One thread
// per 4 adjacent j: two 16-byte loads, four outputs.
// ---------------------------------------------------------------------------
template <typename TA>
__global__ __launch_bounds__(256) void silu_mul_kernel(const float *__restrict__ gu, long M, int F,
                                                       TA *__restrict__ out) {
  const long q = F / 4;
  const long id = (long)blockIdx.x * 256 + threadIdx.x;
  if (id >= M * q) return;
  const long m = id / q;
  const int j = (int)(id - m * q) * 4;
  const float *row = gu + m * 2 * (long)F;
  const f32x4 g = *reinterpret_cast<const f32x4 *>(row + j);
  const f32x4 p = *reinterpret_cast<const f32x4 *>(row + F + j);
#pragma unroll
  for (int i = 0; i < 4; ++i) out[m * F + j + i] = from_f32<TA>(g[i] / (1.f + expf(-g[i])) * p[i]);
}

hipError_t launch_silu_mul(int act, const float *gu, long M, int F, void *out, hipStream_t st) {
  const long threads = M * (F / 4);
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (act == ACT_F32)
    hipLaunchKernelGGL((silu_mul_kernel<float>), grid, dim3(256), 0, st, gu, M, F, static_cast<float *>(out));
  else
    hipLaunchKernelGGL((silu_mul_kernel<bf16>), grid, dim3(256), 0, st, gu, M, F, static_cast<bf16 *>(out));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Grouped dynamic depthwise conv ("spec : add DFlash2 support", Overview):
// out[i,c] = sum_t (base[t,c] + delta[i, t*G + g(c)]) * x[i-t, c], x[<0] = 0.
// One thread per (block, 8 adjacent channels): it loads the block's B input
// rows of its channels (16-byte loads) and the T base rows once, then forms
// the B outputs from registers, so x is read exactly once and a batch of
// blocks is a pure stream.  Every load is issued before the first use, with
// no branch between them, so a thread waits for memory once:
//   DM = 1: C/G a multiple of 8, the 8 channels share one group, one delta
//           value per (position, tap);
//   DM = 2: C/G >= 8, the 8 channels span at most two groups, two values per
//           (position, tap) and a per-channel select;
//   DM = 0: anything else (or T > 4), eight loads per (position, tap), issued
//           where they are used.
// BM >= B bounds the positions a thread walks (8 or 16).
// ---------------------------------------------------------------------------
template <typename TA, int TM, int DM, int BM>
__global__ __launch_bounds__(256) void conv_kernel(const TA *__restrict__ x, int n_blocks, int B,
                                                   int C, int G, int T,
                                                   const TA *__restrict__ base,
                                                   const float *__restrict__ delta,
                                                   TA *__restrict__ out) {
  const int nch = C >> 3;
  const long id = (long)blockIdx.x * 256 + threadIdx.x;
  const long blk = id / nch;
  if (blk >= n_blocks) return;
  const int c = (int)(id - blk * nch) * 8;
  const int cpg = C / G;
  // group of each channel: g(c) = c / cpg, one division, then boundaries
  int gj[8];
  {
    int g = c / cpg, next = (g + 1) * cpg;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (c + j >= next) {
        ++g;
        next += cpg;
      }
      gj[j] = g;
    }
  }
  const TA *xb = x + blk * (long)B * C + c;
  Frag<TA> xr[BM];
#pragma unroll
  for (int i = 0; i < BM; ++i) xr[i] = load_frag(xb + (long)min(i, B - 1) * C);   // rows >= B unused
  // base taps held in registers up to 8 taps; longer filters re-read them
  // from cache per use (registers would otherwise spill)
  constexpr int TR = TM <= 8 ? TM : 1;
  Frag<TA> bv[TR];
#pragma unroll
  for (int t = 0; t < TR; ++t) bv[t] = load_frag(base + (long)min(t, T - 1) * C + c);
  const int TG = T * G;
  const float *db = delta + blk * (long)B * TG;   // this block's delta rows
  constexpr int DI = DM ? BM : 1, DT = DM ? TM : 1;
  float dA[DI][DT], dB[DM == 2 ? DI : 1][DM == 2 ? DT : 1];
  if constexpr (DM != 0) {
#pragma unroll
    for (int i = 0; i < BM; ++i)
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        const float *r = db + (long)min(i, B - 1) * TG + min(t, T - 1) * G;
        dA[i][t] = r[gj[0]];
        if constexpr (DM == 2) dB[i][t] = r[gj[7]];
      }
  }
#pragma unroll
  for (int i = 0; i < BM; ++i) {
    if (i < B) {   // guard, not break: keeps the loop fully unrolled (static register indices)
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        if (t < T && t <= i) {
          float dv[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            if constexpr (DM == 1)
              dv[j] = dA[i][t];
            else if constexpr (DM == 2)
              dv[j] = gj[j] == gj[0] ? dA[i][t] : dB[i][t];
            else
              dv[j] = db[(long)i * TG + t * G + gj[j]];
          }
          const Frag<TA> b = TM <= 8 ? bv[t < TR ? t : 0] : load_frag(base + (long)t * C + c);
#pragma unroll
          for (int j = 0; j < 8; ++j)
            acc[j] += (to_f32(b.v[j]) + dv[j]) * to_f32(xr[i - t].v[j]);
        }
      }
      Frag<TA> o;
#pragma unroll
      for (int j = 0; j < 8; ++j) o.v[j] = from_f32<TA>(acc[j]);
      store_frag(out + (blk * B + i) * (long)C + c, o);
    }
  }
}

// Few blocks (one draft block per step): one thread per (position, 8
// channels), so a single block still spreads over B*C/8 threads; the T input
// rows a position needs are re-read from cache by neighbouring positions.
template <typename TA, int TM, int DM>
__global__ __launch_bounds__(256) void conv_pos_kernel(const TA *__restrict__ x, int n_blocks, int B,
                                                       int C, int G, int T,
                                                       const TA *__restrict__ base,
                                                       const float *__restrict__ delta,
                                                       TA *__restrict__ out) {
  const int nch = C >> 3;
  const long id = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = id / nch;   // blk * B + i
  if (row >= (long)n_blocks * B) return;
  const int c = (int)(id - row * nch) * 8;
  const int i = (int)(row % B);
  const int cpg = C / G;
  int gj[8];
  {
    int g = c / cpg, next = (g + 1) * cpg;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (c + j >= next) {
        ++g;
        next += cpg;
      }
      gj[j] = g;
    }
  }
  const int TG = T * G;
  const float *dr = delta + row * (long)TG;
  Frag<TA> xr[TM], bv[TM];
  float dA[TM], dB[DM == 2 ? TM : 1];
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    const int tt = min(t, min(T - 1, i));   // taps past the block start or T read a valid row, unused
    xr[t] = load_frag(x + (row - tt) * (long)C + c);
    bv[t] = load_frag(base + (long)min(t, T - 1) * C + c);
    if constexpr (DM != 0) {
      dA[t] = dr[min(t, T - 1) * G + gj[0]];
      if constexpr (DM == 2) dB[t] = dr[min(t, T - 1) * G + gj[7]];
    }
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    if (t < T && t <= i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float dv;
        if constexpr (DM == 1)
          dv = dA[t];
        else if constexpr (DM == 2)
          dv = gj[j] == gj[0] ? dA[t] : dB[t];
        else
          dv = dr[t * G + gj[j]];
        acc[j] += (to_f32(bv[t].v[j]) + dv) * to_f32(xr[t].v[j]);
      }
    }
  }
  Frag<TA> o;
#pragma unroll
  for (int j = 0; j < 8; ++j) o.v[j] = from_f32<TA>(acc[j]);
  store_frag(out + row * (long)C + c, o);
}

template <typename TA, int TM, int DM>
static void conv_pos_go(const TA *x, int n_blocks, int B, int C, int G, int T, const TA *base,
                        const float *delta, TA *out, hipStream_t st) {
  const long threads = (long)n_blocks * B * (C / 8);
  hipLaunchKernelGGL((conv_pos_kernel<TA, TM, DM>), dim3((unsigned)((threads + 255) / 256)), dim3(256),
                     0, st, x, n_blocks, B, C, G, T, base, delta, out);
}

template <typename TA, int TM, int DM, int BM>
static void conv_go(dim3 grid, const TA *x, int n_blocks, int B, int C, int G, int T, const TA *base,
                    const float *delta, TA *out, hipStream_t st) {
  hipLaunchKernelGGL((conv_kernel<TA, TM, DM, BM>), grid, dim3(256), 0, st, x, n_blocks, B, C, G, T,
                     base, delta, out);
}

template <typename TA, int BM>
static void conv_launch_bm(dim3 grid, const TA *x, int n_blocks, int B, int C, int G, int T,
                           const TA *base, const float *delta, TA *out, hipStream_t st) {
  const int cpg = C / G;
  if (T <= 4 && cpg % 8 == 0)
    conv_go<TA, 4, 1, BM>(grid, x, n_blocks, B, C, G, T, base, delta, out, st);
  else if (T <= 4 && cpg >= 8)
    conv_go<TA, 4, 2, BM>(grid, x, n_blocks, B, C, G, T, base, delta, out, st);
  else if (T <= 4)
    conv_go<TA, 4, 0, BM>(grid, x, n_blocks, B, C, G, T, base, delta, out, st);
  else if (T <= 8)
    conv_go<TA, 8, 0, BM>(grid, x, n_blocks, B, C, G, T, base, delta, out, st);
  else
    conv_go<TA, 16, 0, BM>(grid, x, n_blocks, B, C, G, T, base, delta, out, st);
}

template <typename TA>
static void conv_launch_t(const void *x, int n_blocks, int B, int C, int G, int T, const void *base,
                          const float *delta, void *out, hipStream_t st) {
  const long threads = (long)n_blocks * (C / 8);
  const dim3 grid((unsigned)((threads + 255) / 256));
  const TA *xp = reinterpret_cast<const TA *>(x);
  const TA *bp = reinterpret_cast<const TA *>(base);
  TA *op = reinterpret_cast<TA *>(out);
  const int cpg = C / G;
  if (grid.x < 64 && T <= 8) {   // too few workgroups to walk whole blocks: spread the positions
    if (T <= 4 && cpg % 8 == 0)
      conv_pos_go<TA, 4, 1>(xp, n_blocks, B, C, G, T, bp, delta, op, st);
    else if (T <= 4 && cpg >= 8)
      conv_pos_go<TA, 4, 2>(xp, n_blocks, B, C, G, T, bp, delta, op, st);
    else if (T <= 4)
      conv_pos_go<TA, 4, 0>(xp, n_blocks, B, C, G, T, bp, delta, op, st);
    else
      conv_pos_go<TA, 8, 0>(xp, n_blocks, B, C, G, T, bp, delta, op, st);
    return;
  }
  if (B <= 8)
    conv_launch_bm<TA, 8>(grid, xp, n_blocks, B, C, G, T, bp, delta, op, st);
  else
    conv_launch_bm<TA, 16>(grid, xp, n_blocks, B, C, G, T, bp, delta, op, st);
}

// ---------------------------------------------------------------------------
// One block's conv in one launch.  A tile is gpt = 16 / T groups: its 16
// MFMA rows are the W_delta rows t*G + g of those groups (lane row r16 =
// (g - g0) * T + t; rows past gpt * T re-read row t*G + g0 and are dropped),
// so a tile holds every tap of its groups.  Workgroup (tile, y): its 8 waves
// stream consecutive k-ranges of kchunk, summed in LDS in a fixed pairwise
// order; with several k-groups each writes a partial and the last to finish
// (completion counter cnt[tile]) sums them in k-group order, as the small
// skinny GEMMs do.  That workgroup then applies the taps to the tile's
// columns: one thread per (row, CV columns of one group; CV = 8, or 4 when
// C / G is a multiple of 4 only), the same arithmetic in the same order as
// conv_pos_kernel.
// ---------------------------------------------------------------------------
struct ConvFusedArgs {
  const void *x, *base, *wd;
  void *out;
  float *part;
  unsigned long long *cnt, stamp;
  int M, B, C, G, T, gpt, kchunk;
};

constexpr int kConvFusedWaves = 8;

static void conv_fused_plan(int C, int G, int T, int *gpt, int *ntile, int *kchunk, int *kgroups) {
  *gpt = std::max(1, 16 / T);
  *ntile = (G + *gpt - 1) / *gpt;
  int kw = (2048 + *ntile - 1) / *ntile;   // waves per tile
  const int kw_max = (C + 127) / 128;
  kw = std::max(kConvFusedWaves, std::min(kw, kw_max));
  int kc = (C + kw - 1) / kw;
  kc = std::max(128, (kc + 63) / 64 * 64);
  *kchunk = kc;
  *kgroups = (C + kConvFusedWaves * kc - 1) / (kConvFusedWaves * kc);
}

bool conv_fused_ok(int M, int C, int G, int T) { return M <= 16 && (C / G) % 4 == 0 && T <= 16; }

size_t conv_fused_part_bytes(int M, int C, int G, int T) {
  if (!conv_fused_ok(M, C, G, T)) return 0;
  int gpt, ntile, kc, kg;
  conv_fused_plan(C, G, T, &gpt, &ntile, &kc, &kg);
  return kg > 1 ? (size_t)kg * ntile * 64 * sizeof(f32x4) : 0;
}

// CV consecutive elements of a row (8, 16 or 32 bytes) as 8- or 16-byte
// accesses
template <typename TA, int CV>
struct CVec {
  TA v[CV];
};
template <typename TA, int CV>
__device__ __forceinline__ CVec<TA, CV> cvec_load(const TA *p) {
  constexpr int NB = CV * (int)sizeof(TA);
  static_assert(NB == 8 || NB == 16 || NB == 32, "8, 16 or 32 bytes");
  if constexpr (NB == 8) {
    return __builtin_bit_cast(CVec<TA, CV>, *reinterpret_cast<const uint2 *>(p));
  } else {
    struct W { u32x4 q[NB / 16]; } w;
#pragma unroll
    for (int i = 0; i < NB / 16; ++i) w.q[i] = reinterpret_cast<const u32x4 *>(p)[i];
    return __builtin_bit_cast(CVec<TA, CV>, w);
  }
}
template <typename TA, int CV>
__device__ __forceinline__ void cvec_store(TA *p, const CVec<TA, CV> &c) {
  constexpr int NB = CV * (int)sizeof(TA);
  if constexpr (NB == 8) {
    *reinterpret_cast<uint2 *>(p) = __builtin_bit_cast(uint2, c);
  } else {
    struct W { u32x4 q[NB / 16]; };
    const W w = __builtin_bit_cast(W, c);
#pragma unroll
    for (int i = 0; i < NB / 16; ++i) reinterpret_cast<u32x4 *>(p)[i] = w.q[i];
  }
}

template <typename TA, int CV>
__global__ __launch_bounds__(kConvFusedWaves * 64) void conv_fused_kernel(ConvFusedArgs a) {
  __shared__ f32x4 red[kConvFusedWaves][64];
  __shared__ float dl[16][16];   // delta of the tile: [row][lane row r16]
  __shared__ unsigned last;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int M = a.M, C = a.C, G = a.G, T = a.T, gpt = a.gpt;
  const int tile = blockIdx.x, g0 = tile * gpt;
  const int ng = min(gpt, G - g0);   // groups of this tile
  // this lane's W_delta row
  const int gl = r16 / T, tl = r16 - gl * T;
  const int wrow = tl * G + g0 + (gl < ng ? gl : 0);
  const int k0 = (blockIdx.y * kConvFusedWaves + wave) * a.kchunk, k1 = min(C, k0 + a.kchunk);
  f32x4 acc[1] = {zero4()};
  if (k0 < k1) {
    const SRow<TA, W_SAME> rows[1] = {srow<TA, W_SAME>(a.wd, nullptr, wrow, C)};
    const TA *xr = reinterpret_cast<const TA *>(a.x) + (long)min(r16, M - 1) * C;
    stream_k<TA, W_SAME, 1>(xr, rows, 1, k0, k1, g, r16 < M, acc);
  }
  red[wave][lane] = acc[0];
  __syncthreads();
  f32x4 v = zero4();
  if (wave == 0) {
    f32x4 t[kConvFusedWaves];
#pragma unroll
    for (int w = 0; w < kConvFusedWaves; ++w) t[w] = red[w][lane];
#pragma unroll
    for (int h = kConvFusedWaves / 2; h >= 1; h /= 2)
#pragma unroll
      for (int w = 0; w < h; ++w)
#pragma unroll
        for (int i = 0; i < 4; ++i) t[w][i] += t[w + h][i];
    v = t[0];
  }
  const int nky = gridDim.y;
  if (nky > 1) {
    const long tstride = (long)gridDim.x * 64;   // float4 per k-group
    if (wave == 0) {
      float *pp = a.part + (((long)blockIdx.y * tstride) + (long)tile * 64 + lane) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) __hip_atomic_store(pp + i, v[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // the partial stores have completed before the arrival counts
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      const bool l = arrive_last(&a.cnt[tile], a.stamp, nky);
      if (l) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      last = l;
    }
    __syncthreads();
    if (!last) return;
    if (wave == 0) {
      // the partials happen-before these loads (release by every arrival,
      // acquire above): ordinary 16-byte loads, eight in flight
      const f32x4 *src = reinterpret_cast<const f32x4 *>(a.part) + (long)tile * 64 + lane;
      v = zero4();
      for (int y0 = 0; y0 < nky; y0 += 8) {
        f32x4 x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = src[(long)min(y0 + j, nky - 1) * tstride];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (y0 + j < nky) {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] += x[j][i];
          }
      }
    }
  }
  // lane (g, r16) holds delta[row r16][lane row 4 g + i]
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) dl[r16][4 * g + i] = v[i];
  }
  __syncthreads();

  // the taps on this tile's columns [g0 cpg, (g0 + ng) cpg): one thread per
  // (row, CV columns of one group)
  const int cpg = C / G, vpg = cpg / CV, nvec = M * ng * vpg;
  const TA *xp = reinterpret_cast<const TA *>(a.x);
  const TA *bp = reinterpret_cast<const TA *>(a.base);
  for (int e = tid; e < nvec; e += kConvFusedWaves * 64) {
    const int row = e / (ng * vpg), rem = e - row * (ng * vpg), gq = rem / vpg;
    const int c = (g0 + gq) * cpg + (rem - gq * vpg) * CV;
    const int i = row % a.B;
    float oc[CV];
#pragma unroll
    for (int j = 0; j < CV; ++j) oc[j] = 0.f;
    // taps in fours, their loads issued together; t ascending
    for (int t0 = 0; t0 < T; t0 += 4) {
      CVec<TA, CV> xr[4], bv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = min(t0 + u, T - 1), tt = min(t, i);   // taps past T or the block start: valid rows, unused
        xr[u] = cvec_load<TA, CV>(xp + (long)(row - tt) * C + c);
        bv[u] = cvec_load<TA, CV>(bp + (long)t * C + c);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = t0 + u;
        if (t < T && t <= i) {
          const float dv = dl[row][gq * T + t];
#pragma unroll
          for (int j = 0; j < CV; ++j) oc[j] += (to_f32(bv[u].v[j]) + dv) * to_f32(xr[u].v[j]);
        }
      }
    }
    CVec<TA, CV> o;
#pragma unroll
    for (int j = 0; j < CV; ++j) o.v[j] = from_f32<TA>(oc[j]);
    cvec_store<TA, CV>(reinterpret_cast<TA *>(a.out) + (long)row * C + c, o);
  }
}

hipError_t launch_conv_fused(int act, const void *x, int n_blocks, int B, int C, int G, int T,
                             const void *base, const void *wd, void *out, float *part,
                             unsigned long long *cnt, hipStream_t st) {
  const int M = n_blocks * B;
  if (!conv_fused_ok(M, C, G, T)) return hipErrorInvalidValue;
  ConvFusedArgs a;
  int ntile, kg;
  conv_fused_plan(C, G, T, &a.gpt, &ntile, &a.kchunk, &kg);
  if (kg > 1 && (!part || !cnt || ntile > kMaxCounters)) return hipErrorInvalidValue;
  a.x = x;
  a.base = base;
  a.wd = wd;
  a.out = out;
  a.part = part;
  a.cnt = cnt;
  a.stamp = kg > 1 ? next_launch_stamp() : 0;
  a.M = M;
  a.B = B;
  a.C = C;
  a.G = G;
  a.T = T;
  const dim3 grid(ntile, kg), block(kConvFusedWaves * 64);
  const bool c8 = (C / G) % 8 == 0;
  if (act == ACT_F32) {
    if (c8) hipLaunchKernelGGL((conv_fused_kernel<float, 8>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((conv_fused_kernel<float, 4>), grid, block, 0, st, a);
  } else {
    if (c8) hipLaunchKernelGGL((conv_fused_kernel<bf16, 8>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((conv_fused_kernel<bf16, 4>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_conv(int act, const void *x, int n_blocks, int B, int C, int G, int T,
                       const void *base, const float *delta, void *out, hipStream_t st) {
  if (act == ACT_F32)
    conv_launch_t<float>(x, n_blocks, B, C, G, T, base, delta, out, st);
  else
    conv_launch_t<bf16>(x, n_blocks, B, C, G, T, base, delta, out, st);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Candidate-selector edges and max-sum path ("spec : add DFlash2 support",
// Overview): edge(p -> c) = < A[p] (.) proj(h), B[c] > + unary[c].
// selector_edges_kernel: one workgroup per position i stages its K candidate
// rows of B and its predecessor rows of A (scaled by proj[i]) in LDS and forms
// the K x K rank-r dot products.  selector_path_kernel: one workgroup runs
// the K-state max-sum recursion over the positions and the backtrack.  When
// all candidate rows fit in LDS, selector_fused_kernel does both at once.
// ---------------------------------------------------------------------------
constexpr int kSelMaxB = 16, kSelMaxK = 32, kSelMaxR = 256;

__device__ __forceinline__ int clamp_idx(int v, long V) {
  return v < 0 ? 0 : (v >= V ? (int)(V - 1) : v);   // never read out of bounds
}

template <typename TA>
__global__ __launch_bounds__(256) void selector_edges_kernel(SelArgs a) {
  extern __shared__ float sm[];
  const int tid = threadIdx.x;
  const int i = blockIdx.x, K = a.K, r = a.r, rl = a.r + 1;   // +1: LDS bank spread
  float *ap = sm;                 // [K][r+1]  A[pred] * proj[i]
  float *bp = sm + K * rl;        // [K][r+1]  B[cand]
  const TA *A = reinterpret_cast<const TA *>(a.cb_pred);
  const TA *Bc = reinterpret_cast<const TA *>(a.cb_succ);
  const float *pj = a.proj + (long)i * r;
  const int npred = i == 0 ? (a.anchor < 0 ? 0 : 1) : K;
  for (int e = tid; e < K * r; e += 256) {
    const int b = e / r, rho = e - b * r;
    const int c = clamp_idx(a.idx[i * K + b], a.V);
    bp[b * rl + rho] = to_f32(Bc[(long)c * r + rho]);
    if (b < npred) {
      const int p = i == 0 ? a.anchor : clamp_idx(a.idx[(i - 1) * K + b], a.V);
      ap[b * rl + rho] = to_f32(A[(long)p * r + rho]) * pj[rho];
    }
  }
  __syncthreads();
  const float *un = a.unary + (long)i * K;
  float *eo = a.edges + (long)i * K * K;
  for (int e = tid; e < K * K; e += 256) {
    const int ai = e / K, bi = e - ai * K;
    float v;
    if (i == 0 && ai > 0) {
      v = -__builtin_inff();
    } else if (npred == 0) {
      v = un[bi];
    } else {
      const float *x = ap + ai * rl, *y = bp + bi * rl;
      float s = 0.f;
      for (int k = 0; k < r; ++k) s += x[k] * y[k];
      v = s + un[bi];
    }
    eo[e] = v;
  }
}

// s_0[b] = edge[0][0][b]; s_i[b] = max_a s_{i-1}[a] + edge[i][a][b] (first max wins)
__global__ __launch_bounds__(256) void selector_path_kernel(SelArgs a) {
  __shared__ float se[kSelMaxB * kSelMaxK * kSelMaxK];
  __shared__ int sidx[kSelMaxB * kSelMaxK];
  __shared__ float score[2][kSelMaxK];
  __shared__ int back[kSelMaxB * kSelMaxK];
  const int tid = threadIdx.x;
  const int B = a.B, K = a.K;
  for (int e = tid; e < B * K * K; e += 256) se[e] = a.edges[e];
  for (int e = tid; e < B * K; e += 256) sidx[e] = clamp_idx(a.idx[e], a.V);
  __syncthreads();
  if (tid < K) score[0][tid] = se[tid];
  __syncthreads();
  for (int i = 1; i < B; ++i) {
    const int cur = (i - 1) & 1;
    if (tid < K) {
      const float *ei = se + i * K * K;
      float best = score[cur][0] + ei[tid];
      int arg = 0;
      for (int ai = 1; ai < K; ++ai) {
        const float v = score[cur][ai] + ei[ai * K + tid];
        if (v > best) {
          best = v;
          arg = ai;
        }
      }
      score[cur ^ 1][tid] = best;
      back[i * K + tid] = arg;
    }
    __syncthreads();
  }
  if (tid == 0) {
    const int fin = (B - 1) & 1;
    int bsl = 0;
    float best = score[fin][0];
    for (int b = 1; b < K; ++b)
      if (score[fin][b] > best) {
        best = score[fin][b];
        bsl = b;
      }
    int acc = B;
    for (int i = B - 1; i >= 0; --i) {
      a.path[i] = sidx[i * K + bsl];
      if (a.target && a.path[i] != a.target[i]) acc = i;
      if (i > 0) bsl = back[i * K + bsl];
    }
    if (a.accept) a.accept[0] = acc;
  }
}

// The whole selector in one launch (used when the candidate rows fit in
// LDS).  Every workgroup forms a k-slice of proj = h . P^T: wave w streams
// 16 rows of P (tile w / Q) over piece range q = w % Q of the slice, the
// pieces of a tile are summed in LDS in order, and the slice is written as a
// partial.  Every workgroup also gathers each position's predecessor rows of
// A and candidate rows of B into LDS (16-byte loads issued together), so
// that the last workgroup to finish (completion counter) finds them there.
// It sums the slices in slice order (the projection never depends on
// arrival order), forms all B x K x K edges (two edges of one predecessor
// per thread, 16-element chunks of each dot product read from LDS at once,
// the same arithmetic as selector_edges_kernel), writes them, and runs the
// max-sum recursion in one wave: lane b holds state b and its back-pointers
// (8 bits per position).  In the top-K + selector kernel the last
// workgroup loads the slices together with the merged ids and gathers the
// candidate rows after them.
// The hand-over of the slices follows the skinny GEMMs' (agent-scope
// stores, release before the arrival, acquire by the last workgroup).
//
// The serial part runs once per launch, so its code is kept small (rolled
// loops over positions): straight-line code executed once waits on
// instruction fetch for every cache line.
constexpr int kSelWaves = 16;
constexpr int kSelThreads = kSelWaves * 64;

// the selector's LDS: tile sums, gathered rows, projection, edges, unaries, ids
template <typename TA>
struct SelLds {
  static constexpr int EPV = 16 / sizeof(TA);   // elements per 16-byte vector
  f32x4 *red;     // [16][64]
  TA *rows;       // [2][B*K][rs]
  float *pj;      // [B][r]
  float *se;      // [B][K][K]
  float *un;      // [B][K]
  int *sidx;      // [B][K]
  int rs;         // padded row stride (elements)
  __device__ SelLds(unsigned char *smem, const SelArgs &a) {
    const int BK = a.B * a.K;
    rs = a.r + EPV;
    red = reinterpret_cast<f32x4 *>(smem);
    rows = reinterpret_cast<TA *>(smem + kSelThreads * sizeof(f32x4));
    pj = reinterpret_cast<float *>(rows + 2 * BK * rs);
    se = pj + a.B * a.r;
    un = se + BK * a.K;
    sidx = reinterpret_cast<int *>(un + BK);
  }
};

// This wave's share of slice `slice` of the projection: tile t = wave / Q of
// P over piece range q = wave % Q (zero for waves past nt * Q).
template <typename TA>
__device__ __forceinline__ f32x4 sel_product(const SelArgs &a, int slice) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int B = a.B, d = a.d;
  const int nt = a.r >> 4, Q = kSelWaves / nt, span = a.pieces * 128;
  const int t = wave / Q, q = wave - t * Q;
  const int k_lo = min(d, (slice * Q + q) * span), k_hi = min(d, k_lo + span);
  f32x4 acc = zero4();
  if (wave < nt * Q && k_lo < k_hi) {
    // lane (g, r16): row 16 t + r16 of P and position min(r16, B - 1) of h
    // (columns r16 >= B of the product are never stored)
    const TA *wr = reinterpret_cast<const TA *>(a.pw) + (long)(t * 16 + r16) * d;
    const TA *xr = reinterpret_cast<const TA *>(a.h) + (long)min(r16, B - 1) * d;
    for (int k = k_lo; k < k_hi; k += 128) {
      // a piece's four 32-wide steps loaded together; steps past the range
      // (a 64-wide last piece) reload the range's last step and are not used
      Frag<TA> wf[4], xf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kc = min(k + 32 * j, k_hi - 32) + 8 * g;
        wf[j] = load_frag(wr + kc);
        xf[j] = load_frag(xr + kc);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (k + 32 * j < k_hi) mma(acc, wf[j], xf[j]);
    }
  }
  return acc;
}

// The slice's tile sums (pieces added in order): thread (wave < nt, lane)
// holds tile `wave`, lane (g, r16).  Ends with the workgroup barrier that
// publishes what was written to LDS before it.
__device__ __forceinline__ f32x4 sel_tile_sum(f32x4 *red, f32x4 acc, int r) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nt = r >> 4, Q = kSelWaves / nt;
  red[wave * 64 + lane] = acc;
  __syncthreads();
  f32x4 v = zero4();
  if (wave < nt) {
#pragma unroll 1
    for (int j = 0; j < Q; ++j) {
      const f32x4 x = red[(wave * Q + j) * 64 + lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] += x[i];
    }
  }
  return v;
}

// slice `slice` of the projection into the partials (waves < nt), agent scope
__device__ __forceinline__ void sel_store_slice(const SelArgs &a, int slice, f32x4 v) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nt = a.r >> 4;
  if (wave < nt) {
    float *pp = a.part + (((long)slice * nt + wave) * 64 + lane) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) __hip_atomic_store(pp + i, v[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The arrival of a workgroup (its stores completed first); true in the last
// of `n` to arrive, which has acquired every earlier release
__device__ __forceinline__ bool sel_arrive(unsigned long long *cnt, unsigned long long stamp, int n) {
  __shared__ unsigned last;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const bool l = arrive_last(cnt, stamp, n);
    if (l) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    last = l;
  }
  __syncthreads();
  return last;
}

// the S slices summed in slice order (waves < nt); the slices happen-before
// these loads (release by every arrival, acquire by this workgroup), so
// ordinary 16-byte loads see them, sixteen in flight
__device__ __forceinline__ f32x4 sel_sum_slices(const SelArgs &a, int S) {
  constexpr int NF = 16;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nt = a.r >> 4;
  const long sstride = (long)nt * 64;   // float4 per slice
  f32x4 v = zero4();
  if (wave < nt) {
    const f32x4 *src = reinterpret_cast<const f32x4 *>(a.part) + wave * 64 + lane;
    for (int s0 = 0; s0 < S; s0 += NF) {
      f32x4 x[NF];
#pragma unroll
      for (int j = 0; j < NF; ++j) x[j] = src[(long)min(s0 + j, S - 1) * sstride];
#pragma unroll
      for (int j = 0; j < NF; ++j)
        if (s0 + j < S) {
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] += x[j][i];
        }
    }
  }
  return v;
}

// Gathers: rows [0, BK) are predecessor a of position i, A[idx[i-1][a]]
// (A[anchor] at i = 0); rows [BK, 2 BK) candidate b of position i,
// B[idx[i][b]] (L.sidx must be visible).  A thread's loads are issued back to
// back (no branch around them or their addresses); vectors past the end
// reload the last one and store it again (the same bytes to the same place).
template <typename TA>
__device__ __forceinline__ void sel_gather(const SelArgs &a, const SelLds<TA> &L) {
  constexpr int EPV = SelLds<TA>::EPV;
  constexpr int NT = kSelThreads;
  const int tid = threadIdx.x;
  const int K = a.K, r = a.r, BK = a.B * a.K, rs = L.rs;
  TA *rows = L.rows;
  const int *sidx = L.sidx;
  const TA *A = reinterpret_cast<const TA *>(a.cb_pred);
  const TA *Bc = reinterpret_cast<const TA *>(a.cb_succ);
  const int anchor = a.anchor < 0 ? 0 : a.anchor;   // row unused without an anchor
  const int vpr = r / EPV, nvec = 2 * BK * vpr;
  constexpr int UNR = 4;
  for (int v0 = tid; v0 < nvec; v0 += NT * UNR) {
    u32x4 buf[UNR];
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
      const int vv = min(v0 + NT * j, nvec - 1);
      const int row = vv / vpr, part = vv - row * vpr;
      const bool pred = row < BK;
      const int rr = pred ? row : row - BK;
      const int i = rr / K, ai = rr - i * K;
      const int pid = i == 0 ? anchor : sidx[max((i - 1) * K + ai, 0)];
      const TA *src = pred ? A + (long)pid * r : Bc + (long)sidx[rr] * r;
      buf[j] = *reinterpret_cast<const u32x4 *>(src + part * EPV);
    }
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
      const int vv = min(v0 + NT * j, nvec - 1);
      const int row = vv / vpr, part = vv - row * vpr;
      *reinterpret_cast<u32x4 *>(rows + row * rs + part * EPV) = buf[j];
    }
  }
}

// The projection v (waves < nt) into LDS, then the edges, the max-sum path
// and the accept length (the gathered rows, ids and unaries are in LDS).
template <typename TA, int KM, bool EXACT>
__device__ __forceinline__ void sel_finish(const SelArgs &a, const SelLds<TA> &L, f32x4 v, int tg) {
  constexpr int NT = kSelThreads;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int B = a.B, K = a.K, r = a.r, BK = a.B * a.K, rs = L.rs, nt = r >> 4;
  const TA *rows = L.rows;
  float *pj = L.pj, *se = L.se;
  const float *un = L.un;
  const int *sidx = L.sidx;
  // the projection of position r16, features 16 t + 4 g + i
  if (wave < nt && r16 < B) {
#pragma unroll
    for (int i = 0; i < 4; ++i) pj[r16 * r + wave * 16 + 4 * g + i] = v[i];
  }
  __syncthreads();

  // thread: predecessor ai of position i and EB successors b0 + j, so that
  // each product x[k] p[k] is formed once for both; every edge is still one
  // running sum over k of (x[k] p[k]) y[k], the arithmetic of
  // selector_edges_kernel.  (Two successors per thread keep eight waves
  // busy: four per thread left one wave per SIMD waiting on its own
  // dependent adds.)
  constexpr int EB = 2, EK = 16;
  const int nbg = (K + EB - 1) / EB;
  for (int t = tid; t < BK * nbg; t += NT) {
    const int pr = t / nbg, b0 = (t - pr * nbg) * EB;
    const int i = pr / K, ai = pr - i * K;
    const bool dead = i == 0 && ai > 0;                // no such predecessor
    const bool lone = i == 0 && a.anchor < 0;          // no predecessor at all
    float s[EB];
#pragma unroll
    for (int j = 0; j < EB; ++j) s[j] = 0.f;
    if (!dead && !lone) {
      const TA *x = rows + (i * K + ai) * rs;
      const TA *y[EB];
#pragma unroll
      for (int j = 0; j < EB; ++j) y[j] = rows + (BK + i * K + min(b0 + j, K - 1)) * rs;
      const float *p = pj + i * r;
      for (int k0 = 0; k0 < r; k0 += EK) {   // r is a multiple of EK
        float ap[EK];
#pragma unroll
        for (int k = 0; k < EK; ++k) ap[k] = to_f32(x[k0 + k]) * p[k0 + k];
#pragma unroll
        for (int j = 0; j < EB; ++j) {
          float yv[EK];
#pragma unroll
          for (int k = 0; k < EK; ++k) yv[k] = to_f32(y[j][k0 + k]);
#pragma unroll
          for (int k = 0; k < EK; ++k) s[j] += ap[k] * yv[k];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < EB; ++j) {
      const int bi = b0 + j;
      if (bi < K) {
        const float ev = dead ? -__builtin_inff() : lone ? un[i * K + bi] : s[j] + un[i * K + bi];
        const int e = pr * K + bi;
        se[e] = ev;
        a.edges[e] = ev;
      }
    }
  }
  __syncthreads();
  if (wave != 0) return;

  // s_0[b] = edge[0][0][b]; s_i[b] = max_a s_{i-1}[a] + edge[i][a][b], the
  // first (lowest a) maximum wins.  Lanes >= K shadow state K-1 (never
  // chosen).  EXACT (K == KM): no per-candidate bound checks in the loop.
  const int bl = min(lane, K - 1);
  float sc = se[bl];
  unsigned long long bp0 = 0, bp1 = 0;   // back-pointers, 8 bits per position (0-7, 8-15)
#pragma unroll 1
  for (int i = 1; i < B; ++i) {
    const float *ei = se + i * K * K;
    float ecol[KM];
#pragma unroll
    for (int qq = 0; qq < KM; ++qq) ecol[qq] = ei[(EXACT ? qq : min(qq, K - 1)) * K + bl];
    float best = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc), 0)) + ecol[0];
    int arg = 0;
#pragma unroll
    for (int qq = 1; qq < KM; ++qq) {
      const float ev = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc), qq)) + ecol[qq];
      if ((EXACT || qq < K) && ev > best) {
        best = ev;
        arg = qq;
      }
    }
    sc = best;
    const unsigned long long bits = (unsigned long long)arg << (8 * (i & 7));
    if (i < 8) bp0 |= bits;
    else bp1 |= bits;
  }
  // best final state, the lowest b on ties
  int b = 0;
  float bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc), 0));
#pragma unroll 1
  for (int qq = 1; qq < K; ++qq) {
    const float ev = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc), qq));
    if (ev > bv) {
      bv = ev;
      b = qq;
    }
  }
  // backtrack: lane i receives the path's state at position i
  int ps = 0;
#pragma unroll 1
  for (int i = B - 1; i >= 0; --i) {
    ps = lane == i ? b : ps;
    if (i > 0) {
      const unsigned long long w = i < 8 ? bp0 : bp1;
      const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)w, b);
      const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(w >> 32), b);
      b = (int)(((((unsigned long long)hi << 32) | lo) >> (8 * (i & 7))) & 0xffu);
    }
  }
  // lanes < B: the candidate id on the path and the accept length (the
  // first position where the path leaves the target)
  const int id = lane < B ? sidx[lane * K + ps] : 0;
  if (lane < B) a.path[lane] = id;
  const unsigned long long miss = __ballot(lane < B && id != tg);
  if (a.accept && lane == 0) a.accept[0] = miss ? (int)__builtin_ctzll(miss) : B;
}

template <typename TA, int KM, bool EXACT>
__global__ __launch_bounds__(kSelThreads) void selector_fused_kernel(SelArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const SelLds<TA> L(smem, a);
  const int tid = threadIdx.x, B = a.B, BK = a.B * a.K;
  // candidate ids, unaries and the target (first: the gathers wait on them)
  int ix = 0;
  float uv = 0.f;
  if (tid < BK) {
    ix = a.idx[tid];
    uv = a.unary[tid];
  }
  const int tg = a.target && tid < B ? a.target[tid] : 0;   // wave 0: position `lane`
  const f32x4 acc = sel_product<TA>(a, blockIdx.x);
  if (tid < BK) {
    L.sidx[tid] = clamp_idx(ix, a.V);
    L.un[tid] = uv;
  }
  f32x4 v = sel_tile_sum(L.red, acc, a.r);   // its barrier publishes the ids too
  sel_gather<TA>(a, L);
  const int S = gridDim.x;
  if (S > 1) {
    sel_store_slice(a, blockIdx.x, v);
    if (!sel_arrive(a.cnt, a.stamp, S)) return;
    v = sel_sum_slices(a, S);
  }
  sel_finish<TA, KM, EXACT>(a, L, v, tg);
}

// The LM head's final merge and the whole selector in one launch (the
// top-K + selector call): workgroups [0, S) form the projection's slices,
// workgroups S + t merge token t's top-K lists and write its ids and unary
// scores (merge_token, the same results as topk_merge_kernel).  The last of
// all S + B workgroups to finish reads the ids, gathers the candidate rows,
// sums the slices and finishes as selector_fused_kernel does.
template <typename TA, int KM, bool EXACT>
__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(TopkArgs ta, SelArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const SelLds<TA> L(smem, a);
  const int tid = threadIdx.x, B = a.B, BK = a.B * a.K;
  const int S = a.n_wg;
  if ((int)blockIdx.x < S) {
    const f32x4 acc = sel_product<TA>(a, blockIdx.x);
    sel_store_slice(a, blockIdx.x, sel_tile_sum(L.red, acc, a.r));
  } else {
    merge_token<KM, kSelThreads>(ta, (int)blockIdx.x - S);
  }
  if (!sel_arrive(a.cnt, a.stamp, S + B)) return;
  // every token's ids and unaries were written before its arrival; their
  // loads and the slices' are in flight together, the gather follows
  int ix = 0;
  float uv = 0.f;
  if (tid < BK) {
    ix = a.idx[tid];
    uv = a.unary[tid];
  }
  const int tg = a.target && tid < B ? a.target[tid] : 0;
  const f32x4 v = sel_sum_slices(a, S);
  if (tid < BK) {
    L.sidx[tid] = clamp_idx(ix, a.V);
    L.un[tid] = uv;
  }
  __syncthreads();
  sel_gather<TA>(a, L);
  sel_finish<TA, KM, EXACT>(a, L, v, tg);
}

static size_t selector_fused_lds(int act, const SelArgs &a) {
  const size_t es = act == ACT_F32 ? 4 : 2;
  const size_t bk = (size_t)a.B * a.K;
  return kSelWaves * 64 * 16 + 2 * bk * (a.r + 16 / es) * es + ((size_t)a.B * a.r + bk * a.K + bk) * 4 +
         bk * 4;
}

#ifndef DFL_SEL_FUSED
#define DFL_SEL_FUSED 1
#endif

bool selector_fused_fits(int act, const SelArgs &a) {
  return DFL_SEL_FUSED && a.r % 16 == 0 && a.r / 16 <= kSelWaves && a.d % 64 == 0 &&
         selector_fused_lds(act, a) + sizeof(unsigned) <= kMaxLdsBytes;
}

// Q waves per 16-row tile of P, each over `pieces` 128-wide k-pieces; at most
// 64 workgroups (k-slices)
void selector_fused_plan(SelArgs &a) {
  const int nt = a.r / 16, Q = kSelWaves / nt;
  const int nchunk = (a.d + 127) / 128;
  a.pieces = std::max(1, (nchunk + Q * 64 - 1) / (Q * 64));
  a.n_wg = (nchunk + Q * a.pieces - 1) / (Q * a.pieces);
}

size_t selector_part_bytes(int r, int d) {
  SelArgs a;
  a.r = r;
  a.d = d;
  selector_fused_plan(a);
  return (size_t)a.n_wg * (r / 16) * 64 * 16;
}

template <typename TA, int KM, bool EXACT>
static hipError_t selector_fused_go(const SelArgs &a, size_t lds, hipStream_t st) {
  auto *k = &selector_fused_kernel<TA, KM, EXACT>;
  const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void *>(k), lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3(a.n_wg), dim3(kSelWaves * 64), lds, st, a);
  return hipSuccess;
}

hipError_t launch_selector(int act, const SelArgs &a, hipStream_t st) {
  if (a.fused) {
    if (!selector_fused_fits(act, a) || a.n_wg < 1 || a.n_wg > 64 || (a.n_wg > 1 && (!a.part || !a.cnt)))
      return hipErrorInvalidValue;
    const size_t flds = selector_fused_lds(act, a);
    hipError_t e;
    if (act == ACT_F32)
      e = a.K == 8  ? selector_fused_go<float, 8, true>(a, flds, st)
          : a.K < 8 ? selector_fused_go<float, 8, false>(a, flds, st)
                    : selector_fused_go<float, 32, false>(a, flds, st);
    else
      e = a.K == 8  ? selector_fused_go<bf16, 8, true>(a, flds, st)
          : a.K < 8 ? selector_fused_go<bf16, 8, false>(a, flds, st)
                    : selector_fused_go<bf16, 32, false>(a, flds, st);
    return e != hipSuccess ? e : hipGetLastError();
  }
  const size_t lds = (size_t)2 * a.K * (a.r + 1) * sizeof(float);
  if (act == ACT_F32)
    hipLaunchKernelGGL((selector_edges_kernel<float>), dim3(a.B), dim3(256), lds, st, a);
  else
    hipLaunchKernelGGL((selector_edges_kernel<bf16>), dim3(a.B), dim3(256), lds, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(selector_path_kernel, dim3(1), dim3(256), 0, st, a);
  return hipGetLastError();
}

bool topk_select_ok(int act, const TopkArgs &ta, const SelArgs &a) {
  // the merge's own LDS (a few hundred bytes) beside the selector's
  return ta.lds_path && ta.K <= 8 && ta.B == a.B && ta.n_wg >= 1 && selector_fused_fits(act, a) &&
         selector_fused_lds(act, a) + 1024 <= kMaxLdsBytes;
}

template <typename TA, bool EXACT>
static hipError_t topk_select_go(const TopkArgs &ta, const SelArgs &a, size_t lds, hipStream_t st) {
  auto *k = &topk_select_kernel<TA, 8, EXACT>;
  const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void *>(k), lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3(a.n_wg + a.B), dim3(kSelThreads), lds, st, ta, a);
  return hipGetLastError();
}

hipError_t launch_topk_select(int act, const TopkArgs &ta, const SelArgs &a, hipStream_t st) {
  if (!topk_select_ok(act, ta, a) || !a.fused || a.n_wg < 1 || a.n_wg > 64 || !a.part || !a.cnt)
    return hipErrorInvalidValue;
  const size_t lds = selector_fused_lds(act, a);
  if (act == ACT_F32)
    return a.K == 8 ? topk_select_go<float, true>(ta, a, lds, st) : topk_select_go<float, false>(ta, a, lds, st);
  return a.K == 8 ? topk_select_go<bf16, true>(ta, a, lds, st) : topk_select_go<bf16, false>(ta, a, lds, st);
}

// ---------------------------------------------------------------------------
// Greedy accept length: the longest prefix where draft and target agree.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void accept_kernel(const int *__restrict__ draft,
                                                     const int *__restrict__ target, int n_seq,
                                                     int B, int *__restrict__ accept) {
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s >= n_seq) return;
  const int *d = draft + (long)s * B;
  const int *t = target + (long)s * B;
  int m = 0;
  while (m < B && d[m] == t[m]) ++m;
  accept[s] = m;
}

hipError_t launch_accept(const int *draft, const int *target, int n_seq, int B, int *accept,
                         hipStream_t st) {
  hipLaunchKernelGGL(accept_kernel, dim3((n_seq + 255) / 256), dim3(256), 0, st, draft, target,
                     n_seq, B, accept);
  return hipGetLastError();
}

}  // namespace dfl
