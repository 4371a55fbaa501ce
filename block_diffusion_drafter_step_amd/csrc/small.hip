// The small kernels of the draft block step: the injection RMSNorm, the
// DFlash2 grouped dynamic depthwise convolution, the candidate-selector
// edges with their best-path readout, and the greedy accept length.
#include "common.h"
#include "kernels.h"

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
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float *__restrict__ y, int d,
                                                      const TA *__restrict__ gamma, float eps,
                                                      TA *__restrict__ z) {
  const long row = blockIdx.x;
  const float *yr = y + row * d;
  float ss = 0.f;
  for (int c = threadIdx.x * 4; c < d; c += 1024) {
    const float4 v = *reinterpret_cast<const float4 *>(yr + c);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  __shared__ float red[4];
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float inv = 1.0f / sqrtf(tot / (float)d + eps);
  TA *zr = z + row * d;
  for (int c = threadIdx.x * 4; c < d; c += 1024) {
    const float4 v = *reinterpret_cast<const float4 *>(yr + c);
    float o[4] = {v.x * inv, v.y * inv, v.z * inv, v.w * inv};
    if (gamma) {
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] *= to_f32(gamma[c + j]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) zr[c + j] = from_f32<TA>(o[j]);
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
// Grouped dynamic depthwise conv ("spec : add DFlash2 support", Overview):
// out[i,c] = sum_t (base[t,c] + delta[i, t*G + g(c)]) * x[i-t, c], x[<0] = 0.
// One thread per (block, position, 4 adjacent channels): its T input rows,
// T delta values per channel and T base values are independent loads issued
// together, so a single block costs one memory round trip, and a batch of
// blocks is a pure stream (x read T times from cache, out written once).
// ---------------------------------------------------------------------------
template <typename TA, int TM>
__global__ __launch_bounds__(256) void conv_kernel(const TA *__restrict__ x, int n_blocks, int B,
                                                   int C, int G, int T,
                                                   const TA *__restrict__ base,
                                                   const float *__restrict__ delta,
                                                   TA *__restrict__ out) {
  const long id = (long)blockIdx.x * 256 + threadIdx.x;
  const int c4 = C >> 2;
  const long row = id / c4;           // block * B + position
  if (row >= (long)n_blocks * B) return;
  const int c = (int)(id - row * c4) * 4;
  const int i = (int)(row % B);
  const int cpg = C / G;
  const int TG = T * G;
  const float *dl = delta + row * (long)TG;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float xv[TM][4], bv[TM][4], dv[TM][4];
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    const bool ok = t < T && i - t >= 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xv[t][j] = ok ? to_f32(x[(row - t) * C + c + j]) : 0.f;
      bv[t][j] = t < T ? to_f32(base[(long)t * C + c + j]) : 0.f;
      dv[t][j] = t < T ? dl[t * G + (c + j) / cpg] : 0.f;
    }
  }
#pragma unroll
  for (int t = 0; t < TM; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] += (bv[t][j] + dv[t][j]) * xv[t][j];
#pragma unroll
  for (int j = 0; j < 4; ++j) out[row * C + c + j] = from_f32<TA>(acc[j]);
}

template <typename TA>
static void conv_launch_t(const void *x, int n_blocks, int B, int C, int G, int T, const void *base,
                          const float *delta, void *out, hipStream_t st) {
  const long threads = (long)n_blocks * B * (C / 4);
  const dim3 grid((unsigned)((threads + 255) / 256));
  const TA *xp = reinterpret_cast<const TA *>(x);
  const TA *bp = reinterpret_cast<const TA *>(base);
  TA *op = reinterpret_cast<TA *>(out);
  if (T <= 4)
    hipLaunchKernelGGL((conv_kernel<TA, 4>), grid, dim3(256), 0, st, xp, n_blocks, B, C, G, T, bp,
                       delta, op);
  else if (T <= 8)
    hipLaunchKernelGGL((conv_kernel<TA, 8>), grid, dim3(256), 0, st, xp, n_blocks, B, C, G, T, bp,
                       delta, op);
  else
    hipLaunchKernelGGL((conv_kernel<TA, 16>), grid, dim3(256), 0, st, xp, n_blocks, B, C, G, T, bp,
                       delta, op);
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
// the K-state max-sum recursion over the positions and the backtrack.
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
    for (int i = B - 1; i >= 0; --i) {
      a.path[i] = sidx[i * K + bsl];
      if (i > 0) bsl = back[i * K + bsl];
    }
  }
}

hipError_t launch_selector(int act, const SelArgs &a, hipStream_t st) {
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
