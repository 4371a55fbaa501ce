// The final merge of the LM head's top-K partial lists (device code shared
// by the merge kernel and the one-launch top-K + selector kernel; see
// topk.hip for the lists' construction).
#pragma once

#include "common.h"
#include "kernels.h"

namespace dfl {

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kL2e = 1.4426950408889634f;

// Partial lists of the workgroups, [token (16)][entry][workgroup]: values and
// indices have K entries per token, the (max, sum) pairs 2.  Lanes of the
// merges take consecutive workgroups, so their loads are coalesced.
__device__ __forceinline__ long part_at(const TopkArgs &a, int tok, int entry, int per_tok, int wg) {
  return ((long)tok * per_tok + entry) * a.n_wg + wg;
}

// pairwise sum of N values in a fixed order: ((x0 + x1) + (x2 + x3)) + ...
template <int N>
__device__ __forceinline__ float tree_sum(const float *x) {
  if constexpr (N == 1) return x[0];
  else return tree_sum<N / 2>(x) + tree_sum<N / 2>(x + N / 2);
}

// one workgroup per token: merge n_wg partial lists and (max, sum) pairs
// (value, index) as one 64-bit key whose unsigned order is the candidate
// order: value descending, then index ascending.  High word: the float's bits
// made monotonic; low word: the complemented index.  0 = no candidate.
__device__ __forceinline__ unsigned long long cand_key(float v, int i) {
  const unsigned u = __float_as_uint(v);
  const unsigned o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)o << 32) | (unsigned)(~(unsigned)i);
}
__device__ __forceinline__ float key_value(unsigned long long k) {
  const unsigned o = (unsigned)(k >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
__device__ __forceinline__ int key_index(unsigned long long k) { return (int)~(unsigned)k; }
__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long x, int o) {
  const int lo = __shfl_xor((int)(unsigned)x, o, kWave);
  const int hi = __shfl_xor((int)(unsigned)(x >> 32), o, kWave);
  return ((unsigned long long)(unsigned)hi << 32) | (unsigned)lo;
}
// a 64-bit value moved between the lanes of each 16-lane row by DPP control CTRL
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long x) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(unsigned)x, CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(unsigned)(x >> 32), CTRL, 0xf, 0xf, false);
  return ((unsigned long long)(unsigned)hi << 32) | (unsigned)lo;
}
__device__ __forceinline__ unsigned long long umax_u64(unsigned long long x, unsigned long long y) {
  return x > y ? x : y;
}
// the largest key of the wave, in every lane (all 64 lanes active): within
// each row of 16, DPP swaps lanes j ^ 1 and j ^ 2, then mirrors the quads
// of each half-row and the halves of the row (each step pairs two groups
// that already agree); across the rows, two lane permutes (j ^ 16, j ^ 32)
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long b) {
  b = umax_u64(b, dpp_u64<0xB1>(b));    // quad_perm 1,0,3,2
  b = umax_u64(b, dpp_u64<0x4E>(b));    // quad_perm 2,3,0,1
  b = umax_u64(b, dpp_u64<0x141>(b));   // row_half_mirror
  b = umax_u64(b, dpp_u64<0x140>(b));   // row_mirror
  b = umax_u64(b, shfl_xor_u64(b, 16));
  return umax_u64(b, shfl_xor_u64(b, 32));
}

// Final merge of token `tok` by one workgroup of NT threads (all of them call
// it): thread t holds partial list t (and, with more than NT workgroup
// partials, merges lists t + NT j into it), the log-sum-exp is a fixed-order
// tree over the threads, and the K winners are picked one at a time by a
// block-wide max over the list heads.  Every vocabulary row sits in exactly
// one partial, so the winning key names the one list whose head advances.
// Threads without a list hold nothing, so 256 or 1024 threads give the same
// results bit for bit; the cross-wave steps read only the `nact` waves that
// hold lists (the others contribute -inf maxima and empty keys).
template <int KM, int NT>
__device__ __forceinline__ void merge_token(const TopkArgs &a, int tok) {
  constexpr int NWV = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K;
  const int nact = min(NWV, (a.n_wg + 63) / 64);
  unsigned long long key[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) key[j] = 0;
  float m = -__builtin_inff(), s = 0.f;
  if (tid < a.n_wg) {
    // entries j >= K re-read entry K-1 (in bounds) and are dropped
    float pv[KM];
    int pi[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      const long e = part_at(a, tok, min(j, K - 1), K, tid);
      pv[j] = a.part_val[e];
      pi[j] = a.part_idx[e];
    }
    m = a.part_ms[part_at(a, tok, 0, 2, tid)];
    s = a.part_ms[part_at(a, tok, 1, 2, tid)];
#pragma unroll
    for (int j = 0; j < KM; ++j) key[j] = j < K ? cand_key(pv[j], pi[j]) : 0ull;
  }
  for (int w = tid + NT; w < a.n_wg; w += NT) {
    const float pm = a.part_ms[part_at(a, tok, 0, 2, w)], ps = a.part_ms[part_at(a, tok, 1, 2, w)];
    if (ps > 0.f) {
      if (pm > m) {
        s = s * exp2f((m - pm) * kL2e);
        m = pm;
      }
      s += ps * exp2f((pm - m) * kL2e);
    }
    for (int j = 0; j < K; ++j) {
      const long e = part_at(a, tok, j, K, w);
      unsigned long long x = cand_key(a.part_val[e], a.part_idx[e]);
      if (x <= key[KM - 1]) break;   // the partial list is sorted: no later entry fits
#pragma unroll
      for (int q = 0; q < KM; ++q) {   // insert, keeping key[] descending
        const unsigned long long hi = key[q] > x ? key[q] : x;
        x = key[q] > x ? x : key[q];
        key[q] = hi;
      }
    }
  }
  __shared__ float wm[NWV], wsum[NWV];
  __shared__ unsigned long long wbest[2][NWV];
  // log-sum-exp: fixed-order tree over the NT threads
  float M = m;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) M = fmaxf(M, shfl_xor(M, o));
  if (lane == 0) wm[wave] = M;
  __syncthreads();
  M = wm[0];
  for (int q = 1; q < nact; ++q) M = fmaxf(M, wm[q]);
  float S = s > 0.f ? s * exp2f((m - M) * kL2e) : 0.f;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) S += shfl_xor(S, o);
  if (lane == 0) wsum[wave] = S;
  __syncthreads();
  S = tree_sum<NWV>(wsum);
  const float lse = M + log2f(S) * kLn2;
  for (int k = 0; k < K; ++k) {
    // two slots: a wave that runs ahead writes the other one
    if (wave < nact) {
      const unsigned long long b = wave_max_u64(key[0]);
      if (lane == 0) wbest[k & 1][wave] = b;
    }
    __syncthreads();
    unsigned long long w = wbest[k & 1][0];
    for (int q = 1; q < nact; ++q) w = umax_u64(w, wbest[k & 1][q]);
    if (key[0] == w) {
#pragma unroll
      for (int j = 0; j < KM - 1; ++j) key[j] = key[j + 1];
      key[KM - 1] = 0;
    }
    if (tid == 0) {
      a.idx[(long)tok * K + k] = key_index(w);
      a.unary[(long)tok * K + k] = key_value(w) - lse;
    }
  }
}


}  // namespace dfl
