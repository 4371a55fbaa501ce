// Weight-streaming core shared by the skinny GEMMs and the LM head.
//
// A wave owns `cnt` (<= TPW) consecutive 16-row tiles of a weight and a
// k-range of it.  It walks the k-range in chunks of 128 (plus one 64 tail):
// per chunk it loads the activation fragments once, then the weight
// fragments of every tile it owns, then issues the MFMAs, so activation loads
// are amortised over TPW tiles and every weight byte is loaded exactly once.
// Each weight load instruction reads 16 rows x 64 contiguous bytes straight
// into registers; measured on MI355X this pattern streams at ~6 TB/s.
//
// Loads are guarded (issued only for tiles the wave owns and chunks that
// exist); measured on MI355X this beat an unguarded form that clamps rows and
// discards the extra results (injection fc 65 vs 80 us, streaming LM head 308
// vs 388 us): the extra bytes cost more than the waits.
//
// k-slot layouts (any assignment is valid if A and B fragments agree):
//   bf16 / fp32 weights: MFMA j of a chunk takes k = 32 j + 8 g .. + 8 from
//                        lane group g.
//   Q8_0 weights:        a lane loads 16 codes at k = 64 m + 16 g; MFMA 2m+e
//                        takes codes/activations k = 64 m + 16 g + 8 e .. + 8.
#pragma once

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dfl {

// Q8_0 weights whose k-ranges all start on 128-element boundaries: the four
// block scales of a 128-wide chunk come from one 8-byte load (2-byte loads
// measured slow on this path).  Internal to the streaming kernels.
constexpr int W_Q8_0_S4 = 2;
constexpr bool is_q8(int wk) { return wk == W_Q8_0 || wk == W_Q8_0_S4; }

// Q8_0 dequantisation of 8 codes held in two dwords: value = bf16(fp32(s) * q).
// (q + 128) comes from v_cvt_f32_ubyte on the sign-flipped byte, and
// fma(q + 128, s, -128 s) = q s exactly (q s needs at most 19 significant bits),
// so the single rounding is the bf16 one, two values per v_cvt_pk_bf16_f32.
typedef float dq_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 dq_bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t dq_pair(uint32_t x, int sh, float s, float c) {
  const dq_f32x2 v = {fmaf((float)((x >> sh) & 0xffu), s, c),
                      fmaf((float)((x >> (sh + 8)) & 0xffu), s, c)};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, dq_bf16x2));
}

__device__ __forceinline__ Frag<bf16> dq8(uint32_t lo, uint32_t hi, float s) {
  const uint32_t a = lo ^ 0x80808080u, b = hi ^ 0x80808080u;
  const float c = -128.0f * s;
  u32x4 r;
  r[0] = dq_pair(a, 0, s, c);
  r[1] = dq_pair(a, 16, s, c);
  r[2] = dq_pair(b, 0, s, c);
  r[3] = dq_pair(b, 16, s, c);
  Frag<bf16> f;
  f.v = __builtin_bit_cast(bf16x8, r);
  return f;
}

// Scales of a lane's code vectors k + 64 m + 16 g .. + 16 (block k/32 + 2 m
// + g/2).  W_Q8_0_S4 with a whole 128-wide chunk: k % 128 == 0 and the row's
// scales start 8-byte aligned, so the chunk's four scales are one 8-byte load.
template <int WK, int NJ>
__device__ __forceinline__ void q8_chunk_scales(const uint16_t *s, int k, int g, float (&sc)[NJ / 2]) {
  if constexpr (WK == W_Q8_0_S4 && NJ == 4) {
    const uint2 q = *reinterpret_cast<const uint2 *>(s + (k >> 5));
    sc[0] = half_bits_to_f32((uint16_t)(g < 2 ? q.x : q.x >> 16));
    sc[1] = half_bits_to_f32((uint16_t)(g < 2 ? q.y : q.y >> 16));
  } else {
#pragma unroll
    for (int m = 0; m < NJ / 2; ++m) sc[m] = half_bits_to_f32(s[(k + 64 * m + 16 * g) >> 5]);
  }
}

// One weight row as seen by a lane.
template <typename TA, int WK>
struct SRow {
  const void *p;        // row start (values or int8 codes)
  const uint16_t *s;    // Q8_0: row's fp16 scales
};

template <typename TA, int WK>
__device__ __forceinline__ SRow<TA, WK> srow(const void *base, const void *scales, long row, int K) {
  SRow<TA, WK> r;
  if constexpr (is_q8(WK)) {
    r.p = reinterpret_cast<const int8_t *>(base) + row * K;
    r.s = reinterpret_cast<const uint16_t *>(scales) + row * (K >> 5);
  } else {
    r.p = reinterpret_cast<const TA *>(base) + row * K;
    r.s = nullptr;
  }
  return r;
}

// Weight loads are ordinary loads (non-temporal ones measured slower on
// MI355X: LM head 384 vs 302 us).
__device__ __forceinline__ uint4 wload16(const void *p) {
  const u32x4 v = *reinterpret_cast<const u32x4 *>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <typename T>
__device__ __forceinline__ Frag<T> wfrag(const T *p);
template <>
__device__ __forceinline__ Frag<bf16> wfrag(const bf16 *p) {
  Frag<bf16> f;
  f.v = __builtin_bit_cast(bf16x8, wload16(p));
  return f;
}
template <>
__device__ __forceinline__ Frag<float> wfrag(const float *p) {
  const uint4 a = wload16(p), b = wload16(p + 4);
  Frag<float> f;
  f.v[0] = __builtin_bit_cast(float, a.x); f.v[1] = __builtin_bit_cast(float, a.y);
  f.v[2] = __builtin_bit_cast(float, a.z); f.v[3] = __builtin_bit_cast(float, a.w);
  f.v[4] = __builtin_bit_cast(float, b.x); f.v[5] = __builtin_bit_cast(float, b.y);
  f.v[6] = __builtin_bit_cast(float, b.z); f.v[7] = __builtin_bit_cast(float, b.w);
  return f;
}

// One chunk's fragments: NJ activation fragments and the weight fragments of
// TPW tiles (Q8_0: 16-byte code vectors plus one scale per vector).
template <typename TA, int WK, int TPW, int NJ>
struct Chunk {
  using FB = typename std::conditional<is_q8(WK), Frag<bf16>, Frag<TA>>::type;
  FB b[NJ];
  Frag<TA> a[is_q8(WK) ? 1 : TPW][is_q8(WK) ? 1 : NJ];
  uint4 c[is_q8(WK) ? TPW : 1][is_q8(WK) ? NJ / 2 : 1];
  float sc[is_q8(WK) ? TPW : 1][is_q8(WK) ? NJ / 2 : 1];
};

// ---- chunk loads (under `u < cnt` and the prefetch conditions) and products ----
template <typename TA, int WK, int TPW, int NJ>
__device__ __forceinline__ void chunk_load_g(Chunk<TA, WK, TPW, NJ> &ch, const TA *xr,
                                           const SRow<TA, WK> (&rows)[TPW], int cnt, int k, int g,
                                           bool tok_ok) {
  if constexpr (is_q8(WK)) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int off = k + 64 * (j >> 1) + 16 * g + 8 * (j & 1);
      ch.b[j] = tok_ok ? load_frag(reinterpret_cast<const bf16 *>(xr) + off) : frag_zero<bf16>();
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      if (u < cnt) {
#pragma unroll
        for (int m = 0; m < NJ / 2; ++m) {
          const int off = k + 64 * m + 16 * g;
          ch.c[u][m] = wload16(reinterpret_cast<const int8_t *>(rows[u].p) + off);
        }
        q8_chunk_scales<WK, NJ>(rows[u].s, k, g, ch.sc[u]);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      ch.b[j] = tok_ok ? load_frag(xr + k + 32 * j + 8 * g) : frag_zero<TA>();
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      if (u < cnt) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          ch.a[u][j] = wfrag(reinterpret_cast<const TA *>(rows[u].p) + k + 32 * j + 8 * g);
      }
    }
  }
}

template <typename TA, int WK, int TPW, int NJ>
__device__ __forceinline__ void chunk_mma_g(const Chunk<TA, WK, TPW, NJ> &ch, int cnt,
                                          f32x4 (&acc)[TPW]) {
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    if (u < cnt) {
      if constexpr (is_q8(WK)) {
#pragma unroll
        for (int m = 0; m < NJ / 2; ++m) {
          mma(acc[u], dq8(ch.c[u][m].x, ch.c[u][m].y, ch.sc[u][m]), ch.b[2 * m]);
          mma(acc[u], dq8(ch.c[u][m].z, ch.c[u][m].w, ch.sc[u][m]), ch.b[2 * m + 1]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NJ; ++j) mma(acc[u], ch.a[u][j], ch.b[j]);
      }
    }
  }
}


// acc[u] += W_u[16 rows][ka, kb) . X[16 tokens][ka, kb)^T for u < cnt; ka, kb
// multiples of 64.  xr points at this lane's token row of X (xr[k] = X[t][k]).
// Software-pipelined: the next 128-wide chunk's loads are issued before the
// current chunk's MFMAs, so two chunks of loads are in flight per wave.
template <typename TA, int WK, int TPW>
__device__ __forceinline__ void stream_range_g(const TA *xr, const SRow<TA, WK> (&rows)[TPW], int cnt,
                                             int ka, int kb, int g, bool tok_ok,
                                             f32x4 (&acc)[TPW]) {
  const int nfull = (kb - ka) >> 7;
  int k = ka;
  if (nfull > 0) {
    Chunk<TA, WK, TPW, 4> c0, c1;
    chunk_load_g(c0, xr, rows, cnt, k, g, tok_ok);
    for (int c = 0; c < nfull; c += 2) {
      if (c + 1 < nfull) chunk_load_g(c1, xr, rows, cnt, k + 128, g, tok_ok);
      chunk_mma_g(c0, cnt, acc);
      k += 128;
      if (c + 1 < nfull) {
        if (c + 2 < nfull) chunk_load_g(c0, xr, rows, cnt, k + 128, g, tok_ok);
        chunk_mma_g(c1, cnt, acc);
        k += 128;
      }
    }
  }
  if (k < kb) {
    Chunk<TA, WK, TPW, 2> ct;
    chunk_load_g(ct, xr, rows, cnt, k, g, tok_ok);
    chunk_mma_g(ct, cnt, acc);
  }
}

template <typename TA, int WK, int TPW>
__device__ __forceinline__ void stream_k(const TA *xr, const SRow<TA, WK> (&rows)[TPW], int cnt, int ka,
                                         int kb, int g, bool tok_ok, f32x4 (&acc)[TPW]) {
  stream_range_g<TA, WK, TPW>(xr, rows, cnt, ka, kb, g, tok_ok, acc);
}

}  // namespace dfl
