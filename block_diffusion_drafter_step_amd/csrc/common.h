// Device helpers shared by the libdflash kernels (gfx950 / CDNA4 only).
//
// Matrix products use the wave64 MFMA instruction v_mfma_f32_16x16x32_bf16.
// A "fragment" is the 8 consecutive k-elements one lane contributes to one
// 16x16x32 product: lane l supplies row (l % 16) of A (or column (l % 16) of
// B) and the k-slot group (l / 16).  The contraction is a sum over k, so
// which physical k a (lane group, slot) pair stands for is free as long as
// the A and B fragments of one product agree; every kernel here assigns
// lane group g the k-range [8g, 8g + 8) of each 32-wide k step, for A and B
// alike.  The 16x16 fp32 result is held as 4 values per lane: lane l holds
// rows 4 * (l / 16) + i (i = 0..3) of column l % 16.
//
// fp32 inputs use the same fragment shape and issue eight
// v_mfma_f32_16x16x4_f32 products, slot s of every lane group forming the
// s-th product; the k-sum is again the same.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfl {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { f32x8 v; };

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// float -> bf16 rounds to nearest even (v_cvt_pk_bf16_f32 on gfx950)
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

template <typename T> __device__ __forceinline__ Frag<T> frag_zero() {
  Frag<T> f;
#pragma unroll
  for (int s = 0; s < 8; ++s) f.v[s] = (T)0.0f;
  return f;
}

// 8 consecutive elements (16 B for bf16, 32 B for fp32); p must be aligned.
__device__ __forceinline__ Frag<bf16> load_frag(const bf16 *p) {
  Frag<bf16> f;
  f.v = *reinterpret_cast<const bf16x8 *>(p);
  return f;
}
__device__ __forceinline__ Frag<float> load_frag(const float *p) {
  Frag<float> f;
  const float4 a = reinterpret_cast<const float4 *>(p)[0];
  const float4 b = reinterpret_cast<const float4 *>(p)[1];
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
  return f;
}

// eight consecutive elements stored as one (bf16: 16-byte, fp32: 32-byte) access
__device__ __forceinline__ void store_frag(bf16 *p, const Frag<bf16> &f) {
  *reinterpret_cast<bf16x8 *>(p) = f.v;
}
__device__ __forceinline__ void store_frag(float *p, const Frag<float> &f) {
  *reinterpret_cast<f32x8 *>(p) = f.v;
}

// Q8_0: 8 int8 codes of one 32-block times the block's fp16 scale, each
// product rounded to bf16 (the declared rounding point of the Q8_0 path).
__device__ __forceinline__ Frag<bf16> dequant8(uint2 codes, float scale) {
  Frag<bf16> f;
  const int lo = (int)codes.x, hi = (int)codes.y;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const float a = (float)((lo << (24 - 8 * s)) >> 24);
    const float b = (float)((hi << (24 - 8 * s)) >> 24);
    f.v[s] = (bf16)(a * scale);
    f.v[4 + s] = (bf16)(b * scale);
  }
  return f;
}

__device__ __forceinline__ float half_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ void mma(f32x4 &acc, const Frag<bf16> &a, const Frag<bf16> &b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4 &acc, const Frag<float> &a, const Frag<float> &b) {
#pragma unroll
  for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[s], b.v[s], acc, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() {
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return z;
}

// Element i of a small pointer array held in kernel arguments, selected with
// compares so the array is never copied to per-lane scratch memory.
template <int N>
__device__ __forceinline__ const void *pick(const void *const (&a)[N], int i) {
  const void *r = a[0];
#pragma unroll
  for (int j = 1; j < N; ++j) r = (i == j) ? a[j] : r;
  return r;
}
template <int N>
__device__ __forceinline__ int pick(const int (&a)[N], int i) {
  int r = a[0];
#pragma unroll
  for (int j = 1; j < N; ++j) r = (i == j) ? a[j] : r;
  return r;
}

// Completion counter of one group of workgroups: a 64-bit word (stamp << 16)
// | count.  `stamp` is unique to the launch, so a word holding any other
// stamp (left by an earlier launch, a call that never completed, or anything
// else written there) counts as zero arrivals: the counters need no clearing,
// in any order of calls.  An arrival first claims the word for its launch --
// a compare-and-swap to (stamp << 16) | 0, tried only while the word still
// holds another stamp, so it never undoes an arrival of this launch -- and
// then counts itself with one fetch-and-add.  No arrival retries more than
// once, however many workgroups finish together (a compare-and-swap loop on
// the count serialises them at one agent-scope round trip each).  Returns
// true for the n-th arrival of this launch.  Release on the add: this
// workgroup's partials are visible before it is counted.
__device__ __forceinline__ bool arrive_last(unsigned long long *c, unsigned long long stamp, int n) {
  unsigned long long old = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  while ((old >> 16) != stamp &&
         !__hip_atomic_compare_exchange_strong(c, &old, stamp << 16, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT)) {
  }
  const unsigned long long prev = __hip_atomic_fetch_add(c, 1ull, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  return (int)(prev & 0xffffu) + 1 == n;
}

// Cross-lane helpers over the 64-wide wave.
__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, kWave); }

}  // namespace dfl
