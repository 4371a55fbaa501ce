// Row-wise top-K of an fp32 score matrix, K <= 1024 ("spec : add DFlash2
// support", the top-k kernel review: a small K selected from very wide rows).
//
// Every element becomes a unique 64-bit key: high word the float's bits made
// order-preserving (negative values complemented, the sign bit set on the
// others; -0.0 is read as +0.0), low word the complemented column index.
// Descending key order is then value descending with equal values in
// ascending index order, and no two keys are equal, so "the K largest keys"
// is exactly the requested set.
//
// One workgroup of 512 threads (128 for segments of at most
// DFL_ROWSEL_SMALL_SEG keys) owns one segment of a row (at most 8192 keys,
// 16 per thread, kept in registers; every load of a thread is issued
// before the first is used).  It finds the K-th largest key with eight radix
// passes over 8-bit digits (most significant first: a 256-bin histogram of
// the keys that still match the chosen prefix, then the digit whose bins
// reach the remaining rank; it stops early once that digit's keys are all
// kept), keeps the K keys at or above it.  A row wider than one segment
// yields one candidate list per segment, padded with the key 0 (no element
// has it: the index word of a real key is at least 2^31) when the segment
// held fewer than K; the same kernel then selects from those lists, pads not
// counted, until one segment is left, whose K keys are bitonic-sorted
// descending.  The final pass writes indices and re-reads the values from
// the input, so they are exact copies.
#include "common.h"
#include "kernels.h"

namespace dfl {

constexpr int kRowSelThreads = 512;
constexpr int kRowSelMaxSeg = 8192;
constexpr int kRowSelPer = kRowSelMaxSeg / kRowSelThreads;   // keys per thread
constexpr int kRowSelMaxK = 1024;
#ifndef DFL_ROWSEL_COPIES
#define DFL_ROWSEL_COPIES 8   // histogram copies (lane l adds to copy l % copies)
#endif
constexpr int kRowSelCopies = DFL_ROWSEL_COPIES;
#ifndef DFL_ROWSEL_SMALL_SEG
#define DFL_ROWSEL_SMALL_SEG 512   // segments up to this many keys run on 128 threads
#endif
static_assert(DFL_ROWSEL_SMALL_SEG <= 128 * kRowSelPer, "a 128-thread segment holds 16 keys per thread");
static_assert((kRowSelCopies & (kRowSelCopies - 1)) == 0 && kRowSelCopies <= 64, "copies: a power of two");

__device__ __forceinline__ unsigned long long row_key(float v, long col) {
  unsigned u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;   // -0.0 equals +0.0
  const unsigned o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)o << 32) | (unsigned)(~(unsigned)col);
}

// one pass: keys of row blockIdx.y, segment blockIdx.x ([seg0, seg0 + len)
// of a row of n_in inputs) -> the segment's K largest keys (sorted
// descending in the final pass).  FROM_KEYS: the input is a previous pass's
// key lists, else fp32 scores.  Output: `keys_out` [row][n_seg][K] (0 pads
// a short list), or, when n_seg == 1 and idx != nullptr, the final indices
// and values.
template <bool FROM_KEYS, int NT>
__global__ __launch_bounds__(NT) void rowsel_kernel(const void *__restrict__ in, long n_in,
                                                                int seg, int K, const float *__restrict__ x,
                                                                long n_cols, unsigned long long *keys_out,
                                                                int32_t *idx, float *val) {
  __shared__ unsigned histc[kRowSelCopies * 257];   // copy c at 257 c (banks staggered)
  __shared__ unsigned hist[256];
  __shared__ unsigned long long sel[kRowSelMaxK];
  __shared__ unsigned sel_n, n_real;
  __shared__ unsigned pick_digit, pick_above;
  const int tid = threadIdx.x;
  const long row = blockIdx.y;
  const int n_seg = gridDim.x;
  const long seg0 = (long)blockIdx.x * seg;
  const int len = (int)min((long)seg, n_in - seg0);
  const long base = row * n_in + seg0;

  // this thread's keys: segment entries tid + j * NT; 0 = no key (past the
  // segment, or a pad).  Loads past the segment re-read its last entry, so
  // the only condition on a load is the segment width (the same for every
  // thread) and they are issued back to back.
  unsigned long long kv[kRowSelPer];
  if constexpr (FROM_KEYS) {
    const unsigned long long *src = reinterpret_cast<const unsigned long long *>(in) + base;
#pragma unroll
    for (int j = 0; j < kRowSelPer; ++j)
      if (j * NT < seg) kv[j] = src[min(tid + j * NT, len - 1)];
#pragma unroll
    for (int j = 0; j < kRowSelPer; ++j)
      if (!(j * NT < seg && tid + j * NT < len)) kv[j] = 0ull;
  } else {
    const float *src = reinterpret_cast<const float *>(in) + base;
    float xv[kRowSelPer];
#pragma unroll
    for (int j = 0; j < kRowSelPer; ++j)
      if (j * NT < seg) xv[j] = src[min(tid + j * NT, len - 1)];
#pragma unroll
    for (int j = 0; j < kRowSelPer; ++j) {
      const int i = tid + j * NT;
      kv[j] = j * NT < seg && i < len ? row_key(xv[j], seg0 + i) : 0ull;
    }
  }
  if (tid == 0) {
    sel_n = 0;
    n_real = 0;
  }
  for (int b = tid; b < kRowSelCopies * 257; b += NT) histc[b] = 0;
  __syncthreads();
  // keys in the segment (pads of a previous pass excluded)
  unsigned nr = (unsigned)len;
  if constexpr (FROM_KEYS) {
    unsigned c = 0;
#pragma unroll
    for (int j = 0; j < kRowSelPer; ++j) c += kv[j] != 0ull;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) c += __shfl_xor(c, o, 64);
    if ((tid & 63) == 0) atomicAdd(&n_real, c);
    __syncthreads();
    nr = n_real;
  }

  unsigned long long thr = 1ull;   // keys >= thr are kept (every key when nr <= K)
  if (nr > (unsigned)K) {
    unsigned long long prefix = 0, mask = 0;
    unsigned remaining = (unsigned)K;
    for (int shift = 56; shift >= 0; shift -= 8) {
      // keys crowd into few bins (the leading digits of similar floats
      // agree), so the lanes of a wave add to separate copies; the copies
      // are zero here (cleared at the start, and by each pass's summation)
      unsigned *mine = histc + (tid & (kRowSelCopies - 1)) * 257;
#pragma unroll
      for (int j = 0; j < kRowSelPer; ++j) {
        const unsigned long long k = kv[j];
        if (k != 0ull && (k & mask) == prefix) atomicAdd(&mine[(unsigned)(k >> shift) & 255u], 1u);
      }
      __syncthreads();
      for (int b = tid; b < 256; b += NT) {
        unsigned sum = 0;
#pragma unroll
        for (int c = 0; c < kRowSelCopies; ++c) {
          sum += histc[c * 257 + b];
          histc[c * 257 + b] = 0;
        }
        hist[b] = sum;
      }
      __syncthreads();
      // wave 0: lane l holds bins 252 - 4l .. 255 - 4l (descending digits);
      // counts above each lane's range by a suffix scan over the lanes
      if (tid < 64) {
        const int l = tid;
        unsigned c[4], s = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c[j] = hist[255 - 4 * l - j];
          s += c[j];
        }
        unsigned incl = s;   // inclusive prefix over lanes 0..l (higher digits first)
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const unsigned t = __shfl_up(incl, o, 64);
          if (l >= o) incl += t;
        }
        const unsigned before = incl - s;
        if (before < remaining && remaining <= incl) {
          unsigned acc = before;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (acc < remaining && remaining <= acc + c[j]) {
              pick_digit = (unsigned)(255 - 4 * l - j);
              pick_above = acc;
            }
            acc += c[j];
          }
        }
      }
      __syncthreads();
      const unsigned d = pick_digit;
      remaining -= pick_above;
      prefix |= (unsigned long long)d << shift;
      mask |= 0xffull << shift;
      // every key left in digit d is kept: the threshold is that digit with
      // all lower bits zero (the same value on every thread)
      const bool done = hist[d] == remaining;
      __syncthreads();   // pick_* and hist are rewritten by the next pass
      if (done) break;
    }
    thr = prefix;   // exactly K keys are >= it (keys are unique and nonzero)
  }

  // keep keys >= thr; the bound on the slot only guards a broken invariant
  const int n_keep = nr > (unsigned)K ? K : (int)nr;
#pragma unroll
  for (int j = 0; j < kRowSelPer; ++j) {
    const unsigned long long k = kv[j];
    if (k != 0ull && k >= thr) {
      const unsigned slot = atomicAdd(&sel_n, 1u);
      if (slot < (unsigned)kRowSelMaxK) sel[slot] = k;
    }
  }
  __syncthreads();
  // bitonic sort of sel[0, P) descending, P = next power of two >= K, pads 0;
  // only the last pass sorts (the next pass takes its keys in any order)
  const bool last = n_seg == 1 && idx;
  int P = 1;
  while (last && P < K) P <<= 1;
  if (!last) P = 0;
  for (int i = n_keep + tid; i < (last ? P : K); i += NT) sel[i] = 0ull;
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < P / 2; t += NT) {
        const int i = 2 * t - (t & (stride - 1));   // lower element of the pair
        const int j = i + stride;
        const bool desc = (i & size) == 0;          // direction of this run
        const unsigned long long a = sel[i], b = sel[j];
        if (desc ? a < b : a > b) {
          sel[i] = b;
          sel[j] = a;
        }
      }
      __syncthreads();
    }
  }

  if (last) {
    for (int j = tid; j < K; j += NT) {
      // a row holds at least K real keys, so no pad (0) reaches the output;
      // the check only keeps a broken invariant from reading out of range
      const unsigned col = ~(unsigned)(sel[j] & 0xffffffffull);
      const bool ok = sel[j] != 0ull && (long)col < n_cols;
      idx[row * K + j] = ok ? (int32_t)col : -1;
      val[row * K + j] = ok ? x[row * n_cols + col] : __builtin_nanf("");
    }
  } else {
    for (int j = tid; j < K; j += NT)
      keys_out[(row * n_seg + blockIdx.x) * (long)K + j] = sel[j];
  }
}

// Segment width of a pass over rows of n elements: at most 8192 (16 keys
// per thread), at least 2K so every pass shrinks the candidates, smaller
// while the grid would leave CUs idle.  A row that fits one segment takes
// the smallest width (a power of two, at least 512) that holds it, so its
// threads issue no loads past the row.
static int rowsel_seg(long n_rows, long n, int K) {
  const int lo = K * 2 > 1024 ? K * 2 : 1024;
  int seg = kRowSelMaxSeg;
  while (seg / 2 >= lo && n_rows * ((n + seg - 1) / seg) < 2 * 256) seg /= 2;
  if (n <= seg) {
    int fit = kRowSelThreads;
    while (fit < n) fit *= 2;
    seg = fit;
  }
  return seg;
}

// candidate keys after each pass (the buffers alternate)
void rowtopk_plan(long n_rows, long n_cols, int K, size_t *buf_a, size_t *buf_b) {
  *buf_a = *buf_b = 0;
  long n = n_cols;
  int pass = 0;
  while (true) {
    const int seg = rowsel_seg(n_rows, n, K);
    const long n_seg = (n + seg - 1) / seg;
    if (n_seg == 1) break;
    const size_t bytes = (size_t)n_rows * n_seg * K * 8;
    size_t *b = (pass & 1) ? buf_b : buf_a;
    if (bytes > *b) *b = bytes;
    n = n_seg * K;
    ++pass;
  }
}

hipError_t launch_rowtopk(const float *x, long n_rows, long n_cols, int K, int32_t *idx, float *val,
                          void *buf_a, void *buf_b, hipStream_t st) {
  const void *in = x;
  long n = n_cols;
  bool keys = false;
  int pass = 0;
  while (true) {
    const int seg = rowsel_seg(n_rows, n, K);
    const long n_seg = (n + seg - 1) / seg;
    unsigned long long *out =
        n_seg == 1 ? nullptr : reinterpret_cast<unsigned long long *>((pass & 1) ? buf_b : buf_a);
    const dim3 grid((unsigned)n_seg, (unsigned)n_rows);
    const bool small = seg <= DFL_ROWSEL_SMALL_SEG;
    if (keys && small)
      hipLaunchKernelGGL((rowsel_kernel<true, 128>), grid, dim3(128), 0, st, in, n, seg, K, x, n_cols, out,
                         idx, val);
    else if (keys)
      hipLaunchKernelGGL((rowsel_kernel<true, kRowSelThreads>), grid, dim3(kRowSelThreads), 0, st, in, n, seg,
                         K, x, n_cols, out, idx, val);
    else if (small)
      hipLaunchKernelGGL((rowsel_kernel<false, 128>), grid, dim3(128), 0, st, in, n, seg, K, x, n_cols, out,
                         idx, val);
    else
      hipLaunchKernelGGL((rowsel_kernel<false, kRowSelThreads>), grid, dim3(kRowSelThreads), 0, st, in, n,
                         seg, K, x, n_cols, out, idx, val);
    if (n_seg == 1) break;
    in = out;
    n = n_seg * K;
    keys = true;
    ++pass;
  }
  return hipGetLastError();
}

}  // namespace dfl
