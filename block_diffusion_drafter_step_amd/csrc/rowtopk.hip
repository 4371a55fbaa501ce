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
// One workgroup of 512 threads owns one segment of a row (at most 8192
// keys, held in LDS).  It finds the K-th largest key with eight radix passes
// over 8-bit digits (most significant first: a 256-bin histogram of the keys
// that still match the chosen prefix, then the digit whose bins reach the
// remaining rank; it stops early once that digit's keys are all kept), keeps
// the K keys at or above it.  A row wider than one segment yields one
// candidate list per segment; the same kernel then selects from those lists,
// until one segment is left, whose K keys are bitonic-sorted descending.  The
// final pass writes indices and re-reads the values from the input, so they
// are exact copies.
#include "common.h"
#include "kernels.h"

namespace dfl {

constexpr int kRowSelThreads = 512;

__device__ __forceinline__ unsigned long long row_key(float v, long col) {
  unsigned u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;   // -0.0 equals +0.0
  const unsigned o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)o << 32) | (unsigned)(~(unsigned)col);
}

// one pass: keys of row blockIdx.y, segment blockIdx.x ([seg0, seg0 + len)
// of a row of n_in inputs) -> the segment's K largest, sorted descending.
// FROM_KEYS: the input is a previous pass's key lists, else fp32 scores.
// Output: `keys_out` [row][n_seg][K] (0 pads a short segment), or, when
// n_seg == 1 and idx != nullptr, the final indices and values.
template <bool FROM_KEYS>
__global__ __launch_bounds__(kRowSelThreads) void rowsel_kernel(const void *__restrict__ in, long n_in,
                                                                int seg, int K, const float *__restrict__ x,
                                                                long n_cols, unsigned long long *keys_out,
                                                                int32_t *idx, float *val) {
  extern __shared__ __attribute__((aligned(16))) unsigned long long rs_keys[];
  __shared__ unsigned hist[256];
  __shared__ unsigned long long sel[1024];
  __shared__ unsigned sel_n;
  __shared__ unsigned pick_digit, pick_above;
  const int tid = threadIdx.x;
  const long row = blockIdx.y;
  const int n_seg = gridDim.x;
  const long seg0 = (long)blockIdx.x * seg;
  const int len = (int)min((long)seg, n_in - seg0);

  // load the segment's keys
  for (int i = tid; i < len; i += kRowSelThreads) {
    if constexpr (FROM_KEYS)
      rs_keys[i] = reinterpret_cast<const unsigned long long *>(in)[row * n_in + seg0 + i];
    else
      rs_keys[i] = row_key(reinterpret_cast<const float *>(in)[row * n_in + seg0 + i], seg0 + i);
  }
  if (tid == 0) sel_n = 0;
  __syncthreads();

  unsigned long long thr = 0;   // keys >= thr are kept
  if (len > K) {
    unsigned long long prefix = 0, mask = 0;
    unsigned remaining = (unsigned)K;
    for (int shift = 56; shift >= 0; shift -= 8) {
      for (int b = tid; b < 256; b += kRowSelThreads) hist[b] = 0;
      __syncthreads();
      for (int i = tid; i < len; i += kRowSelThreads) {
        const unsigned long long k = rs_keys[i];
        if ((k & mask) == prefix) atomicAdd(&hist[(unsigned)(k >> shift) & 255u], 1u);
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
    thr = prefix;   // exactly K keys are >= it
  }

  // keep keys >= thr (all of them when len <= K)
  const int n_keep = len > K ? K : len;
  for (int i = tid; i < len; i += kRowSelThreads) {
    const unsigned long long k = rs_keys[i];
    if (k >= thr) sel[atomicAdd(&sel_n, 1u)] = k;
  }
  __syncthreads();
  // bitonic sort of sel[0, P) descending, P = next power of two >= K, pads 0;
  // only the last pass sorts (the next pass takes its keys in any order)
  const bool last = n_seg == 1 && idx;
  int P = 1;
  while (last && P < K) P <<= 1;
  if (!last) P = 0;
  for (int i = n_keep + tid; i < (last ? P : K); i += kRowSelThreads) sel[i] = 0ull;
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < P / 2; t += kRowSelThreads) {
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
    for (int j = tid; j < K; j += kRowSelThreads) {
      // a row holds at least K real keys, so no pad (0) reaches the output;
      // the check only keeps a broken invariant from reading out of range
      const unsigned col = ~(unsigned)(sel[j] & 0xffffffffull);
      const bool ok = sel[j] != 0ull && (long)col < n_cols;
      idx[row * K + j] = ok ? (int32_t)col : -1;
      val[row * K + j] = ok ? x[row * n_cols + col] : __builtin_nanf("");
    }
  } else {
    for (int j = tid; j < K; j += kRowSelThreads)
      keys_out[(row * n_seg + blockIdx.x) * (long)K + j] = sel[j];
  }
}

// Segment width of a pass over rows of n elements: at most 8192 (LDS),
// at least 2K so every pass shrinks the candidates, smaller while the grid
// would leave CUs idle.
static int rowsel_seg(long n_rows, long n, int K) {
  const int lo = K * 2 > 1024 ? K * 2 : 1024;
  int seg = 8192;
  while (seg / 2 >= lo && n_rows * ((n + seg - 1) / seg) < 2 * 256) seg /= 2;
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
    const size_t lds = (size_t)seg * 8;
    if (keys) {
      (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&rowsel_kernel<true>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      hipLaunchKernelGGL(rowsel_kernel<true>, grid, dim3(kRowSelThreads), lds, st, in, n, seg, K, x, n_cols,
                         out, idx, val);
    } else {
      (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&rowsel_kernel<false>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      hipLaunchKernelGGL(rowsel_kernel<false>, grid, dim3(kRowSelThreads), lds, st, in, n, seg, K, x,
                         n_cols, out, idx, val);
    }
    if (n_seg == 1) break;
    in = out;
    n = n_seg * K;
    keys = true;
    ++pass;
  }
  return hipGetLastError();
}

}  // namespace dfl
