// Shared LM head with top-K candidates and log-softmax unary scores
// ("Turbo dflash", Overview: the draft uses the target's output matrix;
// "spec : add DFlash2 support", Overview: unary[c] is the draft's own score,
// and the top-k review: small K over a very wide row).
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
#include "common.h"
#include "kernels.h"

namespace dfl {

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kL2e = 1.4426950408889634f;

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

template <typename TA, int WK>
struct LmRow {
  const void *p;
  const uint16_t *s;
};

template <typename TA, int WK, int KM>
__global__ __launch_bounds__(256) void lmhead_topk_kernel(TopkArgs a) {
  constexpr int RT = 2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int d = a.d;
  const long V = a.V;
  const long ntiles = (V + 15) / 16;
  const long nwaves = (long)gridDim.x * 4;
  const long wid = (long)blockIdx.x * 4 + wave;
  const long t_beg = wid * ntiles / nwaves, t_end = (wid + 1) * ntiles / nwaves;
  const bool tok_ok = r16 < a.B;
  const TA *hr = reinterpret_cast<const TA *>(a.h) + (long)min(r16, a.B - 1) * d + 8 * g;
  const bool vec_scales = (d & 255) == 0;

  float tv[KM];
  int ti[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    tv[j] = -__builtin_inff();
    ti[j] = 0x7fffffff;
  }
  float m = -__builtin_inff(), ssum = 0.f;

  for (long t = t_beg; t < t_end; t += RT) {
    const void *wp[RT];
    const uint16_t *sp[RT];
#pragma unroll
    for (int u = 0; u < RT; ++u) {
      const long row = min((t + u) * 16 + r16, V - 1);
      if constexpr (WK == W_Q8_0) {
        wp[u] = reinterpret_cast<const int8_t *>(a.w) + row * d;
        sp[u] = reinterpret_cast<const uint16_t *>(a.scales) + row * (d >> 5);
      } else {
        wp[u] = reinterpret_cast<const TA *>(a.w) + row * d;
        sp[u] = nullptr;
      }
    }
    f32x4 acc[RT];
#pragma unroll
    for (int u = 0; u < RT; ++u) acc[u] = zero4();
    int k = 0;
    for (; k + 256 <= d; k += 256) {
      Frag<TA> b[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = tok_ok ? load_frag(hr + k + 32 * j) : frag_zero<TA>();
      if constexpr (WK == W_Q8_0) {
        Frag<bf16> af[RT][8];
#pragma unroll
        for (int u = 0; u < RT; ++u) {
          const int8_t *q = reinterpret_cast<const int8_t *>(wp[u]) + k + 8 * g;
          uint2 c[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) c[j] = *reinterpret_cast<const uint2 *>(q + 32 * j);
          float sc[8];
          if (vec_scales) {
            const uint4 s4 = *reinterpret_cast<const uint4 *>(sp[u] + (k >> 5));
            const uint32_t w4[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
            for (int j = 0; j < 8; ++j)
              sc[j] = half_bits_to_f32((uint16_t)(w4[j >> 1] >> (16 * (j & 1))));
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) sc[j] = half_bits_to_f32(sp[u][(k >> 5) + j]);
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) af[u][j] = dequant8(c[j], sc[j]);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int u = 0; u < RT; ++u) mma(acc[u], af[u][j], b[j]);
      } else {
        Frag<TA> af[RT][8];
#pragma unroll
        for (int u = 0; u < RT; ++u)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            af[u][j] = load_frag(reinterpret_cast<const TA *>(wp[u]) + k + 32 * j + 8 * g);
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int u = 0; u < RT; ++u) mma(acc[u], af[u][j], b[j]);
      }
    }
    for (; k < d; k += 32) {
      const Frag<TA> b = tok_ok ? load_frag(hr + k) : frag_zero<TA>();
#pragma unroll
      for (int u = 0; u < RT; ++u) {
        if constexpr (WK == W_Q8_0) {
          const uint2 c = *reinterpret_cast<const uint2 *>(reinterpret_cast<const int8_t *>(wp[u]) + k + 8 * g);
          mma(acc[u], dequant8(c, half_bits_to_f32(sp[u][k >> 5])), b);
        } else {
          mma(acc[u], load_frag(reinterpret_cast<const TA *>(wp[u]) + k + 8 * g), b);
        }
      }
    }
    // fold: lane holds rows (t+u)*16 + 4g + i of token r16
#pragma unroll
    for (int u = 0; u < RT; ++u) {
      float v[4];
      float tmax = -__builtin_inff();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const long row = (t + u) * 16 + 4 * g + i;
        v[i] = (t + u < t_end && row < V) ? acc[u][i] : -__builtin_inff();
        tmax = fmaxf(tmax, v[i]);
      }
      if (tmax > m) {
        ssum *= exp2f((m - tmax) * kL2e);
        m = tmax;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (v[i] != -__builtin_inff()) ssum += exp2f((v[i] - m) * kL2e);
        list_insert<KM>(tv, ti, v[i], (int)((t + u) * 16 + 4 * g + i));
      }
    }
  }

  // merge the 16 lists of each token (4 lane groups x 4 waves) through LDS:
  // thread (token = tid / 16, list q = tid % 16) offers its list's head; a
  // 16-lane argmax by (value desc, index asc) picks the next entry K times
  __shared__ float lv[256 * KM];
  __shared__ int li[256 * KM];
  __shared__ float lm[256], ls[256];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    lv[tid * KM + j] = tv[j];
    li[tid * KM + j] = ti[j];
  }
  lm[tid] = m;
  ls[tid] = ssum;
  __syncthreads();
  {
    const int tok = tid >> 4, q = tid & 15;
    // list q of token tok was written by thread (q/4)*64 + (q%4)*16 + tok
    const int src = (q >> 2) * 64 + (q & 3) * 16 + tok;
    float pm = lm[src];
    float M = pm;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) M = fmaxf(M, shfl_xor(M, o));
    float ps = ls[src] > 0.f ? ls[src] * exp2f((pm - M) * kL2e) : 0.f;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) ps += shfl_xor(ps, o);
    const long ob = (long)blockIdx.x * 16 + tok;
    if (q == 0) {
      a.part_ms[ob * 2] = M;
      a.part_ms[ob * 2 + 1] = ps;
    }
    int head = 0;
    for (int k = 0; k < a.K; ++k) {
      float bv = head < KM ? lv[src * KM + head] : -__builtin_inff();
      int bi = head < KM ? li[src * KM + head] : 0x7fffffff;
      int bq = q;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
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
        a.part_val[ob * a.K + k] = bv;
        a.part_idx[ob * a.K + k] = bi;
      }
    }
  }
}

// one workgroup per token: merge n_wg partial lists and (max, sum) pairs
template <int KM>
__global__ __launch_bounds__(256) void topk_merge_kernel(TopkArgs a) {
  const int tok = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K;
  float tv[KM];
  int ti[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    tv[j] = -__builtin_inff();
    ti[j] = 0x7fffffff;
  }
  float m = -__builtin_inff(), s = 0.f;
  for (int w = tid; w < a.n_wg; w += 256) {
    const long ob = (long)w * 16 + tok;
    const float pm = a.part_ms[ob * 2], ps = a.part_ms[ob * 2 + 1];
    if (ps > 0.f) {
      if (pm > m) {
        s = s * exp2f((m - pm) * kL2e);
        m = pm;
      }
      s += ps * exp2f((pm - m) * kL2e);
    }
    for (int k = 0; k < K; ++k) {
      const float v = a.part_val[ob * K + k];
      const int ix = a.part_idx[ob * K + k];
      // general insertion by (value desc, index asc)
      if (better(v, ix, tv[KM - 1], ti[KM - 1])) {
        tv[KM - 1] = v;
        ti[KM - 1] = ix;
#pragma unroll
        for (int j = KM - 1; j > 0; --j) {
          const bool sw = better(tv[j], ti[j], tv[j - 1], ti[j - 1]);
          const float xv = tv[j - 1];
          const int xi = ti[j - 1];
          tv[j - 1] = sw ? tv[j] : xv;
          ti[j - 1] = sw ? ti[j] : xi;
          tv[j] = sw ? xv : tv[j];
          ti[j] = sw ? xi : ti[j];
        }
      }
    }
  }
  __shared__ float lv[256 * KM];
  __shared__ int li[256 * KM];
  __shared__ float wm[4], wsum[4], wv[4];
  __shared__ int wi[4], wq[4];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    lv[tid * KM + j] = tv[j];
    li[tid * KM + j] = ti[j];
  }
  // log-sum-exp: fixed-order tree over the 256 threads
  float M = m;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) M = fmaxf(M, shfl_xor(M, o));
  if (lane == 0) wm[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
  float S = s > 0.f ? s * exp2f((m - M) * kL2e) : 0.f;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) S += shfl_xor(S, o);
  if (lane == 0) wsum[wave] = S;
  __syncthreads();
  S = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
  const float lse = M + log2f(S) * kLn2;
  int head = 0;
  for (int k = 0; k < K; ++k) {
    float bv = head < KM ? lv[tid * KM + head] : -__builtin_inff();
    int bi = head < KM ? li[tid * KM + head] : 0x7fffffff;
    int bq = tid;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float ov = shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o, kWave);
      const int oq = __shfl_xor(bq, o, kWave);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
        bq = oq;
      }
    }
    if (lane == 0) {
      wv[wave] = bv;
      wi[wave] = bi;
      wq[wave] = bq;
    }
    __syncthreads();
    float fv = wv[0];
    int fi = wi[0], fq = wq[0];
#pragma unroll
    for (int w = 1; w < 4; ++w)
      if (better(wv[w], wi[w], fv, fi)) {
        fv = wv[w];
        fi = wi[w];
        fq = wq[w];
      }
    if (fq == tid) ++head;
    if (tid == 0) {
      a.idx[(long)tok * K + k] = fi;
      a.unary[(long)tok * K + k] = fv - lse;
    }
    __syncthreads();
  }
}

int topk_plan_wgs(long V) {
  const long ntiles = (V + 15) / 16;
  long wgs = 512;
  // every wave should own at least one 16-row tile
  if (wgs * 4 > ntiles) wgs = (ntiles + 3) / 4;
  return (int)(wgs < 1 ? 1 : wgs);
}

template <typename TA, int WK, int KM>
static void topk_launch_t(const TopkArgs &a, hipStream_t st) {
  hipLaunchKernelGGL((lmhead_topk_kernel<TA, WK, KM>), dim3(a.n_wg), dim3(256), 0, st, a);
  hipLaunchKernelGGL((topk_merge_kernel<KM>), dim3(a.B), dim3(256), 0, st, a);
}

template <typename TA, int WK>
static void topk_launch_k(const TopkArgs &a, hipStream_t st) {
  if (a.K <= 4) topk_launch_t<TA, WK, 4>(a, st);
  else if (a.K <= 8) topk_launch_t<TA, WK, 8>(a, st);
  else if (a.K <= 16) topk_launch_t<TA, WK, 16>(a, st);
  else topk_launch_t<TA, WK, 32>(a, st);
}

hipError_t launch_topk(int act, int wkind, const TopkArgs &a, hipStream_t st) {
  if (act == ACT_F32) topk_launch_k<float, W_SAME>(a, st);
  else if (wkind == W_Q8_0) topk_launch_k<bf16, W_Q8_0>(a, st);
  else topk_launch_k<bf16, W_SAME>(a, st);
  return hipGetLastError();
}

}  // namespace dfl
