// Non-causal block attention over [injected context | block] ("Turbo dflash",
// Overview and The Problem; the block's positions all see each other and
// the whole injected cache).
//
// The work is HBM-bound: every context K/V row is read once and used by all
// query heads of its GQA group (Hq/Hkv heads x B block tokens).  A workgroup
// owns one KV head and one contiguous chunk of keys (split-K over the context,
// "flash-decoding"); its 4 waves share each 64-key K/V tile through LDS and
// each wave runs one query head of the group against it:
//   S^T = K_tile Q_h^T        (keys x tokens, 16x16x32 MFMA, K from LDS)
//   online softmax per token   (fp32, base-2 exponent, running max / sum)
//   O^T += V_tile^T P^T        (dims x tokens; V is stored transposed in LDS)
// The S^T layout leaves each lane with one token and eight keys, which is
// exactly the B-operand layout P^T needs, so probabilities never leave
// registers.  A second kernel merges the splits with their log-sum-exp
// weights in a fixed order.
#include "common.h"
#include "kernels.h"

namespace dfl {

// keys per LDS tile (64 or 128) and the number of split workgroups aimed for
#ifndef DFL_ATTN_KT
#define DFL_ATTN_KT 64
#endif
#ifndef DFL_ATTN_WGS
#define DFL_ATTN_WGS 512
#endif
constexpr int kAttnKT = DFL_ATTN_KT;
constexpr float kLog2e = 1.4426950408889634f;

// four consecutive elements moved as one 8-byte (bf16) or 16-byte (fp32) access
template <typename TA>
struct alignas(4 * sizeof(TA)) Quad {
  TA v[4];
};

template <typename TA, int HD>
struct AttnCfg {
  static constexpr int KPAD = 16 / (int)sizeof(TA);
  static constexpr int KLD = HD + KPAD;             // K tile row (elements)
  static constexpr int VLD = kAttnKT + 4;           // Vt row: the tile's keys + 4
  static constexpr int VEC = 16 / (int)sizeof(TA);  // elements per 16-byte chunk
  static constexpr int NQF = HD / 32;               // Q fragments (k-steps over dims)
  static constexpr int NDT = HD / 16;               // 16-dim output tiles
};

// pointer to row `j` of the keys (or values) seen by KV head `kvh`
template <typename TA, int HD>
__device__ __forceinline__ const TA *key_row(const AttnArgs &a, const TA *cache, int kvh, long j,
                                             int col_off) {
  if (j < a.n_ctx) return cache + ((long)kvh * a.cap + j) * HD;
  const long t = j - a.n_ctx;
  const long qld = (long)(a.Hq + 2 * a.Hkv) * HD;
  return reinterpret_cast<const TA *>(a.qkv) + t * qld + col_off + (long)kvh * HD;
}

template <typename TA, int HD, int HPW>
__global__ __launch_bounds__(256) void attn_split_kernel(AttnArgs a) {
  using C = AttnCfg<TA, HD>;
  __shared__ __attribute__((aligned(16))) TA Ks[kAttnKT * C::KLD];
  __shared__ __attribute__((aligned(16))) TA Vt[HD * C::VLD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int kvh = blockIdx.y, sp = blockIdx.x;
  const int grp = a.Hq / a.Hkv;
  const long S = a.n_ctx + a.B;
  const long key0 = (long)sp * a.chunk;
  const long key1 = min(S, key0 + a.chunk);
  const TA *ck = reinterpret_cast<const TA *>(a.ck);
  const TA *cv = reinterpret_cast<const TA *>(a.cv);
  const int kcol = a.Hq * HD, vcol = (a.Hq + a.Hkv) * HD;
  const long qld = (long)(a.Hq + 2 * a.Hkv) * HD;
  const float sl2 = a.scale * kLog2e;

  // this wave's query heads: hq = kvh*grp + wave + 4*hh, hh < HPW
  Frag<TA> qf[HPW][C::NQF];
  f32x4 o[HPW][C::NDT];
  float m_run[HPW], l_run[HPW];
  bool active[HPW];
  const bool tok_ok = r16 < a.B;
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const int hl = wave + 4 * hh;
    active[hh] = hl < grp;
    const int hq = kvh * grp + (active[hh] ? hl : 0);
    const TA *qp = reinterpret_cast<const TA *>(a.qkv) + (long)min(r16, a.B - 1) * qld + (long)hq * HD;
#pragma unroll
    for (int f = 0; f < C::NQF; ++f)
      qf[hh][f] = tok_ok ? load_frag(qp + 32 * f + 8 * g) : frag_zero<TA>();
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) o[hh][dt] = zero4();
    m_run[hh] = -__builtin_inff();
    l_run[hh] = 0.f;
  }

  // tile loader: K chunks copied as-is; V gathered 4 keys x 8 dims per thread
  // and written transposed
  constexpr int KCH = kAttnKT * HD / C::VEC;            // 16-byte K chunks per tile
  constexpr int VITEMS = (kAttnKT / 4) * (HD / 8);       // (4 keys x 8 dims) V items
  constexpr int KPT = (KCH + 255) / 256, VPT = (VITEMS + 255) / 256;
  uint4 kreg[KPT];
  Frag<TA> vreg[VPT][4];

  auto load_tile = [&](long t0) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int c = tid + 256 * j;
      const int row = c / (HD / C::VEC), ch = c % (HD / C::VEC);
      const long key = t0 + row;
      kreg[j] = make_uint4(0, 0, 0, 0);
      if (c < KCH && key < key1)
        kreg[j] = *reinterpret_cast<const uint4 *>(key_row<TA, HD>(a, ck, kvh, key, kcol) + ch * C::VEC);
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int it = tid + 256 * j;
      const int kq = it / (HD / 8), d8 = it % (HD / 8);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const long key = t0 + 4 * kq + u;
        vreg[j][u] = (it < VITEMS && key < key1)
                         ? load_frag(key_row<TA, HD>(a, cv, kvh, key, vcol) + d8 * 8)
                         : frag_zero<TA>();
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int c = tid + 256 * j;
      if (c < KCH) {
        const int row = c / (HD / C::VEC), ch = c % (HD / C::VEC);
        *reinterpret_cast<uint4 *>(Ks + row * C::KLD + ch * C::VEC) = kreg[j];
      }
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int it = tid + 256 * j;
      if (it < VITEMS) {
        const int kq = it / (HD / 8), d8 = it % (HD / 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          Quad<TA> q4;
#pragma unroll
          for (int u = 0; u < 4; ++u) q4.v[u] = vreg[j][u].v[e];
          *reinterpret_cast<Quad<TA> *>(Vt + (d8 * 8 + e) * C::VLD + 4 * kq) = q4;
        }
      }
    }
  };

  const int ntile = (int)((key1 - key0 + kAttnKT - 1) / kAttnKT);
  load_tile(key0);
  store_tile();
  __syncthreads();
  for (int tI = 0; tI < ntile; ++tI) {
    const long t0 = key0 + (long)tI * kAttnKT;
    const long tn = key0 + (long)min(tI + 1, ntile - 1) * kAttnKT;
    load_tile(tn);
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      if (!active[hh]) continue;
#pragma unroll
      for (int sb = 0; sb < kAttnKT / 32; ++sb) {
        // S^T for 32 keys: two 16-key tiles, lane holds keys 4g+i (+16), token r16
        f32x4 s[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          s[st] = zero4();
          const TA *kp = Ks + (32 * sb + 16 * st + r16) * C::KLD + 8 * g;
#pragma unroll
          for (int f = 0; f < C::NQF; ++f) mma(s[st], load_frag(kp + 32 * f), qf[hh][f]);
        }
        float p[8];
        float mx = -__builtin_inff();
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const long key = t0 + 32 * sb + 16 * st + 4 * g + i;
            const float v = key < key1 ? s[st][i] * sl2 : -__builtin_inff();
            p[st * 4 + i] = v;
            mx = fmaxf(mx, v);
          }
        mx = fmaxf(mx, shfl_xor(mx, 16));
        mx = fmaxf(mx, shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run[hh], mx);
        const float alpha = m_new == -__builtin_inff() ? 1.f : exp2f(m_run[hh] - m_new);
        // the row sum uses the probabilities exactly as the P.V product sees them
        float ls = 0.f;
        Frag<TA> pf;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pf.v[e] = from_f32<TA>(p[e] == -__builtin_inff() ? 0.f : exp2f(p[e] - m_new));
          ls += to_f32(pf.v[e]);
        }
        ls += shfl_xor(ls, 16);
        ls += shfl_xor(ls, 32);
        l_run[hh] = l_run[hh] * alpha + ls;
        m_run[hh] = m_new;
        // O^T[dim][tok] += V^T[dim][keys] P^T[keys][tok]; lane slots: keys 4g..4g+3, 16+4g..
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) {
          o[hh][dt] *= alpha;
          const TA *vp = Vt + (16 * dt + r16) * C::VLD + 32 * sb + 4 * g;
          const Quad<TA> v0 = *reinterpret_cast<const Quad<TA> *>(vp);
          const Quad<TA> v1 = *reinterpret_cast<const Quad<TA> *>(vp + 16);
          Frag<TA> vf;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            vf.v[e] = v0.v[e];
            vf.v[4 + e] = v1.v[e];
          }
          mma(o[hh][dt], vf, pf);
        }
      }
    }
    __syncthreads();
    store_tile();
    __syncthreads();
  }

  // partials: lane holds dims 16*dt + 4g + i of token r16
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    if (!active[hh] || !tok_ok) continue;
    const int hq = kvh * grp + wave + 4 * hh;
    const long base = ((long)hq * a.B + r16) * a.n_split + sp;
    float *po = a.part_o + base * HD;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) po[16 * dt + 4 * g + i] = o[hh][dt][i];
    if (g == 0) {
      a.part_ml[base * 2] = m_run[hh];
      a.part_ml[base * 2 + 1] = l_run[hh];
    }
  }
}

// O[t][h*hd + d] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// One workgroup per (query head, token): thread (p, q) owns dims 4q..4q+3 and
// the splits s = p, p + P, ... (P = 256 / (HD/4)); the P partial sums are then
// added in p order through LDS, so the result is bitwise reproducible.
constexpr int kMaxSplit = 1024;

template <typename TA, int HD>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  constexpr int NQ = HD / 4, P = 256 / NQ;
  __shared__ float wsp[kMaxSplit];
  __shared__ float red[8];
  __shared__ float4 part[P][NQ];
  const int ht = blockIdx.x;  // hq * B + t
  const int hq = ht / a.B, t = ht - hq * a.B;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ns = a.n_split;
  const float *ml = a.part_ml + (long)ht * ns * 2;
  float mx = -__builtin_inff();
  for (int s = tid; s < ns; s += 256) mx = fmaxf(mx, ml[2 * s]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, shfl_xor(mx, o));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float lsum = 0.f;
  for (int s = tid; s < ns; s += 256) {
    const float m = ml[2 * s];
    const float w = m == -__builtin_inff() ? 0.f : exp2f(m - M);
    wsp[s] = w;
    lsum += w * ml[2 * s + 1];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) lsum += shfl_xor(lsum, o);
  __syncthreads();
  if (lane == 0) red[4 + wave] = lsum;
  __syncthreads();
  const float L = (red[4] + red[5]) + (red[6] + red[7]);
  const int q = tid % NQ, p = tid / NQ;
  const float *po = a.part_o + (long)ht * ns * HD + 4 * q;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  int s = p;
  for (; s + 3 * P < ns; s += 4 * P) {
    float4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = *reinterpret_cast<const float4 *>(po + (long)(s + j * P) * HD);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float w = wsp[s + j * P];
      acc.x += w * v[j].x; acc.y += w * v[j].y; acc.z += w * v[j].z; acc.w += w * v[j].w;
    }
  }
  for (; s < ns; s += P) {
    const float4 v = *reinterpret_cast<const float4 *>(po + (long)s * HD);
    const float w = wsp[s];
    acc.x += w * v.x; acc.y += w * v.y; acc.z += w * v.z; acc.w += w * v.w;
  }
  part[p][q] = acc;
  __syncthreads();
  if (p == 0) {
    float4 r = part[0][q];
#pragma unroll
    for (int j = 1; j < P; ++j) {
      const float4 v = part[j][q];
      r.x += v.x; r.y += v.y; r.z += v.z; r.w += v.w;
    }
    TA *o = reinterpret_cast<TA *>(a.o) + (long)t * a.Hq * HD + (long)hq * HD + 4 * q;
    const float inv = 1.0f / L;
    o[0] = from_f32<TA>(r.x * inv);
    o[1] = from_f32<TA>(r.y * inv);
    o[2] = from_f32<TA>(r.z * inv);
    o[3] = from_f32<TA>(r.w * inv);
  }
}

void attn_plan(long n_keys, int Hkv, int *chunk, int *n_split) {
  const int hk = Hkv > 0 ? Hkv : 1;
  long target = DFL_ATTN_WGS / hk;
  if (target < 1) target = 1;
  long c = (n_keys + target - 1) / target;
  c = ((c + kAttnKT - 1) / kAttnKT) * kAttnKT;
  if (c < kAttnKT) c = kAttnKT;
  long ns = (n_keys + c - 1) / c;
  // the combine kernel holds one weight per split in LDS
  while (ns > kMaxSplit) {
    c += kAttnKT;
    ns = (n_keys + c - 1) / c;
  }
  *chunk = (int)c;
  *n_split = (int)(ns < 1 ? 1 : ns);
}

template <typename TA, int HD>
static void attn_launch_t(const AttnArgs &a, hipStream_t st) {
  if (a.Hq / a.Hkv <= 4)
    hipLaunchKernelGGL((attn_split_kernel<TA, HD, 1>), dim3(a.n_split, a.Hkv), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((attn_split_kernel<TA, HD, 2>), dim3(a.n_split, a.Hkv), dim3(256), 0, st, a);
  hipLaunchKernelGGL((attn_combine_kernel<TA, HD>), dim3(a.Hq * a.B), dim3(256), 0, st, a);
}

hipError_t launch_attention(int act, const AttnArgs &a, hipStream_t st) {
  if (act == ACT_F32) {
    if (a.hd == 64) attn_launch_t<float, 64>(a, st);
    else attn_launch_t<float, 128>(a, st);
  } else {
    if (a.hd == 64) attn_launch_t<bf16, 64>(a, st);
    else attn_launch_t<bf16, 128>(a, st);
  }
  return hipGetLastError();
}

}  // namespace dfl
