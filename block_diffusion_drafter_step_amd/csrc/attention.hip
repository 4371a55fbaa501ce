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
// (a select, not a branch: loads stay unconditional)
template <typename TA, int HD>
__device__ __forceinline__ const TA *key_row(const AttnArgs &a, const TA *cache, int kvh, long j,
                                             int col_off) {
  const bool ctx = j < a.n_ctx;
  const long t = ctx ? 0 : j - a.n_ctx;
  const long qld = (long)(a.Hq + 2 * a.Hkv) * HD;
  const TA *c = cache + ((long)kvh * a.cap + (ctx ? j : 0)) * HD;
  const TA *b = reinterpret_cast<const TA *>(a.qkv) + t * qld + col_off + (long)kvh * HD;
  return ctx ? c : b;
}

// Staged tile: K copied as-is, V gathered 4 keys x 8 dims per thread and
// written transposed.  Two LDS stages and two register sets: while the waves
// compute on one stage, the next tile waits in registers and the one after is
// in flight, so two tiles' loads overlap every compute phase.  Loads are
// unconditional (keys past the chunk are clamped to its last key; their
// scores are masked to -inf), which keeps the compiler's waits graded.
template <typename TA, int HD>
struct TileRegs {
  using C = AttnCfg<TA, HD>;
  static constexpr int KCH = kAttnKT * HD / C::VEC;         // 16-byte K chunks per tile
  static constexpr int VITEMS = (kAttnKT / 4) * (HD / 8);    // (4 keys x 8 dims) V items
  static constexpr int KPT = (KCH + 255) / 256, VPT = (VITEMS + 255) / 256;
};

// the keys of one KV head that one split workgroup owns: [key0, key1)
struct KeyRange {
  const AttnArgs *a;
  int kvh, kcol, vcol, ntile;
  long key0, key1;
};

// tile tI (clamped to the last one) of the range into registers
template <typename TA, int HD>
__device__ __forceinline__ void attn_load_tile(const KeyRange &kr, int tid, int tI,
                                               u32x4 (&rk)[TileRegs<TA, HD>::KPT],
                                               Frag<TA> (&rv)[TileRegs<TA, HD>::VPT][4]) {
  using C = AttnCfg<TA, HD>;
  using R = TileRegs<TA, HD>;
  const AttnArgs &a = *kr.a;
  const TA *ck = reinterpret_cast<const TA *>(a.ck);
  const TA *cv = reinterpret_cast<const TA *>(a.cv);
  const long t0 = kr.key0 + (long)min(tI, kr.ntile - 1) * kAttnKT;
#pragma unroll
  for (int j = 0; j < R::KPT; ++j) {
    const int c = min(tid + 256 * j, R::KCH - 1);
    const int row = c / (HD / C::VEC), ch = c % (HD / C::VEC);
    const long key = min(t0 + row, kr.key1 - 1);
    rk[j] = *reinterpret_cast<const u32x4 *>(key_row<TA, HD>(a, ck, kr.kvh, key, kr.kcol) + ch * C::VEC);
  }
#pragma unroll
  for (int j = 0; j < R::VPT; ++j) {
    const int it = min(tid + 256 * j, R::VITEMS - 1);
    const int kq = it / (HD / 8), d8 = it % (HD / 8);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const long key = min(t0 + 4 * kq + u, kr.key1 - 1);
      rv[j][u] = load_frag(key_row<TA, HD>(a, cv, kr.kvh, key, kr.vcol) + d8 * 8);
    }
  }
}

// registers -> one LDS stage (K as-is, V transposed)
template <typename TA, int HD>
__device__ __forceinline__ void attn_store_tile(TA *ks, TA *vt, int tid,
                                                const u32x4 (&rk)[TileRegs<TA, HD>::KPT],
                                                const Frag<TA> (&rv)[TileRegs<TA, HD>::VPT][4]) {
  using C = AttnCfg<TA, HD>;
  using R = TileRegs<TA, HD>;
#pragma unroll
  for (int j = 0; j < R::KPT; ++j) {
    const int c = tid + 256 * j;
    if (c < R::KCH) {
      const int row = c / (HD / C::VEC), ch = c % (HD / C::VEC);
      *reinterpret_cast<u32x4 *>(ks + row * C::KLD + ch * C::VEC) = rk[j];
    }
  }
#pragma unroll
  for (int j = 0; j < R::VPT; ++j) {
    const int it = tid + 256 * j;
    if (it < R::VITEMS) {
      const int kq = it / (HD / 8), d8 = it % (HD / 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        Quad<TA> q4;
#pragma unroll
        for (int u = 0; u < 4; ++u) q4.v[u] = rv[j][u].v[e];
        *reinterpret_cast<Quad<TA> *>(vt + (d8 * 8 + e) * C::VLD + 4 * kq) = q4;
      }
    }
  }
}

// one tile from an LDS stage into this wave's running softmax and output
template <typename TA, int HD, int HPW>
__device__ __forceinline__ void attn_compute_tile(const TA *ks, const TA *vt, long t0, long key1,
                                                  float sl2, int g, int r16,
                                                  const Frag<TA> (&qf)[HPW][AttnCfg<TA, HD>::NQF],
                                                  f32x4 (&o)[HPW][AttnCfg<TA, HD>::NDT],
                                                  float (&m_run)[HPW], float (&l_run)[HPW],
                                                  const bool (&active)[HPW]) {
  using C = AttnCfg<TA, HD>;
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
        const TA *kp = ks + (32 * sb + 16 * st + r16) * C::KLD + 8 * g;
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
        const TA *vp = vt + (16 * dt + r16) * C::VLD + 32 * sb + 4 * g;
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
}

// Staged tiles: two LDS stages and two register sets.  While the waves
// compute on one stage, the next tile waits in registers and the one after is
// in flight, so two tiles' loads overlap every compute phase; one barrier per
// tile.  Loads are unconditional (keys past the chunk are clamped to its last
// key and their scores masked to -inf), which keeps the compiler's waits
// graded instead of draining every load at a branch.
template <typename TA, int HD, int HPW>
__global__ __launch_bounds__(256, 2) void attn_split_kernel(AttnArgs a) {
  using C = AttnCfg<TA, HD>;
  using R = TileRegs<TA, HD>;
  constexpr int KS = kAttnKT * C::KLD, VS = HD * C::VLD;   // stage sizes (elements)
  __shared__ __attribute__((aligned(16))) TA Ks[2 * KS];
  __shared__ __attribute__((aligned(16))) TA Vt[2 * VS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int kvh = blockIdx.y, sp = blockIdx.x;
  const int grp = a.Hq / a.Hkv;
  const long S = a.n_ctx + a.B;
  KeyRange kr;
  kr.a = &a;
  kr.kvh = kvh;
  kr.kcol = a.Hq * HD;
  kr.vcol = (a.Hq + a.Hkv) * HD;
  kr.key0 = (long)sp * a.chunk;
  kr.key1 = min(S, kr.key0 + a.chunk);
  kr.ntile = (int)((kr.key1 - kr.key0 + kAttnKT - 1) / kAttnKT);
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

  // tile n computes from stage n % 2
  // (a native vector type: HIP's uint4 is a struct whose copies defeat
  // register promotion of the two register sets)
  u32x4 k0[R::KPT], k1[R::KPT];
  Frag<TA> v0[R::VPT][4], v1[R::VPT][4];
  const int ntile = kr.ntile;
  attn_load_tile<TA, HD>(kr, tid, 0, k0, v0);
  attn_store_tile<TA, HD>(Ks, Vt, tid, k0, v0);
  attn_load_tile<TA, HD>(kr, tid, 1, k1, v1);
  attn_load_tile<TA, HD>(kr, tid, 2, k0, v0);
  __syncthreads();
  for (int tI = 0; tI < ntile; tI += 2) {
    attn_compute_tile<TA, HD, HPW>(Ks, Vt, kr.key0 + (long)tI * kAttnKT, kr.key1, sl2, g, r16, qf, o,
                                   m_run, l_run, active);
    attn_store_tile<TA, HD>(Ks + KS, Vt + VS, tid, k1, v1);   // tile tI + 1
    attn_load_tile<TA, HD>(kr, tid, tI + 3, k1, v1);
    __syncthreads();
    if (tI + 1 < ntile) {
      attn_compute_tile<TA, HD, HPW>(Ks + KS, Vt + VS, kr.key0 + (long)(tI + 1) * kAttnKT, kr.key1,
                                     sl2, g, r16, qf, o, m_run, l_run, active);
      attn_store_tile<TA, HD>(Ks, Vt, tid, k0, v0);           // tile tI + 2
      attn_load_tile<TA, HD>(kr, tid, tI + 4, k0, v0);
      __syncthreads();
    }
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
