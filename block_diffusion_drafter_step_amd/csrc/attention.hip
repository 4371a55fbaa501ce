// Non-causal block attention over [injected context | block] ("Turbo dflash",
// Overview and The Problem; the block's positions all see each other and
// the whole injected cache).
//
// The work is HBM-bound: every context K/V row is read once and used by all
// query heads of its GQA group (Hq/Hkv heads x B block tokens).  V is cached
// in transposed panels of 32 positions ([Hkv][capacity/32][hd][32]), so the
// K tile (32 keys x dims) and the V^T tile (dims x 32 keys) of a tile are
// each one contiguous run of memory.  A workgroup
// owns one KV head and one contiguous chunk of context keys (split-K over the
// context, "flash-decoding"); 32-key K and V^T tiles stream through a 4-stage
// LDS ring filled by direct-to-LDS loads, and each of its 4 waves runs one
// query head of the group (two for 8-head groups) against every tile:
//   S^T = K_tile Q_h^T        (keys x tokens, 16x16x32 MFMA)
//   online softmax per token   (fp32, base-2 exponent, running max / sum)
//   O^T += V^T_tile P^T        (dims x tokens)
// The keys of the two 16-key S^T tiles are interleaved (tile st, row m holds
// key 8(m/4) + 4st + m%4), so each lane ends up holding eight consecutive
// keys of one token: exactly the P^T operand whose matching V^T fragment is
// one 16-byte run of a V^T row.  Probabilities never leave registers.  The
// block's own B keys come from the Q | Kb | Vb buffer in the combine kernel,
// which merges the splits and the block with their log-sum-exp weights in a
// fixed order.
#include "common.h"
#include "kernels.h"
#include "stream.h"

namespace dfl {

#ifndef DFL_ATTN_WGS
#define DFL_ATTN_WGS 512
#endif
constexpr int kAttnKT = 32;      // keys per tile (one ring stage)
#ifndef DFL_ATTN_STAGES
#define DFL_ATTN_STAGES 3
#endif
constexpr int kAttnStages = DFL_ATTN_STAGES;
constexpr float kLog2e = 1.4426950408889634f;
// Lazy softmax reference: a column's reference maximum moves only when its
// scores exceed it by more than 2^kLazyMax, so the accumulators are rescaled
// about once per split and the unnormalised weights stay <= 2^kLazyMax.  The
// reference starts at a finite floor (not -inf), so masked scores (-inf) give
// weight exp2(-inf) = 0 with no special case.
constexpr float kLazyMax = 8.f;
constexpr float kRefFloor = -1e30f;
// 2^x by the hardware instruction (v_exp_f32): the weights are rounded to the
// act type right after, and exp2(-inf) = 0
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __attribute__((address_space(3))) void attn_lds_void;

template <typename TA, int HD>
struct AttnCfg {
  static constexpr int ES = (int)sizeof(TA);
  static constexpr int EPC = 16 / ES;                 // elements per 16-byte chunk
  static constexpr int RK = HD * ES;                  // K tile row (one key), bytes
  static constexpr int RV = kAttnKT * ES;             // V^T tile row (one dim), bytes
  static constexpr int NKC = RK / 16, NVC = RV / 16;  // chunks per row
  static constexpr int KBYTES = kAttnKT * RK;
  static constexpr int STAGE = KBYTES + HD * RV;      // 2 * KT * HD * ES
  static constexpr int NKI = KBYTES / 1024;           // 1 KB direct-to-LDS loads per stage
  static constexpr int NI = STAGE / 1024;
  static constexpr int NPW = NI / 4;                  // ... per wave
  static constexpr int NQF = HD / 32;                 // Q fragments (k-steps over dims)
  static constexpr int NDT = HD / 16;                 // 16-dim output tiles
  static_assert(NI % 4 == 0, "stage must split evenly over 4 waves");
};

// LDS chunk slots.  K rows: the chunk XOR folds key-row bits 0-1 and 3-4,
// which are distinct over the 16 (interleaved) keys of one S^T tile; V^T
// rows: XOR with dim-row bits 1-2 (or 1-3).  Both were measured free of bank
// conflicts for ds_read_b128 on gfx950; any XOR keeps each row a permutation.
template <int NKC>
__device__ __forceinline__ int kswz(int row, int c) {
  return c ^ (((((row >> 3) & 3) << 2) | (row & 3)) & (NKC - 1));
}
template <int NVC>
__device__ __forceinline__ int vswz(int row, int c) {
  return c ^ ((row >> 1) & (NVC - 1));
}

// one direct-to-LDS 16-byte load per lane (lane i lands at byte 16 i)
__device__ __forceinline__ void attn_dma16(const void *g, attn_lds_void *l) {
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
}

template <int N>
__device__ __forceinline__ void attn_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// wait for this wave's LDS reads, then s_barrier; no workgroup fence (that
// would also wait for every direct-to-LDS load still in flight)
__device__ __forceinline__ void attn_ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((0x3F & 0xF) | ((0x3F >> 4) << 14) | (0x7 << 4) | (0x0 << 8));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// the context keys [key0, key1) of KV head kvh that one workgroup owns
struct KeyRange {
  const char *ck, *cv;   // this head's K rows and V^T panels
  const char *sk, *sv;   // Q8_0 caches: this head's K and V scales ([cap][hd/32] fp16)
  long cap;
  long key0, key1;
  int ntile;
};

// ---------------------------------------------------------------------------
// Q8_0 caches (head_dim 128) through the same ring: a stage holds a tile's
// raw codes and scales, 9 KB against 16 KB of bf16,
//   [K codes 32 keys x 128 | V^T codes 128 dims x 32 | K scales 32 x 4 fp16 |
//    V scales 32 x 4 fp16 | 512 spare bytes]
// each wave issuing two 1 KB code loads and one 256-byte scale load (waves
// 2-3 repeat the scales into the spare bytes, so every wave counts the same
// loads).  Once a stage has landed, the workgroup's 256 threads decode it
// into one bf16 tile in the layout (and swizzle) of a bf16 stage, each code
// once, to bf16_rne(fp32(scale) * code); the bf16 tile code then runs on it.
// ---------------------------------------------------------------------------
constexpr int kQ8HD = 128;
constexpr int kQ8Codes = kAttnKT * kQ8HD;        // 4 KB of K codes, 4 KB of V^T codes
constexpr int kQ8Stage = 2 * kQ8Codes + 1024;    // + K scales, V scales, spare
constexpr int kQ8NPW = 3;                        // loads per wave per stage
#ifndef DFL_ATTN_Q8_STAGES
#define DFL_ATTN_Q8_STAGES 3
#endif
constexpr int kQ8Stages = DFL_ATTN_Q8_STAGES;

__device__ __forceinline__ void attn_dma4(const void *g, attn_lds_void *l) {
  __builtin_amdgcn_global_load_lds(g, l, 4, 0, 0);
}

__device__ __forceinline__ void attn_issue_q8(const KeyRange &kr, char *stage, int tI, int wave, int lane) {
  const long t0 = kr.key0 + (long)min(tI, kr.ntile - 1) * kAttnKT;
  // K piece `wave`: keys 8 wave .. + 8 (a tile starts inside the capacity,
  // which is a multiple of 64, so all 32 rows of it lie inside too)
  {
    const int row = 8 * wave + (lane >> 3), c = lane & 7;
    attn_dma16(kr.ck + (t0 + row) * kQ8HD + 16 * c, (attn_lds_void *)(stage + wave * 1024));
  }
  // V^T piece `wave`: dims 32 wave .. + 32 of the tile's panel
  {
    const int d = 32 * wave + (lane >> 1), h = lane & 1;
    const char *panel = kr.cv + (t0 / kAttnKT) * (long)(kQ8HD * kAttnKT);
    attn_dma16(panel + d * kAttnKT + 16 * h, (attn_lds_void *)(stage + kQ8Codes + wave * 1024));
  }
  // scales of the tile's 32 positions: 256 contiguous bytes each
  const char *sc = (wave & 1) ? kr.sv : kr.sk;
  attn_dma4(sc + t0 * (kQ8HD / 32) * 2 + 4 * lane, (attn_lds_void *)(stage + 2 * kQ8Codes + 256 * wave));
}

// eight codes, each with its own scale, to bf16 (exact product, one rounding)
__device__ __forceinline__ Frag<bf16> dq8_each(uint32_t lo, uint32_t hi, const float (&s)[8]) {
  const uint32_t a = lo ^ 0x80808080u, b = hi ^ 0x80808080u;
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w = j < 2 ? a : b;
    const int sh = 16 * (j & 1);
    const dq_f32x2 v = {fmaf((float)((w >> sh) & 0xffu), s[2 * j], -128.f * s[2 * j]),
                        fmaf((float)((w >> (sh + 8)) & 0xffu), s[2 * j + 1], -128.f * s[2 * j + 1])};
    r[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, dq_bf16x2));
  }
  Frag<bf16> f;
  f.v = __builtin_bit_cast(bf16x8, r);
  return f;
}

// the 256 threads of a workgroup decode a landed Q8_0 stage into `dec`, a
// bf16 tile laid out as a bf16 stage of AttnCfg<bf16, 128>
__device__ __forceinline__ void attn_decode_q8(const char *raw, char *dec, int tid) {
  using C = AttnCfg<bf16, kQ8HD>;
  const char *ksc = raw + 2 * kQ8Codes, *vsc = ksc + 256;
  {   // K: key tid / 8, dims 16 c .. + 16 under the scale of block c / 2
    const int key = tid >> 3, c = tid & 7;
    const uint4 q = *reinterpret_cast<const uint4 *>(raw + key * kQ8HD + 16 * c);
    const float sc = half_bits_to_f32(*reinterpret_cast<const uint16_t *>(ksc + key * 8 + 2 * (c >> 1)));
    char *row = dec + key * C::RK;
    *reinterpret_cast<Frag<bf16> *>(row + 16 * kswz<C::NKC>(key, 2 * c)) = dq8(q.x, q.y, sc);
    *reinterpret_cast<Frag<bf16> *>(row + 16 * kswz<C::NKC>(key, 2 * c + 1)) = dq8(q.z, q.w, sc);
  }
  {   // V^T: dim tid / 2, keys 16 h .. + 16, each under its own key's scale of block d / 32
    const int d = tid >> 1, h = tid & 1;
    const uint4 q = *reinterpret_cast<const uint4 *>(raw + kQ8Codes + d * kAttnKT + 16 * h);
    const char *vs = vsc + (16 * h) * 8 + 2 * (d >> 5);
    float s0[8], s1[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s0[e] = half_bits_to_f32(*reinterpret_cast<const uint16_t *>(vs + 8 * e));
      s1[e] = half_bits_to_f32(*reinterpret_cast<const uint16_t *>(vs + 8 * (8 + e)));
    }
    char *row = dec + C::KBYTES + d * C::RV;
    *reinterpret_cast<Frag<bf16> *>(row + 16 * vswz<C::NVC>(d, 2 * h)) = dq8_each(q.x, q.y, s0);
    *reinterpret_cast<Frag<bf16> *>(row + 16 * vswz<C::NVC>(d, 2 * h + 1)) = dq8_each(q.z, q.w, s1);
  }
}

// Issue tile tI (clamped to the last) into `stage`: this wave's NPW of the
// stage's 1 KB loads.  K rows past the chunk re-read its last key (they only
// feed masked scores); a tile starts on a panel boundary, so its V^T is the
// whole panel, which lies inside the capacity.
template <typename TA, int HD>
__device__ __forceinline__ void attn_issue(const KeyRange &kr, char *stage, int tI, int wave,
                                           int lane) {
  using C = AttnCfg<TA, HD>;
  const long t0 = kr.key0 + (long)min(tI, kr.ntile - 1) * kAttnKT;
#pragma unroll
  for (int j = 0; j < C::NPW; ++j) {
    const int q = wave + 4 * j;   // 1 KB piece of the stage
    if (q < C::NKI) {
      constexpr int RPI = 1024 / C::RK;   // key rows per piece
      const int row = q * RPI + lane / C::NKC, slot = lane % C::NKC;
      const long key = min(t0 + row, kr.key1 - 1);
      attn_dma16(kr.ck + key * C::RK + 16 * kswz<C::NKC>(row, slot),
                 (attn_lds_void *)(stage + q * 1024));
    } else {
      constexpr int RPI = 1024 / C::RV;   // dim rows per piece
      const int qv = q - C::NKI;
      const int d = qv * RPI + lane / C::NVC, slot = lane % C::NVC;
      const char *panel = kr.cv + (t0 / kAttnKT) * (long)(HD * C::RV);
      attn_dma16(panel + d * C::RV + 16 * vswz<C::NVC>(d, slot), (attn_lds_void *)(stage + q * 1024));
    }
  }
}

// an 8-element MFMA fragment of an LDS row from its (swizzled) 16-byte chunks
template <typename TA>
__device__ __forceinline__ Frag<TA> lds_frag2(const char *row, int c0, int c1);
template <>
__device__ __forceinline__ Frag<bf16> lds_frag2<bf16>(const char *row, int c0, int) {
  return *reinterpret_cast<const Frag<bf16> *>(row + 16 * c0);
}
template <>
__device__ __forceinline__ Frag<float> lds_frag2<float>(const char *row, int c0, int c1) {
  Frag<float> f;
  const f32x4 a = *reinterpret_cast<const f32x4 *>(row + 16 * c0);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(row + 16 * c1);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f.v[i] = a[i];
    f.v[4 + i] = b[i];
  }
  return f;
}

// one tile from an LDS stage into this wave's running softmax and output
template <typename TA, int HD, int HPW>
__device__ __forceinline__ void attn_tile(const char *stage, long t0, long key1, float sl2, int g,
                                          int r16, const Frag<TA> (&qf)[HPW][AttnCfg<TA, HD>::NQF],
                                          f32x4 (&o)[HPW][AttnCfg<TA, HD>::NDT], float (&m_run)[HPW],
                                          float (&l_run)[HPW], const bool (&active)[HPW]) {
  using C = AttnCfg<TA, HD>;
  constexpr int CPF = 8 / C::EPC;   // chunks per fragment (1 bf16, 2 fp32)
  // K fragments of both S^T tiles (row m of tile st = key 8(m/4) + 4st + m%4)
  Frag<TA> kf[2][C::NQF];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const int row = 8 * (r16 >> 2) + 4 * st + (r16 & 3);
    const char *kr = stage + row * C::RK;
#pragma unroll
    for (int f = 0; f < C::NQF; ++f) {
      const int c = (32 * f + 8 * g) / C::EPC;
      kf[st][f] = lds_frag2<TA>(kr, kswz<C::NKC>(row, c), kswz<C::NKC>(row, c + CPF - 1));
    }
  }
  // V^T fragments: dims 16 dt + r16, keys 8g .. 8g+7
  Frag<TA> vf[C::NDT];
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt) {
    const int d = 16 * dt + r16;
    const char *vr = stage + C::KBYTES + d * C::RV;
    const int c = (8 * g) / C::EPC;
    vf[dt] = lds_frag2<TA>(vr, vswz<C::NVC>(d, c), vswz<C::NVC>(d, c + CPF - 1));
  }
  // keys of this tile inside the range (wave-uniform, 32 but for the last)
  const int lim = (int)min(key1 - t0, (long)kAttnKT);
  // a tile that ends inside its V^T panel: the panel's positions from key1 on
  // may hold anything (a NaN would survive its zero probability), so their
  // values are replaced by zeros; element e of a fragment is key 8g + e
  if (lim < kAttnKT) {
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (8 * g + e >= lim) vf[dt].v[e] = from_f32<TA>(0.f);
  }
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    if (!active[hh]) continue;
    f32x4 s[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      s[st] = zero4();
#pragma unroll
      for (int f = 0; f < C::NQF; ++f) mma(s[st], kf[st][f], qf[hh][f]);
    }
    // lane: token r16, keys 8g + 4st + i
    float p[8];
    float mx = -__builtin_inff();
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = 8 * g + 4 * st + i < lim ? s[st][i] * sl2 : -__builtin_inff();
        p[st * 4 + i] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    // lazy reference maximum (a wave-uniform branch, rare after the first tile)
    const bool up = mx > m_run[hh] + kLazyMax;
    if (__builtin_amdgcn_ballot_w64(up)) {
      const float alpha = up ? hw_exp2(m_run[hh] - mx) : 1.f;
      if (up) m_run[hh] = mx;
      l_run[hh] *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt) o[hh][dt] *= alpha;
    }
    // the row sum uses the weights exactly as the P.V product sees them
    float ls = 0.f;
    Frag<TA> pf;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pf.v[e] = from_f32<TA>(hw_exp2(p[e] - m_run[hh]));
      ls += to_f32(pf.v[e]);
    }
    ls += shfl_xor(ls, 16);
    ls += shfl_xor(ls, 32);
    l_run[hh] += ls;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) mma(o[hh][dt], vf[dt], pf);
  }
}

#ifndef DFL_ATTN_STREAMS
#define DFL_ATTN_STREAMS 2   // key streams per split workgroup (1 or 2)
#endif
#ifndef DFL_ATTN_OCC
#define DFL_ATTN_OCC 2   // workgroups per CU the split kernel's registers are sized for
#endif

// NS key streams per workgroup: waves 4 s .. 4 s + 3 walk the s-th contiguous
// part of the workgroup's keys through their own ring, and the streams'
// running softmax states are merged in LDS at the end, so one workgroup
// writes one partial per query row for NS parts of the context.
// KQ8: the cache holds Q8_0 codes and scales (bf16 activations, head_dim
// 128, one stream): the ring carries raw stages and each landed stage is
// decoded once into one of two bf16 tiles; tile t+1 is decoded in the same
// barrier interval in which tile t is multiplied (one barrier per tile).
template <typename TA, int HD, int HPW, int NS, bool KQ8 = false>
__global__ __launch_bounds__(256 * NS, (NS == 1 ? DFL_ATTN_OCC : 1)) void attn_split_kernel(AttnArgs a) {
  using C = AttnCfg<TA, HD>;
  static_assert(!KQ8 || (HD == kQ8HD && sizeof(TA) == 2), "Q8_0: bf16, head_dim 128");
  constexpr int STG = KQ8 ? kQ8Stage : C::STAGE;   // bytes of one ring stage
  constexpr int NPW = KQ8 ? kQ8NPW : C::NPW;       // loads per wave per stage
  constexpr int S = KQ8 ? kQ8Stages : kAttnStages; // ring stages
  extern __shared__ __attribute__((aligned(1024))) char attn_smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int stream = wave_all >> 2, wave = wave_all & 3;
  const int g = lane >> 4, r16 = lane & 15;
  const int kvh = blockIdx.y, sp = blockIdx.x;
  const int grp = a.Hq / a.Hkv;
  KeyRange kr;
  if constexpr (KQ8) {   // one byte per code, four fp16 scales per position
    kr.ck = reinterpret_cast<const char *>(a.ck) + (long)kvh * a.cap * HD;
    kr.cv = reinterpret_cast<const char *>(a.cv) + (long)kvh * a.cap * HD;
    kr.sk = reinterpret_cast<const char *>(a.cks) + (long)kvh * a.cap * (HD / 32) * 2;
    kr.sv = reinterpret_cast<const char *>(a.cvs) + (long)kvh * a.cap * (HD / 32) * 2;
  } else {
    kr.ck = reinterpret_cast<const char *>(a.ck) + (long)kvh * a.cap * C::RK;
    kr.cv = reinterpret_cast<const char *>(a.cv) + (long)kvh * a.cap * HD * C::ES;   // cap/32 panels
    kr.sk = kr.sv = nullptr;
  }
  kr.cap = a.cap;
  // the workgroup's keys [w0, w1) in NS parts of whole tiles
  const long w0 = (long)sp * a.chunk, w1 = min(a.n_ctx, w0 + a.chunk);
  const long part = ((a.chunk / NS + kAttnKT - 1) / kAttnKT) * kAttnKT;
  kr.key0 = min(w1, w0 + stream * part);
  kr.key1 = min(w1, kr.key0 + part);
  kr.ntile = (int)((kr.key1 - kr.key0 + kAttnKT - 1) / kAttnKT);
  // every stream runs the first stream's tile count (the barriers are the
  // workgroup's); past its own tiles a stream re-reads its last tile and
  // skips the arithmetic, and a stream without keys loads nothing
  const int nloop = (int)((min(w1, w0 + part) - w0 + kAttnKT - 1) / kAttnKT);
  const bool loads = kr.ntile > 0;
  char *ring = attn_smem + stream * (S * STG);
  // KQ8: this stream's two decoded bf16 tiles
  char *dec = attn_smem + NS * S * STG + stream * 2 * AttnCfg<bf16, kQ8HD>::STAGE;
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
    m_run[hh] = kRefFloor;
    l_run[hh] = 0.f;
  }

  // ring: tile t is read from stage t % S; stages t+1 .. t+S-2 are in flight
  auto issue = [&](int t) {
    if constexpr (KQ8) attn_issue_q8(kr, ring + (t % S) * STG, t, wave, lane);
    else attn_issue<TA, HD>(kr, ring + (t % S) * STG, t, wave, lane);
  };
  if constexpr (KQ8) {
    // Tiles 0 .. S-1 fill every stage; at the top of iteration t tiles up
    // to t+S-1 are issued, tile t+1 has landed after the barrier, whose
    // other side also orders iteration t-1 (reads of decoded tile t-1,
    // decode of tile t) before this one.  Stage t % S was decoded in
    // iteration t-1, so tile t+S refills it.  The stream's 256 threads
    // decode; past its own tiles a stream only keeps the barriers.
    constexpr int DB = AttnCfg<bf16, kQ8HD>::STAGE;
    const int stid = tid & 255;
    if (loads) {
#pragma unroll
      for (int s = 0; s < S; ++s) issue(s);
    }
    attn_wait_vm<NPW * (S - 1)>();   // tile 0 has landed
    attn_ring_barrier();
    if (loads) attn_decode_q8(ring, dec, stid);
    for (int tI = 0; tI < nloop; ++tI) {
      attn_wait_vm<NPW * (S - 2)>();   // this wave's loads of tile tI+1 have landed
      attn_ring_barrier();             // ... everyone's; decoded tile tI is complete
      if (loads) issue(tI + S);
      if (tI < kr.ntile)
        attn_tile<TA, HD, HPW>(dec + (tI & 1) * DB, kr.key0 + (long)tI * kAttnKT, kr.key1, sl2, g, r16, qf,
                               o, m_run, l_run, active);
      if (tI + 1 < kr.ntile) attn_decode_q8(ring + ((tI + 1) % S) * STG, dec + ((tI + 1) & 1) * DB, stid);
    }
  } else {
    if (loads) {
#pragma unroll
      for (int s = 0; s < S - 1; ++s) issue(s);
    }
    for (int tI = 0; tI < nloop; ++tI) {
      attn_wait_vm<NPW * (S - 2)>();   // this wave's loads of tile tI have landed
      attn_ring_barrier();             // ... everyone's; tile tI-1 is no longer read
      if (loads) issue(tI + S - 1);
      if (tI < kr.ntile)
        attn_tile<TA, HD, HPW>(ring + (tI % S) * STG, kr.key0 + (long)tI * kAttnKT, kr.key1, sl2, g, r16,
                               qf, o, m_run, l_run, active);
    }
  }
  attn_wait_vm<0>();

  if constexpr (NS > 1) {
    // streams 1.. hand their (o, m, l) to stream 0 through the (now idle)
    // ring memory; stream 0 merges them in stream order
    static_assert(NS == 2, "two streams");
    static_assert((4 * HPW * C::NDT * 4 * 64 + 4 * HPW * 64 * 2) * 4 <= NS * kAttnStages * C::STAGE,
                  "the merge area fits the rings' LDS");
    float *xo = reinterpret_cast<float *>(attn_smem);
    float *xm = xo + 4 * HPW * C::NDT * 4 * 64;
    __syncthreads();   // every wave is done reading the rings
    if (stream == 1) {
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        const int base = (wave * HPW + hh) * 64 + lane;
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) xo[((base * C::NDT + dt) << 2) + i] = o[hh][dt][i];
        xm[2 * base] = m_run[hh];
        xm[2 * base + 1] = l_run[hh];
      }
    }
    __syncthreads();
    if (stream == 1) return;
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const int base = (wave * HPW + hh) * 64 + lane;
      const float m1 = xm[2 * base], l1 = xm[2 * base + 1];
      const float m = fmaxf(m_run[hh], m1);
      if (m == -__builtin_inff()) continue;   // neither stream saw a key
      const float a0 = exp2f(m_run[hh] - m), a1 = exp2f(m1 - m);
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o[hh][dt][i] = o[hh][dt][i] * a0 + xo[((base * C::NDT + dt) << 2) + i] * a1;
      l_run[hh] = l_run[hh] * a0 + l1 * a1;
      m_run[hh] = m;
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

// O[t][h*hd + d] = (sum_s 2^(m_s - M) O_s + 2^(m_b - M) O_b) /
//                  (sum_s 2^(m_s - M) l_s + 2^(m_b - M) l_b),
// where (m_b, l_b, O_b) is the block's own B keys, scored here from Q, Kb, Vb
// (probabilities rounded to the act type as the split kernel rounds them).
// One wave per (query head, token), no barriers: lane l owns dims
// DPL*l .. DPL*l+DPL-1 (DPL = HD/64) and split l of every group of SG (32 or
// 64) splits; every load of the first SG splits and of the block is issued
// before the first use.  Weights reach all lanes by readlane; splits are added in
// increasing order and the block term last, so the result is bitwise
// reproducible.
constexpr int kMaxSplit = 1024;

template <typename TA, int HD, int SG>
__global__ __launch_bounds__(64) void attn_combine_kernel(AttnArgs a) {
  constexpr int DPL = HD / 64;
  const int ht = blockIdx.x;  // hq * B + t
  const int hq = ht / a.B, t = ht - hq * a.B;
  const int kvh = hq / (a.Hq / a.Hkv);
  const int lane = threadIdx.x;
  const int ns = a.n_split;
  const long qld = (long)(a.Hq + 2 * a.Hkv) * HD;
  const TA *qkv = reinterpret_cast<const TA *>(a.qkv);
  const float *po = a.part_o + (long)ht * ns * HD + DPL * lane;
  const float *ml = a.part_ml + (long)ht * ns * 2;

  // loads: partial rows 0..63, (m, l) of split `lane`, Q, Kb[0..15], Vb[0..15]
  float ov[SG][DPL];
  float2 mlv = make_float2(-__builtin_inff(), 0.f);
  if (ns > 0) {
#pragma unroll
    for (int s = 0; s < SG; ++s)
#pragma unroll
      for (int e = 0; e < DPL; ++e) ov[s][e] = po[(long)min(s, ns - 1) * HD + e];
    if (lane < ns && lane < SG) mlv = *reinterpret_cast<const float2 *>(ml + 2 * lane);
  }
  float qv[DPL], kv[16][DPL], vv[16][DPL];
  {
    const TA *qr = qkv + (long)t * qld + (long)hq * HD + DPL * lane;
#pragma unroll
    for (int e = 0; e < DPL; ++e) qv[e] = to_f32(qr[e]);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const TA *row = qkv + (long)min(j, a.B - 1) * qld + DPL * lane;
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        kv[j][e] = to_f32(row[(long)(a.Hq + kvh) * HD + e]);
        vv[j][e] = to_f32(row[(long)(a.Hq + a.Hkv + kvh) * HD + e]);
      }
    }
  }

  // block scores s_j = Q[t] . Kb[j] * scale (base 2), on every lane
  float sb[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    float x = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) x += qv[e] * kv[j][e];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += shfl_xor(x, o);
    sb[j] = x * a.scale * kLog2e;
  }
  float mb = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (j < a.B) mb = fmaxf(mb, sb[j]);
  float lb = 0.f, pb[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    pb[j] = j < a.B ? to_f32(from_f32<TA>(exp2f(sb[j] - mb))) : 0.f;
    lb += pb[j];
  }

  // the global maximum over every split and the block
  float mx = mlv.x;
  for (int s = lane + SG; s < ns; s += SG)
    if (lane < SG) mx = fmaxf(mx, ml[2 * s]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, shfl_xor(mx, o));
  const float M = fmaxf(mx, mb);

  // weighted sums over the splits, SG at a time
  float acc[DPL], lsum = 0.f;
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
  for (int s0 = 0; s0 < ns; s0 += SG) {
    float2 m_l = mlv;
    if (s0 > 0) {
      m_l = make_float2(-__builtin_inff(), 0.f);
      if (lane < SG && s0 + lane < ns) m_l = *reinterpret_cast<const float2 *>(ml + 2 * (s0 + lane));
#pragma unroll
      for (int s = 0; s < SG; ++s)
#pragma unroll
        for (int e = 0; e < DPL; ++e) ov[s][e] = po[(long)min(s0 + s, ns - 1) * HD + e];
    }
    const float w = m_l.x == -__builtin_inff() ? 0.f : exp2f(m_l.x - M);   // zero past ns
    float lw = w * m_l.y;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) lw += shfl_xor(lw, o);
    lsum += lw;
#pragma unroll
    for (int s = 0; s < SG; ++s) {
      const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), s));
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] += ws * ov[s][e];
    }
  }

  // the block's keys: O_b = sum_j p_j Vb[j], added last
  const float wb = exp2f(mb - M);
  const float L = lsum + wb * lb;
  float ob[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    ob[e] = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) ob[e] += pb[j] * vv[j][e];
  }
  TA *o = reinterpret_cast<TA *>(a.o) + (long)t * a.Hq * HD + (long)hq * HD + DPL * lane;
  const float inv = 1.0f / L;
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = from_f32<TA>((acc[e] + wb * ob[e]) * inv);
}

// the cached context keys are split over about DFL_ATTN_WGS workgroups in
// chunks of whole tiles; no context, no splits
void attn_plan(long n_keys, int Hkv, int streams, int *chunk, int *n_split) {
  if (n_keys <= 0) {
    *chunk = kAttnKT;
    *n_split = 0;
    return;
  }
  const int hk = Hkv > 0 ? Hkv : 1;
  long target = DFL_ATTN_WGS / (streams > 1 ? streams : 1) / hk;
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
  *n_split = (int)ns;
}

// an upper bound on attn_plan's split count that never decreases with
// n_keys (attn_plan's own count can: a longer context may round to longer
// chunks), so a workspace sized for a maximum context fits every shorter one
int attn_max_splits(long n_keys, int Hkv) {
  if (n_keys <= 0) return 0;
  const int hk = Hkv > 0 ? Hkv : 1;
  long target = DFL_ATTN_WGS / hk;
  if (target < 1) target = 1;
  const long tiles = (n_keys + kAttnKT - 1) / kAttnKT;
  long b = tiles < target ? tiles : target;
  return (int)(b < kMaxSplit ? b : kMaxSplit);
}

template <typename TA, int HD, int HPW, int NS>
static hipError_t attn_split_go(const AttnArgs &a, hipStream_t st) {
  const size_t lds = (size_t)NS * kAttnStages * AttnCfg<TA, HD>::STAGE;
  auto *k = &attn_split_kernel<TA, HD, HPW, NS>;
  const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void *>(k), lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3(a.n_split, a.Hkv), dim3(256 * NS), lds, st, a);
  return hipSuccess;
}

// Q8_0 cache through the ring: raw stages plus the decoded bf16 tile
#ifndef DFL_ATTN_Q8_STREAMS
#define DFL_ATTN_Q8_STREAMS 2   // key streams per workgroup of the Q8_0-cache kernel (1 or 2)
#endif
template <int HPW>
static hipError_t attn_split_q8_go(const AttnArgs &a, hipStream_t st) {
  constexpr int NS = DFL_ATTN_Q8_STREAMS;
  const size_t lds = (size_t)NS * (kQ8Stages * kQ8Stage + 2 * AttnCfg<bf16, kQ8HD>::STAGE);
  auto *k = &attn_split_kernel<bf16, kQ8HD, HPW, NS, true>;
  const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void *>(k), lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3(a.n_split, a.Hkv), dim3(256 * NS), lds, st, a);
  return hipSuccess;
}

// key streams per split workgroup: two when both rings fit the LDS (and the
// merge area, 4 HPW waves' (o, m, l), fits one of them)
template <typename TA, int HD>
constexpr int attn_streams_t() {
  return DFL_ATTN_STREAMS >= 2 && 2 * kAttnStages * AttnCfg<TA, HD>::STAGE <= 160 * 1024 ? 2 : 1;
}
int attn_streams(int act, int hd) {
  if (act == ACT_F32) return hd == 64 ? attn_streams_t<float, 64>() : attn_streams_t<float, 128>();
  return hd == 64 ? attn_streams_t<bf16, 64>() : attn_streams_t<bf16, 128>();
}

bool attn_q8_ok(int hd, int grp, int B) {
  (void)B;
  return hd == kQ8HD && grp <= 8;
}

void attn_plan_call(int act, int hd, int grp, int B, int kvq, long n_keys, int Hkv, int *chunk, int *n_split) {
  (void)grp;
  (void)B;
  // Q8_0 caches: DFL_ATTN_Q8_STREAMS streams per workgroup
  attn_plan(n_keys, Hkv, kvq ? DFL_ATTN_Q8_STREAMS : attn_streams(act, hd), chunk, n_split);
}

template <typename TA, int HD>
static void attn_combine_go(const AttnArgs &a, hipStream_t st) {
  // splits 32 at a time when there are at most 32 (half the loads and broadcasts)
  if (a.n_split <= 32)
    hipLaunchKernelGGL((attn_combine_kernel<TA, HD, 32>), dim3(a.Hq * a.B), dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL((attn_combine_kernel<TA, HD, 64>), dim3(a.Hq * a.B), dim3(64), 0, st, a);
}

template <typename TA, int HD>
static hipError_t attn_launch_t(const AttnArgs &a, hipStream_t st) {
  constexpr int NS = attn_streams_t<TA, HD>();
  if (a.n_split > 0) {
    const hipError_t e = a.Hq / a.Hkv <= 4 ? attn_split_go<TA, HD, 1, NS>(a, st)
                                           : attn_split_go<TA, HD, 2, NS>(a, st);
    if (e != hipSuccess) return e;
  }
  attn_combine_go<TA, HD>(a, st);
  return hipSuccess;
}

hipError_t launch_attention(int act, const AttnArgs &a, hipStream_t st) {
  if (a.kvq) {   // bf16 activations, head_dim 128 (checked by the caller)
    if (a.n_split > 0) {
      const hipError_t e = a.Hq / a.Hkv <= 4 ? attn_split_q8_go<1>(a, st) : attn_split_q8_go<2>(a, st);
      if (e != hipSuccess) return e;
    }
    attn_combine_go<bf16, 128>(a, st);
  } else {
    hipError_t e;
    if (act == ACT_F32) e = a.hd == 64 ? attn_launch_t<float, 64>(a, st) : attn_launch_t<float, 128>(a, st);
    else e = a.hd == 64 ? attn_launch_t<bf16, 64>(a, st) : attn_launch_t<bf16, 128>(a, st);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

}  // namespace dfl
