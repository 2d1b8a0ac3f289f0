// Fused decode attention over the packed 2/4-bit cache.
//
// [paper] "OmniKVQuant: KV Cache Quantization for Omni-LLMs", §1 and Fig. 1(d):
// the query is rotated once per head instead of inverse-rotating every cached
// key, the online softmax follows FlashAttention's order, value accumulators
// stay in the rotated space of each modality, and the inverse value rotations
// are batched across head outputs; no dense FP16 cache is built ([abstract]).
//
// Split-KV: kernel 1 (decode_partial) gives every (sequence, KV head, split of
// consecutive windows) one 64-lane wave and writes (running max, sum, three
// per-modality accumulators in rotated space); kernel 2 (decode_combine) merges
// the splits with the log-sum-exp rule and applies sum_m U_m A_m once per head.
//
// Per 32-token window the wave issues two matrix-core contractions
// (v_mfma_f32_16x16x32_f16):
//   scores^T [32 tok x 16 col] = codes [32 x d] . Qt [d x 16]
//   acc_m^T  [d x 16 col]     += levels^T [d x 32 tok] . Pt [32 x 16]
// The 16 columns are the G <= 8 query heads of the KV head, twice: columns
// 0..7 carry the fp16 "hi" part and 8..15 the "lo" remainder of the fp32
// operand, so each product keeps ~22 significant bits and the two halves add
// up after the contraction (one DPP row rotate).
//   Key codes enter as fp16 subnormals: masking a stored word leaves
//   code * 2^(bits*p - 24) in each half, exact in fp16 and exact in the f32
//   accumulation; the per-K-step power of two is folded into Qt.
//   Score algebra: score_log2 = Z_h * (q^.m_w + 2^24 * C) with
//   q^ = log2(e) * scale * R q / Z_h (|q^| <= 1, Z_h a power of two),
//   C = sum_c code_c * 2^-24 * (q^_c s_c); the q^.m_w term comes from one extra
//   contraction per 16 windows with k_min as the operand.
//   Value levels come from a per-context table of fp16 level pairs indexed by
//   two packed codes (LDS, conflict-free for 2-bit).
#include <math.h>

#include "omnikv_internal.h"

namespace omnikv {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t uint4_t __attribute__((ext_vector_type(4)));

constexpr float kLazyRescale = 8.0f;  // rescale the accumulators only when the max grows by > 2^8

__device__ __forceinline__ float f16_value(uint16_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

__device__ __forceinline__ float4_t mfma16(uint4_t a, uint4_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
}

// value of lane (l ^ 8) within each row of 16 lanes (DPP row_ror:8)
__device__ __forceinline__ float row_ror8(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false));
}

// Cross-half lane swaps.  Written in asm: the compiler's combine of the
// permlane{16,32}_swap builtins can replace the second result by the first
// (as if the operand were the same in every lane), which drops the lanes the
// swap brings in.  Each asm swaps two registers in place and touches no memory.
// The s_nop pairs give the wait states a VALU write needs before a permlane
// reads the register, and a permlane result before the next VALU reads it
// (the hazard recognizer does not look inside asm).
//   swap32(a, b): lanes 32..63 of a <-> lanes 0..31 of b
//   swap16(a, b): odd 16-lane rows of a <-> even rows of b
__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}

// reduce over the four 16-lane groups holding the same column (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float group_max(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap32(a, b);  // a = lower half in both halves, b = upper half in both halves
  x = fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
  a = __builtin_bit_cast(uint32_t, x);
  b = a;
  swap16(a, b);
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float group_sum(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap32(a, b);
  x = __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
  a = __builtin_bit_cast(uint32_t, x);
  b = a;
  swap16(a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

template <int D>
struct RhtConst;
template <>
struct RhtConst<64> {
  static constexpr float value = 0.125f;
};
template <>
struct RhtConst<128> {
  static constexpr float value = 0.08838834764831845f;
};

// Key operand geometry (window-block layout of include/omnikv.h).
template <int D, int KB>
struct KeyOp {
  static constexpr int words = D * KB / 64;  // per lane
  // effective slot of K-step s after the shift: the operand holds code * 2^(KB*peff - 24)
  __device__ static constexpr int peff(int s) {
    return (D == 128 && KB == 4) ? (s & 1) : s;
  }
  __device__ static constexpr int word(int tau, int s, int i) {
    if (D == 128 && KB == 2) return i;
    if (D == 128 && KB == 4) return 4 * tau + i;
    if (D == 64 && KB == 2) return i & 1;
    return i;
  }
  __device__ static constexpr int shift(int tau, int s, int i) {
    if (D == 128 && KB == 2) return 8 * tau;
    if (D == 128 && KB == 4) return 8 * (s >> 1);
    if (D == 64 && KB == 2) return 8 * (i >> 1) + 4 * tau;
    return 8 * tau;
  }
  __device__ static constexpr uint32_t mask(int s) {
    return (((1u << KB) - 1u) * 0x00010001u) << (KB * peff(s));
  }
};

struct PartialArgs {
  const float* q;
  const int32_t* seq_lens;
  const uint32_t* k_codes;
  const uint16_t* k_min;
  const uint16_t* k_scale;
  const uint32_t* v_codes;
  const uint16_t* v_scale;
  const uint8_t* modality;
  const float* signs;
  const uint32_t* pair_table;
  int hq, hkv, group, modalities;
  int64_t t_cap;
  int64_t max_len;   // host bound of seq_lens; device lengths are clamped to it
  float scale_log2;  // softmax scale * log2(e)
  int wps, splits;
  float2* ws_ml;     // [unit][split][8] (max, sum) in log2 units
  uint32_t* ws_mask; // [unit][split] modalities present
  float* ws_acc;     // [unit][split][M][8][D]
};

template <int M>
__device__ __forceinline__ void acc_mfma(float4_t (&acc)[kMaxModalities][8], const uint4_t (&av)[8],
                                         uint4_t bv, int nu) {
#pragma unroll
  for (int u = 0; u < 8; ++u)
    if (u < nu) acc[M][u] = mfma16(av[u], bv, acc[M][u]);
}

template <int D, int KB, int VB>
__global__ __launch_bounds__(64) void decode_partial_kernel(PartialArgs a) {
  constexpr int NC = D / 64;        // channels per lane in the query rotation
  constexpr int NS = D / 32;        // K-steps of the score contraction
  constexpr int NU = D / 16;        // channel tiles of the value contraction
  constexpr int KW = KeyOp<D, KB>::words;
  constexpr int VW = D * VB / 64;   // value words per lane
  constexpr int PPW = 16 / VB;      // value code pairs per word
  constexpr uint32_t PMASK = (1u << (2 * VB)) - 1u;
  using KO = KeyOp<D, KB>;

  __shared__ float q_lds[kMaxGroup][D];
  __shared__ float a_lds[16][kMaxGroup];
  __shared__ uint32_t vtab[1 << (2 * VB)];

  const int lane = threadIdx.x;
  const int unit = blockIdx.y;                     // b * hkv + kvh
  const int split = blockIdx.x;
  const int b = unit / a.hkv, kvh = unit % a.hkv;
  const int len = static_cast<int>(min<int64_t>(max<int64_t>(a.seq_lens[b], 0), a.max_len));
  const int nwin = (len + kWindow - 1) / kWindow;
  const int wbeg = split * a.wps;
  const int wend = min(nwin, wbeg + a.wps);
  const size_t pidx = static_cast<size_t>(unit) * a.splits + split;
  if (wbeg >= wend) {
    if (lane < kMaxGroup) a.ws_ml[pidx * kMaxGroup + lane] = make_float2(-INFINITY, 0.0f);
    if (lane == 0) a.ws_mask[pidx] = 0u;
    return;
  }
  const int n = lane & 15, g = lane >> 4, h = n & 7, part = n >> 3;
  const bool head_ok = h < a.group;
  const int64_t nwin_cap = a.t_cap / kWindow;

  for (int i = lane; i < (1 << (2 * VB)); i += 64) vtab[i] = a.pair_table[i];

  // ---- query rotation q' = c_d H D q, once per head, scaled to log2 units
  float zmax_mine = 0.0f;
  {
    float sg[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) sg[c] = a.signs[lane + 64 * c];
    for (int hh = 0; hh < kMaxGroup; ++hh) {
      float z[NC];
      const bool ok = hh < a.group;
      const float* qp = a.q + (static_cast<size_t>(b) * a.hq + kvh * a.group + (ok ? hh : 0)) * D;
#pragma unroll
      for (int c = 0; c < NC; ++c) z[c] = ok ? qp[lane + 64 * c] * sg[c] : 0.0f;
#pragma unroll
      for (int st = 1; st < 64; st <<= 1) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const float p = __shfl_xor(z[c], st, 64);
          z[c] = (lane & st) ? (p - z[c]) : (z[c] + p);
        }
      }
      if constexpr (NC == 2) {
        const float x0 = z[0] + z[1], x1 = z[0] - z[1];
        z[0] = x0;
        z[1] = x1;
      }
      float am = 0.0f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        z[c] = z[c] * RhtConst<D>::value * a.scale_log2;
        q_lds[hh][lane + 64 * c] = z[c];
        am = fmaxf(am, fabsf(z[c]));
      }
#pragma unroll
      for (int st = 32; st >= 1; st >>= 1) am = fmaxf(am, __shfl_xor(am, st, 64));
      if (hh == h) zmax_mine = am;
    }
  }
  __syncthreads();
  // Z_h: power of two with |q'/Z_h| <= 1
  int zexp = 0;
  if (zmax_mine > 0.0f) (void)frexpf(zmax_mine, &zexp);
  const float zinv = ldexpf(1.0f, -zexp);
  const float zh = ldexpf(1.0f, zexp);
  const float zfac = ldexpf(1.0f, zexp + 24);

  // ---- per-lane operand constants.  Lane (n, g) feeds column n: head h, part hi/lo.
  // score operand for K-step s, dword i = channels c0, c0+1 with c0 = g*D/4 + 8 s + 2 i
  half2_t alpha[NS][4], beta[NS][4], gamma[NS][4];
  uint4_t bqa[NS];  // q^ hi (part 0) or lo (part 1) for the k_min contraction
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    uint32_t bw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      half2_t al, be, ga, qa;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int c = g * (D / 4) + 8 * s + 2 * i + e;
        const float qh = q_lds[h][c] * zinv;                               // |qh| <= 1
        const float qt = qh * ldexpf(1.0f, -KB * KO::peff(s));              // exact scaling
        const _Float16 th = static_cast<_Float16>(qt);
        const _Float16 tl = static_cast<_Float16>(qt - static_cast<float>(th));
        al[e] = th;
        be[e] = part ? th : static_cast<_Float16>(0.0f);
        ga[e] = part ? tl : static_cast<_Float16>(0.0f);
        const _Float16 hh = static_cast<_Float16>(qh);
        const _Float16 hl = static_cast<_Float16>(qh - static_cast<float>(hh));
        qa[e] = part ? hl : hh;
      }
      alpha[s][i] = al;
      beta[s][i] = be;
      gamma[s][i] = ga;
      bw[i] = __builtin_bit_cast(uint32_t, qa);
    }
    bqa[s] = uint4_t{bw[0], bw[1], bw[2], bw[3]};
  }

  float m_ref = -INFINITY;
  float l_part = 0.0f;
  float4_t acc[kMaxModalities][8];
#pragma unroll
  for (int m = 0; m < kMaxModalities; ++m)
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[m][u] = float4_t{0.f, 0.f, 0.f, 0.f};
  uint32_t seen = 0u;

  const size_t unit_win = static_cast<size_t>(unit) * nwin_cap;
  const uint16_t* vsc = a.v_scale + static_cast<size_t>(unit) * a.t_cap;
  const uint8_t* tags = a.modality + static_cast<size_t>(b) * a.t_cap;

  for (int wb = wbeg; wb < wend; wb += 16) {
    // ---- q^ . m_w for 16 windows: rows = windows, K = channels
    {
      float4_t ca = float4_t{0.f, 0.f, 0.f, 0.f};
      const int wr = wb + n;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        uint4_t am = uint4_t{0u, 0u, 0u, 0u};
        if (wr < wend)
          am = *reinterpret_cast<const uint4_t*>(a.k_min + (unit_win + wr) * D + g * (D / 4) + 8 * s);
        ca = mfma16(am, bqa[s], ca);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = ca[i] + row_ror8(ca[i]);
        if (part == 0) a_lds[4 * g + i][h] = v * zh;
      }
    }
    __syncthreads();
    const int wlast = min(wend, wb + 16);
    for (int w = wb; w < wlast; ++w) {
      const size_t wi = unit_win + w;
      // ---- loads
      uint32_t kw[KW];
      {
        const uint4_t* kp = reinterpret_cast<const uint4_t*>(a.k_codes + wi * (D * KB) + lane * KW);
#pragma unroll
        for (int x = 0; x < KW / 4; ++x) {
          const uint4_t t = kp[x];
          kw[4 * x] = t[0]; kw[4 * x + 1] = t[1]; kw[4 * x + 2] = t[2]; kw[4 * x + 3] = t[3];
        }
        if constexpr (KW == 2) {
          const uint2 t = *reinterpret_cast<const uint2*>(a.k_codes + wi * (D * KB) + lane * KW);
          kw[0] = t.x; kw[1] = t.y;
        }
      }
      uint32_t sw[D / 8];  // k_scale pairs for channels g*D/4 .. g*D/4 + D/4 - 1
      {
        const uint4_t* sp = reinterpret_cast<const uint4_t*>(a.k_scale + wi * D + g * (D / 4));
#pragma unroll
        for (int x = 0; x < D / 32; ++x) {
          const uint4_t t = sp[x];
          sw[4 * x] = t[0]; sw[4 * x + 1] = t[1]; sw[4 * x + 2] = t[2]; sw[4 * x + 3] = t[3];
        }
      }
      uint32_t vw[VW];
      {
        if constexpr (VW >= 4) {
          const uint4_t* vp = reinterpret_cast<const uint4_t*>(a.v_codes + wi * (D * VB) + lane * VW);
#pragma unroll
          for (int x = 0; x < VW / 4; ++x) {
            const uint4_t t = vp[x];
            vw[4 * x] = t[0]; vw[4 * x + 1] = t[1]; vw[4 * x + 2] = t[2]; vw[4 * x + 3] = t[3];
          }
        } else {
          const uint2 t = *reinterpret_cast<const uint2*>(a.v_codes + wi * (D * VB) + lane * VW);
          vw[0] = t.x; vw[1] = t.y;
        }
      }
      const int tokb = w * kWindow;
      uint2 sig2[2];
      uint32_t tg[2];
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        sig2[tau] = *reinterpret_cast<const uint2*>(vsc + tokb + 16 * tau + 4 * g);
        tg[tau] = *reinterpret_cast<const uint32_t*>(tags + tokb + 16 * tau + 4 * g);
      }

      // ---- scores
      float4_t cs[2] = {float4_t{0.f, 0.f, 0.f, 0.f}, float4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        uint32_t bq[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const half2_t sv = __builtin_bit_cast(half2_t, sw[4 * s + i]);
          const half2_t t1 = beta[s][i] * sv;
          const half2_t t2 = __builtin_elementwise_fma(alpha[s][i], sv, -t1);
          bq[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(gamma[s][i], sv, t2));
        }
        const uint4_t bqv = uint4_t{bq[0], bq[1], bq[2], bq[3]};
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
          uint4_t ak;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            ak[i] = (kw[KO::word(tau, s, i)] >> KO::shift(tau, s, i)) & KO::mask(s);
          cs[tau] = mfma16(ak, bqv, cs[tau]);
        }
      }
      const float aw = a_lds[w - wb][h];
      float sc[2][4];
      float wmax = -INFINITY;
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = cs[tau][i] + row_ror8(cs[tau][i]);
          float x = fmaf(v, zfac, aw);
          if (tokb + 16 * tau + 4 * g + i >= len) x = -INFINITY;
          sc[tau][i] = x;
          wmax = fmaxf(wmax, x);
        }
      }
      wmax = group_max(wmax);
      const float m_new = fmaxf(m_ref, wmax);
      const bool grow = m_new > m_ref + kLazyRescale;
      if (__any(grow)) {
        const float alf = grow ? exp2f(m_ref - m_new) : 1.0f;
        if (grow) m_ref = m_new;
        l_part *= alf;
#pragma unroll
        for (int m = 0; m < kMaxModalities; ++m)
#pragma unroll
          for (int u = 0; u < NU; ++u) acc[m][u] *= alf;
      }
      // ---- probabilities (relative to m_ref) times the value scale, split hi/lo
      float pt[2][4];
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool valid = tokb + 16 * tau + 4 * g + i < len;
          const float p = valid ? exp2f(sc[tau][i] - m_ref) : 0.0f;
          l_part += p;
          const uint32_t sbits = (i < 2 ? sig2[tau].x : sig2[tau].y) >> (16 * (i & 1));
          // tokens past the length may hold any bits: keep them out of the products
          pt[tau][i] = valid ? p * f16_value(static_cast<uint16_t>(sbits & 0xFFFFu)) : 0.0f;
        }
      }
      uint32_t bvw[4];
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        half2_t hv;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float x = pt[qd >> 1][2 * (qd & 1) + e];
          const _Float16 hi = static_cast<_Float16>(x);
          const float rest = part ? static_cast<float>(hi) : 0.0f;
          hv[e] = static_cast<_Float16>(x - rest);
        }
        bvw[qd] = __builtin_bit_cast(uint32_t, hv);
      }
      // ---- value levels: one table read per pair of codes
      uint4_t av[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (u < NU) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int p = 4 * u + i;
            av[u][i] = vtab[(vw[p / PPW] >> (2 * VB * (p % PPW))) & PMASK];
          }
        } else {
          av[u] = uint4_t{0u, 0u, 0u, 0u};
        }
      }
      // ---- modality routing
      const uint32_t t0tag = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(tg[0] & 0xFFu));
      const uint32_t rep = t0tag * 0x01010101u;
      const bool uniform = __all((tg[0] == rep) && (tg[1] == rep));
      if (uniform) {
        const uint4_t bv = uint4_t{bvw[0], bvw[1], bvw[2], bvw[3]};
        if (t0tag == 0) acc_mfma<0>(acc, av, bv, NU);
        else if (t0tag == 1) acc_mfma<1>(acc, av, bv, NU);
        else acc_mfma<2>(acc, av, bv, NU);
        seen |= 1u << t0tag;
      } else {
#pragma unroll
        for (int m = 0; m < kMaxModalities; ++m) {
          // keep the fp16 halves of tokens whose tag is m
          uint32_t bm[4];
          bool any = false;
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            const uint32_t tw = tg[qd >> 1];
            const uint32_t t0 = (tw >> (16 * (qd & 1))) & 0xFFu;
            const uint32_t t1 = (tw >> (16 * (qd & 1) + 8)) & 0xFFu;
            const uint32_t msk = (t0 == static_cast<uint32_t>(m) ? 0x0000FFFFu : 0u) |
                                 (t1 == static_cast<uint32_t>(m) ? 0xFFFF0000u : 0u);
            any = any || (msk != 0u);
            bm[qd] = bvw[qd] & msk;
          }
          if (__any(any)) {
            const uint4_t bv = uint4_t{bm[0], bm[1], bm[2], bm[3]};
            if (m == 0) acc_mfma<0>(acc, av, bv, NU);
            else if (m == 1) acc_mfma<1>(acc, av, bv, NU);
            else acc_mfma<2>(acc, av, bv, NU);
            seen |= 1u << m;
          }
        }
      }
    }
    __syncthreads();
  }

  // ---- epilogue: partial results of this split
  const float l = group_sum(l_part);
  if (lane < kMaxGroup && lane < a.group) a.ws_ml[pidx * kMaxGroup + lane] = make_float2(m_ref, l);
  if (lane == 0) a.ws_mask[pidx] = seen;
#pragma unroll
  for (int m = 0; m < kMaxModalities; ++m) {
    if (!(seen & (1u << m))) continue;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      float4_t v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = acc[m][u][i] + row_ror8(acc[m][u][i]);
      if (part == 0 && head_ok) {
        float* dst = a.ws_acc + ((pidx * kMaxModalities + m) * kMaxGroup + h) * D + 16 * u + 4 * g;
        *reinterpret_cast<float4_t*>(dst) = v;
      }
    }
  }
}

struct CombineArgs {
  const int32_t* seq_lens;
  const float* rotations;  // [M][d][d]
  int hq, hkv, group, modalities, splits;
  const float2* ws_ml;
  const uint32_t* ws_mask;
  const float* ws_acc;
  float* out;
};

// One block per (sequence, KV head): merge the splits, then out = sum_m U_m A_m.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(CombineArgs a) {
  __shared__ float A[kMaxModalities][kMaxGroup][D];
  __shared__ float wsum[kMaxGroup];
  const int unit = blockIdx.x;
  const int b = unit / a.hkv, kvh = unit % a.hkv;
  const int tid = threadIdx.x;
  const size_t base = static_cast<size_t>(unit) * a.splits;
  // (head, channel) pairs handled by this thread
  for (int e = tid; e < kMaxGroup * D; e += blockDim.x) {
    const int h = e / D, c = e % D;
    float mx = -INFINITY;
    for (int s = 0; s < a.splits; ++s) {
      const float2 ml = a.ws_ml[(base + s) * kMaxGroup + h];
      if (h < a.group && ml.y > 0.0f) mx = fmaxf(mx, ml.x);
    }
    float lsum = 0.0f;
    float acc[kMaxModalities] = {0.0f, 0.0f, 0.0f};
    if (h < a.group && mx > -INFINITY) {
      for (int s = 0; s < a.splits; ++s) {
        const float2 ml = a.ws_ml[(base + s) * kMaxGroup + h];
        if (!(ml.y > 0.0f)) continue;
        const float wgt = exp2f(ml.x - mx);
        lsum += wgt * ml.y;
        const uint32_t msk = a.ws_mask[base + s];
#pragma unroll
        for (int m = 0; m < kMaxModalities; ++m)
          if (msk & (1u << m))
            acc[m] += wgt * a.ws_acc[(((base + s) * kMaxModalities + m) * kMaxGroup + h) * D + c];
      }
    }
    const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
#pragma unroll
    for (int m = 0; m < kMaxModalities; ++m) A[m][h][c] = acc[m] * inv;
  }
  __syncthreads();
  for (int e = tid; e < a.group * D; e += blockDim.x) {
    const int h = e / D, c = e % D;
    float o = 0.0f;
    for (int m = 0; m < a.modalities; ++m) {
      const float* Ur = a.rotations + (static_cast<size_t>(m) * D + c) * D;  // row c of U_m
      for (int kk = 0; kk < D; ++kk) o = fmaf(Ur[kk], A[m][h][kk], o);
    }
    a.out[(static_cast<size_t>(b) * a.hq + kvh * a.group + h) * D + c] = o;
  }
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace

DecodePlan plan_decode(const Shape& sh, int batch, int64_t max_len, int requested) {
  DecodePlan p{};
  const int64_t nwin = (max_len + kWindow - 1) / kWindow;
  const int64_t units = static_cast<int64_t>(batch) * sh.hkv;
  int64_t splits;
  if (requested > 0) {
    splits = requested;
  } else {
    const int64_t target = 2048;  // ~2 waves per SIMD on 256 CUs
    splits = (target + units - 1) / units;
    splits = std::min<int64_t>(splits, std::max<int64_t>(1, (nwin + 7) / 8));
  }
  splits = std::max<int64_t>(1, std::min<int64_t>(splits, std::max<int64_t>(1, nwin)));
  const int64_t wps = std::max<int64_t>(1, (nwin + splits - 1) / splits);
  if (requested <= 0) splits = std::max<int64_t>(1, (nwin + wps - 1) / wps);
  p.splits = static_cast<int>(splits);
  p.windows_per_split = static_cast<int>(wps);
  const size_t parts = static_cast<size_t>(units) * splits;
  p.workspace_bytes = align256(parts * kMaxGroup * sizeof(float2)) + align256(parts * sizeof(uint32_t)) +
                      align256(parts * kMaxModalities * kMaxGroup * sh.d * sizeof(float));
  return p;
}

template <int D, int KB, int VB>
static hipError_t launch_decode_t(const Shape& sh, const DeviceTables& tb, const DecodePlan& plan,
                                  const float* q, const int32_t* seq_lens, int batch, int64_t max_len,
                                  const uint32_t* kc, const uint16_t* km, const uint16_t* ks,
                                  const uint32_t* vc, const uint16_t* vs, const uint8_t* mod,
                                  int64_t t_cap, float scale, void* ws, float* out, hipStream_t st) {
  const size_t parts = static_cast<size_t>(batch) * sh.hkv * plan.splits;
  char* w = static_cast<char*>(ws);
  float2* ml = reinterpret_cast<float2*>(w);
  w += align256(parts * kMaxGroup * sizeof(float2));
  uint32_t* mask = reinterpret_cast<uint32_t*>(w);
  w += align256(parts * sizeof(uint32_t));
  float* accw = reinterpret_cast<float*>(w);

  PartialArgs pa{q, seq_lens, kc, km, ks, vc, vs, mod, tb.signs, tb.pair_table, sh.hq, sh.hkv, sh.group,
                 sh.modalities, t_cap, max_len, scale * 1.4426950408889634f, plan.windows_per_split, plan.splits,
                 ml, mask, accw};
  const dim3 grid(static_cast<unsigned>(plan.splits), static_cast<unsigned>(batch * sh.hkv));
  decode_partial_kernel<D, KB, VB><<<grid, 64, 0, st>>>(pa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  CombineArgs ca{seq_lens, tb.rotations, sh.hq, sh.hkv, sh.group, sh.modalities, plan.splits, ml, mask, accw, out};
  decode_combine_kernel<D><<<dim3(static_cast<unsigned>(batch * sh.hkv)), 256, 0, st>>>(ca);
  return hipGetLastError();
}

hipError_t launch_decode(const Shape& sh, const DeviceTables& tb, const DecodePlan& plan, const float* q,
                         const int32_t* seq_lens, int batch, int64_t max_len, const uint32_t* kc,
                         const uint16_t* km, const uint16_t* ks, const uint32_t* vc, const uint16_t* vs,
                         const uint8_t* mod, int64_t t_cap, float scale, void* ws, float* out,
                         hipStream_t st) {
#define OMNIKV_DEC(D_, KB_, VB_)                                                                          \
  if (sh.d == D_ && sh.kbits == KB_ && sh.vbits == VB_)                                                   \
    return launch_decode_t<D_, KB_, VB_>(sh, tb, plan, q, seq_lens, batch, max_len, kc, km, ks, vc, vs, mod, t_cap, \
                                         scale, ws, out, st);
  OMNIKV_DEC(128, 2, 2)
  OMNIKV_DEC(128, 4, 4)
  OMNIKV_DEC(128, 2, 4)
  OMNIKV_DEC(128, 4, 2)
  OMNIKV_DEC(64, 2, 2)
  OMNIKV_DEC(64, 4, 4)
  OMNIKV_DEC(64, 2, 4)
  OMNIKV_DEC(64, 4, 2)
#undef OMNIKV_DEC
  return hipErrorInvalidValue;
}

}  // namespace omnikv
