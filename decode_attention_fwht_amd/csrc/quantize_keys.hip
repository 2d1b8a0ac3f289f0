// Key write path: shared randomized Hadamard rotation, then one min-max range
// per (KV head, 32-token window, rotated channel) mapped onto the fixed uniform
// codebook {0, ..., 2^bits - 1}.
//   [paper] "OmniKVQuant: KV Cache Quantization for Omni-LLMs", §1 Introduction
//   (TurboQuant's rotation; temporal key drift), §3.1 Implementation details
//   (32-token groups; MXFP4 metadata by default), §3.3 Error comparison (m_gc, s_gc
//   in FP16).
//
// One 64-lane wave owns one window of one (sequence, KV head).  A token spans D/8 lanes
// of one 16-lane row, eight consecutive channels per lane, so a wave holds 64/(D/8)
// tokens at a time: the Hadamard stages h = 1, 2, 4 stay inside the lane and the larger
// ones pair lanes of the same row (data-parallel-primitive moves, no LDS).  Every stage
// adds or subtracts the same two values as the documented butterfly order, so codes and
// metadata are bit-identical to any implementation of the same definition.
#include <type_traits>

#include "omnikv_internal.h"

namespace omnikv {
namespace {

template <int D>
struct RhtConst;
template <>
struct RhtConst<64> {
  static constexpr float value = 0.125f;
};
template <>
struct RhtConst<128> {
  static constexpr float value = 0.08838834764831845f;  // nearest fp32 to 1/sqrt(128)
};

__device__ __forceinline__ uint16_t f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}
__device__ __forceinline__ float f16_value(uint16_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

template <bool BF16>
__device__ __forceinline__ float load_elem(const void* p, size_t idx) {
  if constexpr (BF16) {
    const uint16_t b = static_cast<const uint16_t*>(p)[idx];
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
  } else {
    return static_cast<const float*>(p)[idx];
  }
}

// (word within the lane, bit) of key code (window-token tile tau, K-step s, element j);
// mirrors the window-block layout documented in include/omnikv.h.
template <int D, int KB>
__device__ __forceinline__ void key_slot(int tau, int s, int j, int& lw, int& bit) {
  const int i = j >> 1, e = j & 1;
  int slot;
  if constexpr (D == 128 && KB == 2) {
    lw = i;
    slot = 4 * tau + s;
  } else if constexpr (D == 128 && KB == 4) {
    lw = 4 * tau + i;
    slot = s;
  } else if constexpr (D == 64 && KB == 2) {
    lw = i & 1;
    slot = 4 * (i >> 1) + 2 * tau + s;
  } else {
    lw = i;
    slot = 2 * tau + s;
  }
  bit = 16 * e + KB * slot;
}

constexpr int kWavesPerBlock = 4;

// value of lane l + N within each 16-lane row (0 past the row's end)
template <int N>
__device__ __forceinline__ uint32_t row_shl(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x100 + N, 0xF, 0xF, false));
}

// Lane labels of the key rotation.  A token's 128 (64) channels sit 8 per lane on LPT = 16 (8)
// lanes; lane l of the token's row holds channel group q = a + 2b + 4c + 8d, where
// l = a ^ 2b ^ 7c ^ 8d (c, d: bits 2, 3 of l; a, b: bits 0, 1 of l, each xor c).  Flipping
// group bit 0, 1, 2 or 3 is then lane l ^ 1, l ^ 2, l ^ 7 or l ^ 8: quad_perm, quad_perm,
// row_half_mirror and row_ror:8, one DPP pattern each, so every butterfly stage across
// lanes is one fused multiply-add with a DPP source.  A 32-channel block (group bits c, d
// fixed) still fills one quad of lanes.
__device__ __forceinline__ int channel_group(int l) {
  const int c = (l >> 2) & 1, d = (l >> 3) & 1;
  const int a = (l & 1) ^ c, b = ((l >> 1) & 1) ^ c;
  return a + 2 * b + 4 * c + 8 * d;
}

// One butterfly stage over a lane's eight values: z[e] += sgn * (z[e] of the lane whose
// channel group differs in bit K), one v_fmac_f32 with a DPP source each.  Written in asm:
// the compiler does not fold a DPP move into fmac.  The leading wait states cover a value
// written by the instruction just before the block (a DPP source needs two); inside the
// block each source was written at least eight instructions earlier.
#define OMNIKV_FMAC8(pat)                                                                   \
  "s_nop 1\n\t"                                                                             \
  "v_fmac_f32_dpp %0, %0, %8 " pat " row_mask:0xf bank_mask:0xf\n\t"                        \
  "v_fmac_f32_dpp %1, %1, %8 " pat " row_mask:0xf bank_mask:0xf\n\t"                        \
  "v_fmac_f32_dpp %2, %2, %8 " pat " row_mask:0xf bank_mask:0xf\n\t"                        \
  "v_fmac_f32_dpp %3, %3, %8 " pat " row_mask:0xf bank_mask:0xf\n\t"                        \
  "v_fmac_f32_dpp %4, %4, %8 " pat " row_mask:0xf bank_mask:0xf\n\t"                        \
  "v_fmac_f32_dpp %5, %5, %8 " pat " row_mask:0xf bank_mask:0xf\n\t"                        \
  "v_fmac_f32_dpp %6, %6, %8 " pat " row_mask:0xf bank_mask:0xf\n\t"                        \
  "v_fmac_f32_dpp %7, %7, %8 " pat " row_mask:0xf bank_mask:0xf"
template <int K>
__device__ __forceinline__ void group_stage(float (&z)[8], float sgn) {
#define OMNIKV_FMAC8_OPS                                                                     \
  : "+v"(z[0]), "+v"(z[1]), "+v"(z[2]), "+v"(z[3]), "+v"(z[4]), "+v"(z[5]), "+v"(z[6]), "+v"(z[7]) \
  : "v"(sgn)
  if constexpr (K == 0) asm(OMNIKV_FMAC8("quad_perm:[1,0,3,2]") OMNIKV_FMAC8_OPS);
  else if constexpr (K == 1) asm(OMNIKV_FMAC8("quad_perm:[2,3,0,1]") OMNIKV_FMAC8_OPS);
  else if constexpr (K == 2) asm(OMNIKV_FMAC8("row_half_mirror") OMNIKV_FMAC8_OPS);
  else asm(OMNIKV_FMAC8("row_ror:8") OMNIKV_FMAC8_OPS);
#undef OMNIKV_FMAC8_OPS
}
#undef OMNIKV_FMAC8

// value of lane l ^ (1 << k) within each 16-lane row (k = 0 .. 3).  Each move reads a
// valid source lane for every lane it writes, so no lane needs a prior value (no zero fill
// or copy before the move).
template <int K>
__device__ __forceinline__ float row_xor(float x) {
  const int v = __builtin_bit_cast(int, x);
  if constexpr (K == 0) {  // quad_perm [1, 0, 3, 2]
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false));
  } else if constexpr (K == 1) {  // quad_perm [2, 3, 0, 1]
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false));
  } else if constexpr (K == 2) {
    // lanes 0-3 and 8-11 of a row read lane + 4 (row_shl:4), lanes 4-7 and 12-15 lane - 4
    // (row_shr:4); the bank mask picks which lanes each move writes
    const int lo = __builtin_amdgcn_mov_dpp(v, 0x104, 0xF, 0x5, false);
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(lo, v, 0x114, 0xF, 0xA, false));
  } else {  // row_ror:8
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false));
  }
}

// ---- MXFP4 metadata (OCP microscaling: blocks of 32 elements, one E8M0 exponent, E2M1
// elements).  Shared exponent of a block whose largest magnitude is amax:
// floor(log2 amax) - 2, at least -127 (zero and subnormal amax give -127).
__device__ __forceinline__ int mx_exponent(float amax) {
  const int ef = static_cast<int>((__float_as_uint(amax) >> 23) & 0xFFu);
  return ef == 0 ? -127 : max(ef - 127 - 2, -127);
}
// E2M1 code (sign in bit 3) of x / 2^e, rounded to nearest with ties to the even code and
// magnitudes past 6 saturating, and its decoded value (E2M1 value times 2^e, exact).
// inv = 2^-e exactly, so v = |x| * inv is exact wherever it can reach a rounding boundary.
// Round-to-nearest-even of the significand is rint(v / step) * step with the step of v's
// binade: 0.5 below 2 (with the subnormal code 0.5), 1 in [2, 4), 2 from 4.
__device__ __forceinline__ uint32_t mx_encode(float x, float inv, int e, float& value) {
  const float v = fabsf(x) * inv;
  const bool b0 = v < 2.0f, b1 = v < 4.0f;
  const float step = b0 ? 0.5f : (b1 ? 1.0f : 2.0f);
  const float rstep = b0 ? 2.0f : (b1 ? 1.0f : 0.5f);
  const float qv = fminf(__builtin_rintf(v * rstep) * step, 6.0f);  // powers of two: exact
  // code: 2 qv below 1 (0 or 1), else 2 (binade + 1) + mantissa bit = (fp32 bits >> 22) - 252
  const uint32_t c = qv < 1.0f ? static_cast<uint32_t>(2.0f * qv) : (__float_as_uint(qv) >> 22) - 252u;
  value = __builtin_copysignf(ldexpf(qv, e), x);
  return c | ((__float_as_uint(x) >> 31) << 3);
}

template <int D, int KB, bool BF16, bool MX>
__global__ __launch_bounds__(256, 4) void quantize_keys_kernel(
    const void* __restrict__ k, int hkv, WindowSource src, int64_t nwin_cap,
    int64_t tasks, const float* __restrict__ signs, uint32_t* __restrict__ k_codes,
    uint16_t* __restrict__ k_min, uint16_t* __restrict__ k_scale) {
  constexpr int L = (1 << KB) - 1;           // largest code
  constexpr int KW = D * KB / 64;            // output words per lane
  constexpr int NS = D / 32;                 // K-steps of the decode operand
  constexpr int ROW = D + 8;                 // padded LDS row (bytes)
  constexpr int LPT = D / 8;                 // lanes per token
  constexpr int TPI = 64 / LPT;              // tokens per pass
  constexpr int NP = kWindow / TPI;          // passes per window
  constexpr int XS = D == 128 ? 4 : 3;       // cross-lane stages (lane bits 0 .. XS-1)
  __shared__ uint8_t codes_lds[kWavesPerBlock][kWindow][ROW];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t task = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave;  // wave-uniform (scalar math)
  // task -> (sequence, window, head), heads fastest so a block reads adjacent token rows
  const WindowTask wt = map_window_task(src, task, tasks, hkv);
  const bool active = wt.active;
  const int64_t b = wt.b;
  const int h = wt.h;
  const size_t blk = (static_cast<size_t>(b) * hkv + h) * nwin_cap + wt.tok0 / kWindow;
  // channels 8q .. 8q + 7 of token TPI * pass + r (q: the lane's channel group)
  const int q = channel_group(lane % LPT), r = lane / LPT;

  // c_d times the sign the cross stages leave on this lane's values
  const float rht_lane = (__builtin_popcount(q & ((1 << XS) - 1)) & 1) ? -RhtConst<D>::value : RhtConst<D>::value;
  if (active) {
    float sg[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sg[e] = signs[8 * q + e];
    // bf16 input: the signs flip the sign bits of each raw word (both halves at once)
    uint32_t sx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sx[i] = (sg[2 * i] < 0.0f ? 0x00008000u : 0u) | (sg[2 * i + 1] < 0.0f ? 0x80000000u : 0u);
    float y[NP][8];
    float mn[8], mx[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      mn[e] = INFINITY;
      mx[e] = -INFINITY;
    }
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const int t = TPI * pp + r;
      const size_t row = ((static_cast<size_t>(wt.src_row) + t) * hkv + h) * D + 8 * q;
      float z[8];
      if constexpr (BF16) {
        const uint4 raw = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(k) + row);
        const uint32_t wds[4] = {raw.x ^ sx[0], raw.y ^ sx[1], raw.z ^ sx[2], raw.w ^ sx[3]};
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = __uint_as_float((e & 1) ? (wds[e >> 1] & 0xFFFF0000u) : (wds[e >> 1] << 16));
      } else {
        const float4 f0 = *reinterpret_cast<const float4*>(static_cast<const float*>(k) + row);
        const float4 f1 = *reinterpret_cast<const float4*>(static_cast<const float*>(k) + row + 4);
        z[0] = f0.x; z[1] = f0.y; z[2] = f0.z; z[3] = f0.w;
        z[4] = f1.x; z[5] = f1.y; z[6] = f1.z; z[7] = f1.w;
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = z[e] * sg[e];
      }
      // stages h = 1, 2, 4 inside the lane: lower index keeps a + b, upper gets a - b
#pragma unroll
      for (int hh = 1; hh < 8; hh <<= 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (e & hh) continue;
          const float a0 = z[e], b0 = z[e + hh];
          z[e] = a0 + b0;
          z[e + hh] = a0 - b0;
        }
      }
      // stages h = 8 << kk across the lanes whose groups differ in bit kk.  Every lane
      // computes own + sgn * partner (one rounding), sgn = -1 where group bit kk is set: the
      // lower lane gets a + b, the upper b - a = -(a - b).  The stored value is therefore the
      // butterfly's result times (-1)^(bits set among those stages), a sign of the lane that
      // the final scale takes back (rounding is symmetric, so the values are those of the
      // plain butterflies).
      auto cross = [&](auto kk_c) {
        constexpr int kk = decltype(kk_c)::value;
        group_stage<kk>(z, ((q >> kk) & 1) ? -1.0f : 1.0f);
      };
      cross(std::integral_constant<int, 0>{});
      cross(std::integral_constant<int, 1>{});
      cross(std::integral_constant<int, 2>{});
      if constexpr (XS == 4) cross(std::integral_constant<int, 3>{});
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float yy = z[e] * rht_lane;
        y[pp][e] = yy;
        mn[e] = fminf(mn[e], yy);
        mx[e] = fmaxf(mx[e], yy);
      }
    }
    // the window's extremes: combine the TPI token rows holding the same channels
#pragma unroll
    for (int sh = LPT; sh < 64; sh <<= 1) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        mn[e] = fminf(mn[e], __shfl_xor(mn[e], sh, 64));
        mx[e] = fmaxf(mx[e], __shfl_xor(mx[e], sh, 64));
      }
    }
    float mf[8], sf[8];
    if constexpr (!MX) {
      uint16_t m16[8], s16[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float lo = mn[e] + 0.0f;  // a zero extreme is +0
        const float hi = mx[e] + 0.0f;
        const float step = (hi - lo) / static_cast<float>(L);
        m16[e] = f16_bits(lo);
        s16[e] = f16_bits(step);
        mf[e] = f16_value(m16[e]);
        sf[e] = f16_value(s16[e]);
      }
      if (r == 0) {
        uint32_t pm[4], ps[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          pm[x] = static_cast<uint32_t>(m16[2 * x]) | (static_cast<uint32_t>(m16[2 * x + 1]) << 16);
          ps[x] = static_cast<uint32_t>(s16[2 * x]) | (static_cast<uint32_t>(s16[2 * x + 1]) << 16);
        }
        *reinterpret_cast<uint4*>(k_min + blk * D + 8 * q) = make_uint4(pm[0], pm[1], pm[2], pm[3]);
        *reinterpret_cast<uint4*>(k_scale + blk * D + 8 * q) = make_uint4(ps[0], ps[1], ps[2], ps[3]);
      }
    } else {
      // MXFP4 records: a 32-channel block is the four lanes q = 4k .. 4k + 3 of a token
      float lo[8], step[8], am = 0.0f, as = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        lo[e] = mn[e] + 0.0f;
        step[e] = (mx[e] + 0.0f - lo[e]) / static_cast<float>(L);
        am = fmaxf(am, fabsf(lo[e]));
        as = fmaxf(as, fabsf(step[e]));
      }
      am = fmaxf(am, row_xor<0>(am));
      am = fmaxf(am, row_xor<1>(am));
      as = fmaxf(as, row_xor<0>(as));
      as = fmaxf(as, row_xor<1>(as));
      const int em = mx_exponent(am), es = mx_exponent(as);
      const float im = __uint_as_float(static_cast<uint32_t>(127 - em) << 23);  // 2^-em
      const float is = __uint_as_float(static_cast<uint32_t>(127 - es) << 23);
      uint32_t wm = 0u, ws = 0u;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t cm = mx_encode(lo[e], im, em, mf[e]), cs = mx_encode(step[e], is, es, sf[e]);
        wm |= cm << (4 * e);
        ws |= cs << (4 * e);
      }
      // exponent bytes of the D/32 blocks, gathered in lane q = 0 of each token (lanes q = 4,
      // 8, 12 of the same 16-lane row, read by row shifts)
      const uint32_t bm = static_cast<uint32_t>(em + 127), bs = static_cast<uint32_t>(es + 127);
      uint32_t xm = bm, xs = bs;
      xm |= row_shl<4>(bm) << 8;
      xs |= row_shl<4>(bs) << 8;
      if constexpr (D == 128) {
        xm |= (row_shl<8>(bm) << 16) | (row_shl<12>(bm) << 24);
        xs |= (row_shl<8>(bs) << 16) | (row_shl<12>(bs) << 24);
      }
      if (r == 0) {
        uint8_t* rm = reinterpret_cast<uint8_t*>(k_min) + blk * mx_record_bytes(D);
        uint8_t* rs = reinterpret_cast<uint8_t*>(k_scale) + blk * mx_record_bytes(D);
        *reinterpret_cast<uint32_t*>(rm + 4 * q) = wm;
        *reinterpret_cast<uint32_t*>(rs + 4 * q) = ws;
        if (q == 0) {
          // exponents, then zeros to the end of the record
          *reinterpret_cast<uint4*>(rm + D / 2) = make_uint4(xm, 0u, 0u, 0u);
          *reinterpret_cast<uint4*>(rs + D / 2) = make_uint4(xs, 0u, 0u, 0u);
        }
      }
    }
    // code = #{j : y >= m + s (j + 1/2)}; the thresholds rise with j, so for 4-bit codes a
    // binary search over j finds the same count.  A pass's eight codes (one byte each) go
    // to LDS with one 8-byte store.
    float th[8][KB == 2 ? L : 1];
    if constexpr (KB == 2) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int j = 0; j < L; ++j) th[e][j] = mf[e] + sf[e] * (static_cast<float>(j) + 0.5f);
    } else {
      // the search's first candidate is j = 7 for every element of a channel
#pragma unroll
      for (int e = 0; e < 8; ++e) th[e][0] = mf[e] + sf[e] * 7.5f;
    }
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      uint32_t cw[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if constexpr (KB == 2) {
          // the thresholds rise with j: the high bit is y >= theta_1, the low bit y >= theta_2
          // or y >= theta_0 after it (the same count, two compares); both bits go straight to
          // their byte
          const bool hi = y[pp][e] >= th[e][1];
          const bool lo = y[pp][e] >= (hi ? th[e][2] : th[e][0]);
          cw[e >> 2] |= (hi ? (2u << (8 * (e & 3))) : 0u) | (lo ? (1u << (8 * (e & 3))) : 0u);
        } else {
          // invariant: y >= theta_j for every j < code.  The code is carried as a float (small
          // integers and halves are exact), so a candidate's j + 1/2 takes one add and its
          // threshold is the definition's fl(m + fl(s (j + 1/2))); the first candidate, j = 7,
          // has its threshold per channel.
          static_assert(KB != 4 || L == 15, "four halvings cover codes 0 .. 15");
          float fc = y[pp][e] >= th[e][0] ? 8.0f : 0.0f;
#pragma unroll
          for (int stp = 4; stp >= 1; stp >>= 1) {
            const float thj = mf[e] + sf[e] * (fc + (static_cast<float>(stp) - 0.5f));
            fc = (y[pp][e] >= thj) ? fc + static_cast<float>(stp) : fc;
          }
          cw[e >> 2] |= static_cast<uint32_t>(fc) << (8 * (e & 3));
        }
      }
      *reinterpret_cast<uint2*>(&codes_lds[wave][TPI * pp + r][8 * q]) = make_uint2(cw[0], cw[1]);
    }
  }
  __syncthreads();
  if (!active) return;
  // pack: lane = 16 g + rho holds tokens rho, rho + 16 of channels g*D/4 + 8 s + j
  const int rho = lane & 15, g = lane >> 4;
  uint32_t words[KW];
#pragma unroll
  for (int x = 0; x < KW; ++x) words[x] = 0u;
  // codes j = 2i and 2i + 1 of a group of eight share a word, 16 bits apart: one byte
  // select puts both in place, one shift-or adds them to the word
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint2 eight = *reinterpret_cast<const uint2*>(&codes_lds[wave][16 * tau + rho][g * (D / 4) + 8 * s]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t src = i < 2 ? eight.x : eight.y;
        const uint32_t pair = __builtin_amdgcn_perm(0u, src, (i & 1) ? 0x0C030C02u : 0x0C010C00u);
        int lw, bit;
        key_slot<D, KB>(tau, s, 2 * i, lw, bit);
        words[lw] |= pair << bit;
      }
    }
  }
  uint32_t* dst = k_codes + blk * (D * KB) + lane * KW;
#pragma unroll
  for (int x = 0; x < KW; x += 2) *reinterpret_cast<uint2*>(dst + x) = make_uint2(words[x], words[x + 1]);
}

template <int D, int KB, bool MX>
hipError_t launch_kb(const DeviceTables& tb, const void* k, bool bf16, int hkv, int batch, const WindowSource& src,
                     int64_t t_cap, uint32_t* kc, uint16_t* km, uint16_t* ks, hipStream_t stream) {
  const int64_t tasks = static_cast<int64_t>(batch) * hkv * src.windows_per_sequence();
  if (tasks > kMaxWindowTasks) return hipErrorInvalidConfiguration;  // the task indices are 32-bit
  const dim3 grid(static_cast<unsigned>((tasks + kWavesPerBlock - 1) / kWavesPerBlock));
  if (bf16)
    quantize_keys_kernel<D, KB, true, MX><<<grid, 256, 0, stream>>>(k, hkv, src, t_cap / kWindow, tasks, tb.signs,
                                                                    kc, km, ks);
  else
    quantize_keys_kernel<D, KB, false, MX><<<grid, 256, 0, stream>>>(k, hkv, src, t_cap / kWindow, tasks, tb.signs,
                                                                     kc, km, ks);
  return hipGetLastError();
}

template <bool MX>
hipError_t launch_meta(const Shape& sh, const DeviceTables& tb, const void* k, bool bf16, int batch,
                       const WindowSource& src, int64_t t_cap, uint32_t* kc, uint16_t* km, uint16_t* ks,
                       hipStream_t stream) {
  if (sh.d == 128 && sh.kbits == 2) return launch_kb<128, 2, MX>(tb, k, bf16, sh.hkv, batch, src, t_cap, kc, km, ks, stream);
  if (sh.d == 128 && sh.kbits == 4) return launch_kb<128, 4, MX>(tb, k, bf16, sh.hkv, batch, src, t_cap, kc, km, ks, stream);
  if (sh.d == 64 && sh.kbits == 2) return launch_kb<64, 2, MX>(tb, k, bf16, sh.hkv, batch, src, t_cap, kc, km, ks, stream);
  return launch_kb<64, 4, MX>(tb, k, bf16, sh.hkv, batch, src, t_cap, kc, km, ks, stream);
}

}  // namespace

hipError_t launch_quantize_keys(const Shape& sh, const DeviceTables& tb, const void* k, bool bf16,
                                int batch, const WindowSource& src, int64_t t_cap, uint32_t* kc,
                                uint16_t* km, uint16_t* ks, hipStream_t stream) {
  if (sh.mx) return launch_meta<true>(sh, tb, k, bf16, batch, src, t_cap, kc, km, ks, stream);
  return launch_meta<false>(sh, tb, k, bf16, batch, src, t_cap, kc, km, ks, stream);
}

}  // namespace omnikv
