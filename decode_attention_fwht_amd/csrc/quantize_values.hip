// Value write path: per-token RMS scale, rotation by the basis U_m of the
// token's modality ([paper] "OmniKVQuant: KV Cache Quantization for Omni-LLMs",
// §2.3 "Modality-aware value rotation"), then the fixed Lloyd-Max codebook.
//
// One 64-lane wave owns one 32-token window of one (sequence, KV head); lane l
// computes rotated channels l and l + 64 of every token.  The rotation is the
// plain dot product accumulated in index order with every product and sum
// rounded to fp32, so the codes are bit-identical to any implementation of the
// same definition.
#include <type_traits>

#include "omnikv_internal.h"

namespace omnikv {
namespace {

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

constexpr int kWaves = 4;

template <int D, int VB, bool BF16>
__global__ __launch_bounds__(256) void quantize_values_kernel(
    const void* __restrict__ v, const uint8_t* __restrict__ modality, int hkv, WindowSource src,
    int64_t t_cap, int64_t tasks, const float* __restrict__ rot,
    const float* __restrict__ boundaries, uint32_t* __restrict__ v_codes,
    uint16_t* __restrict__ v_scale) {
  constexpr int NC = D / 64;
  constexpr int NB = (1 << VB) - 1;           // boundaries
  constexpr int VW = D * VB / 64;             // output words per lane
  constexpr int PPW = 16 / VB;                // code pairs per word
  constexpr int ROW = D + 8;
  // the window transposed, [channel][token]: the rotation reads four tokens of one
  // channel with one (broadcast) LDS read
  __shared__ __attribute__((aligned(16))) float vals[kWaves][D][kWindow];
  __shared__ uint8_t codes_lds[kWaves][kWindow][ROW];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t task = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
  const WindowTask wt = map_window_task(src, task, tasks, hkv);
  const bool active = wt.active;
  const int64_t b = wt.b;
  const int h = wt.h;
  const int64_t tok0 = wt.tok0;                                // absolute token of the window
  const size_t blk = (static_cast<size_t>(b) * hkv + h) * (t_cap / kWindow) + tok0 / kWindow;

  if (active) {
#pragma unroll 4
    for (int t = 0; t < kWindow; ++t) {
      const size_t row = ((static_cast<size_t>(wt.src_row) + t) * hkv + h) * D;
#pragma unroll
      for (int c = 0; c < NC; ++c) vals[wave][lane + 64 * c][t] = load_elem<BF16>(v, row + lane + 64 * c);
    }
  }
  __syncthreads();
  if (active) {
    // modality of every token of the window (uniform across the wave)
    const uint8_t* tagp = modality + static_cast<size_t>(b) * t_cap + tok0;
    uint32_t tw[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) tw[x] = reinterpret_cast<const uint32_t*>(tagp)[x];
    int tag[kWindow];
#pragma unroll
    for (int t = 0; t < kWindow; ++t) tag[t] = min(static_cast<int>((tw[t >> 2] >> (8 * (t & 3))) & 0xFF), kMaxModalities - 1);
    bool uniform = true;
#pragma unroll
    for (int t = 1; t < kWindow; ++t) uniform = uniform && (tag[t] == tag[0]);

    // per-token scale: stride-halving tree of squares, then sqrt(S / d)
    float sig[kWindow];
#pragma unroll
    for (int t = 0; t < kWindow; ++t) {
      float sq[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const float x = vals[wave][lane + 64 * c][t];
        sq[c] = x * x;
      }
      float s = (NC == 2) ? (sq[0] + sq[1]) : sq[0];     // pairs (i, i + 64) for d = 128
#pragma unroll
      for (int hh = 32; hh >= 1; hh >>= 1) s = s + __shfl_xor(s, hh, 64);
      const float sigma = sqrtf(s * (1.0f / static_cast<float>(D)));
      const uint16_t s16 = f16_bits(sigma);
      if (lane == t) v_scale[(static_cast<size_t>(b) * hkv + h) * t_cap + tok0 + t] = s16;
      sig[t] = f16_value(s16);
    }

    // rotation v'_c = sum_k U[k][c] v_k, k ascending, separately rounded products and sums
    float acc[kWindow][NC];
#pragma unroll
    for (int t = 0; t < kWindow; ++t)
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[t][c] = 0.0f;
    // U rows are fetched a batch of KB ahead of their use; the sums stay in k order
    constexpr int KB = 8;
    auto xs4 = [&](int kk, int t4) -> float4 {
      return *reinterpret_cast<const float4*>(&vals[wave][kk][4 * t4]);
    };
    if (uniform) {
      const float* U = rot + static_cast<size_t>(tag[0]) * D * D + lane;
      float u[KB][NC];
#pragma unroll
      for (int j = 0; j < KB; ++j)
#pragma unroll
        for (int c = 0; c < NC; ++c) u[j][c] = U[j * D + 64 * c];
      for (int k0 = 0; k0 < D; k0 += KB) {
        float un[KB][NC];
#pragma unroll
        for (int j = 0; j < KB; ++j)
#pragma unroll
          for (int c = 0; c < NC; ++c) un[j][c] = (k0 + KB < D) ? U[(k0 + KB + j) * D + 64 * c] : 0.0f;
#pragma unroll
        for (int j = 0; j < KB; ++j) {
#pragma unroll
          for (int t4 = 0; t4 < kWindow / 4; ++t4) {
            const float4 x = xs4(k0 + j, t4);
#pragma unroll
            for (int c = 0; c < NC; ++c) {
              acc[4 * t4][c] = acc[4 * t4][c] + u[j][c] * x.x;
              acc[4 * t4 + 1][c] = acc[4 * t4 + 1][c] + u[j][c] * x.y;
              acc[4 * t4 + 2][c] = acc[4 * t4 + 2][c] + u[j][c] * x.z;
              acc[4 * t4 + 3][c] = acc[4 * t4 + 3][c] + u[j][c] * x.w;
            }
          }
        }
#pragma unroll
        for (int j = 0; j < KB; ++j)
#pragma unroll
          for (int c = 0; c < NC; ++c) u[j][c] = un[j][c];
      }
    } else {
      const float* U = rot + lane;
      for (int kk = 0; kk < D; kk += 2) {
        float u[2][kMaxModalities][NC];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int m = 0; m < kMaxModalities; ++m)
#pragma unroll
            for (int c = 0; c < NC; ++c) u[j][m][c] = U[(static_cast<size_t>(m) * D + kk + j) * D + 64 * c];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int t4 = 0; t4 < kWindow / 4; ++t4) {
            const float4 x4 = xs4(kk + j, t4);
            const float xv[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int t = 4 * t4 + e;
#pragma unroll
              for (int c = 0; c < NC; ++c) {
                const float um = tag[t] == 0 ? u[j][0][c] : (tag[t] == 1 ? u[j][1][c] : u[j][2][c]);
                acc[t][c] = acc[t][c] + um * xv[e];
              }
            }
          }
        }
      }
    }
    float beta[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) beta[j] = boundaries[j];
#pragma unroll
    for (int t = 0; t < kWindow; ++t) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        int code = 0;
#pragma unroll
        for (int j = 0; j < NB; ++j) code += (acc[t][c] >= sig[t] * beta[j]) ? 1 : 0;
        codes_lds[wave][t][lane + 64 * c] = static_cast<uint8_t>(code);
      }
    }
  }
  __syncthreads();
  if (!active) return;
  // pack: lane = 16 g + rho holds channels 16 u + rho of tokens {4g..4g+3, 16+4g..16+4g+3}
  const int rho = lane & 15, g = lane >> 4;
  uint32_t words[VW];
#pragma unroll
  for (int x = 0; x < VW; ++x) words[x] = 0u;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int t = (j < 4) ? (4 * g + j) : (16 + 4 * g + (j - 4));
#pragma unroll
    for (int u = 0; u < D / 16; ++u) {
      const uint32_t code = codes_lds[wave][t][16 * u + rho];
      const int p = 4 * u + (j >> 1);
      words[p / PPW] |= code << (2 * VB * (p % PPW) + VB * (j & 1));
    }
  }
  uint32_t* dst = v_codes + blk * (D * VB) + lane * VW;
#pragma unroll
  for (int x = 0; x < VW; x += 2) *reinterpret_cast<uint2*>(dst + x) = make_uint2(words[x], words[x + 1]);
}

// ---------------------------------------------------------------------------------------
// bf16 inputs on the matrix cores.  v' = U_m^T v for the 32 tokens of a window is one
// [32 x d] x [d x d] product: v_mfma_f32_16x16x32_bf16 with the bf16 values as they come
// and the two leading parts of U_m's split into three bf16 parts whose sum is U_m exactly.
// That result and the defined sequential fp32 sum both lie within a bounded number of fp32
// roundings of the exact dot product, each rounding at most 2^-23 of the sum of |terms|,
// and that sum is at most (largest column norm of U_m) x ||v_t||_2; the omitted third part
// adds at most its own largest column norm x ||v_t||_2; so the two differ by at most
// eps_t = eps_c ||v_t||_2 (+ a tiny absolute term for underflow).  A code is taken from
// the matrix-core value when that value is farther than eps_t from every threshold - the
// sequential sum then falls on the same side of each - and otherwise from the sequential
// sum itself, recomputed for that element alone.  Either way the code is the one the
// definition gives.  An all-zero token needs no recomputation: both sums are zero.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t uint4_t __attribute__((ext_vector_type(4)));

constexpr int kNearList = 64;    // near-threshold elements a wave lists (the rest: their own lane)
constexpr int kNearBatch = 8;    // listed elements whose products are formed together

// acc * 2 + (this lane's bit of the lane mask m): one v_addc whose carry-in is the mask, so
// a comparison's lane mask enters a bit field with no 0/1 value in between
__device__ __forceinline__ uint32_t push_bit(uint32_t acc, uint64_t m) {
  uint32_t r;
  uint64_t carry_out;
  asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=s"(carry_out) : "v"(acc), "s"(m));
  return r;
}
// A fp32 value v as the sum of two bf16 operands plus a small remainder: hi is v with its
// low 16 bits cleared (exact), lo the nearest bf16 to v - hi (exact in fp32), so
// |v - hi - lo| <= 2^-8 |v - hi| < 2^-15 |v| (for |v| >= 2^-126; below, at most half the
// smallest bf16 subnormal, 2^-134).
__device__ __forceinline__ void split_bf16(float x, uint32_t& hi16, uint32_t& lo16) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t h = u & 0xFFFF0000u;
  const float r = x - __uint_as_float(h);
  const uint32_t ru = __float_as_uint(r);
  // round to nearest even at bit 16 (r is finite: x - hi of a finite x)
  const uint32_t l = (ru + 0x7FFFu + ((ru >> 16) & 1u)) & 0xFFFF0000u;
  hi16 = h >> 16;
  lo16 = l >> 16;
}

// F32: the values come as fp32; each enters the matrix cores as a bf16 hi and lo part
// (split_bf16), and the tolerance covers the remainder.  Otherwise bf16 values as they come.
// bf16 values with a symmetric codebook fit four waves per SIMD (at most 128 VGPRs); the
// bound holds them there (the fp32 and asymmetric 4-bit forms need more registers)
template <int D, int VB, bool SYM, bool F32>
__global__ __launch_bounds__(256, (!F32 && (SYM || VB == 2)) ? 4 : 1) void quantize_values_mfma_kernel(
    const void* __restrict__ vin, const uint8_t* __restrict__ modality, int hkv, WindowSource src,
    int64_t t_cap, int64_t tasks, const uint4_t* __restrict__ rot_b16,
    const float* __restrict__ rot_t, const float* __restrict__ boundaries, float eps_c,
    uint32_t* __restrict__ v_codes, uint16_t* __restrict__ v_scale) {
  constexpr int NCT = D / 16;                 // channel tiles
  constexpr int NKS = D / 32;                 // k-steps
  constexpr int NB = (1 << VB) - 1;           // boundaries
  constexpr int VW = D * VB / 64;             // output words per lane
  constexpr int PPW = 16 / VB;                // code pairs per word
  constexpr int TPW = PPW / 4;                // channel tiles per output word
  __shared__ float sig_lds[kWaves][kWindow];
  __shared__ float eps_lds[kWaves][kWindow];
  // elements near a threshold, per wave: (token, channel, modality) entries, the sequential
  // definition's codes for them, and one batch's fp32 products (rows padded by 4 floats so
  // the summing lanes' 16-byte reads fall in different banks)
  __shared__ uint32_t near_entry[kWaves][kNearList];
  __shared__ uint8_t near_code[kWaves][kNearList];
  __shared__ __attribute__((aligned(16))) float near_prod[kWaves][kNearBatch][D + 4];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t task = static_cast<int64_t>(blockIdx.x) * kWaves + wave;  // wave-uniform (scalar math)
  const WindowTask wt = map_window_task(src, task, tasks, hkv);
  const bool active = wt.active;
  const int64_t b = wt.b;
  const int h = wt.h;
  const int64_t tok0 = wt.tok0;
  const size_t blk = (static_cast<size_t>(b) * hkv + h) * (t_cap / kWindow) + tok0 / kWindow;
  const size_t row0 = (static_cast<size_t>(wt.src_row) * hkv + h) * D;  // element of token 0
  const size_t rstride = static_cast<size_t>(hkv) * D;                             // elements per token
  const int nn = lane & 15, g = lane >> 4;

  // ---- the window as matrix-core A operands: lane (nn, g) holds token 16 tt + nn,
  // channels 32 ks + 8 g .. + 7 (bf16 as they come; fp32 as hi parts in av, lo parts in al)
  const uint16_t* v = static_cast<const uint16_t*>(vin);
  const float* vf = static_cast<const float*>(vin);
  uint4_t av[2][NKS];
  uint4_t al[F32 ? 2 : 1][F32 ? NKS : 1];
  float xf[F32 ? 2 : 1][F32 ? NKS : 1][F32 ? 8 : 1];  // fp32: the values themselves, for the scale
  uint32_t tw[8];
  if (active) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if constexpr (F32) {
          const float* src8 = vf + row0 + (16 * tt + nn) * rstride + 32 * ks + 8 * g;
          const float4 f0 = *reinterpret_cast<const float4*>(src8);
          const float4 f1 = *reinterpret_cast<const float4*>(src8 + 4);
          const float e8[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            uint32_t h0, l0, h1, l1;
            split_bf16(e8[2 * x], h0, l0);
            split_bf16(e8[2 * x + 1], h1, l1);
            av[tt][ks][x] = h0 | (h1 << 16);
            al[tt][ks][x] = l0 | (l1 << 16);
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) xf[tt][ks][e] = e8[e];
        } else {
          av[tt][ks] = *reinterpret_cast<const uint4_t*>(v + row0 + (16 * tt + nn) * rstride + 32 * ks + 8 * g);
        }
      }
    const uint32_t* tagp = reinterpret_cast<const uint32_t*>(modality + static_cast<size_t>(b) * t_cap + tok0);
#pragma unroll
    for (int x = 0; x < 8; ++x) tw[x] = tagp[x];
  }

  // ---- per-token scale, from the operands already in registers.  The stride-halving tree
  // of squares pairs channels c and c + 64 (d = 128: k-steps ks and ks + 2 of the lane),
  // then c + 32 (k-steps 0 and 1), c + 16 (lanes g and g + 2: lane ^ 32), c + 8 (g and
  // g + 1: lane ^ 16), then 4, 2, 1 inside the lane.  A cross-lane level adds the two lanes' partial sums,
  // which both lanes then hold, so the four lanes of a token all end with its S; every sum
  // is the tree's own, so S is the definition's exactly.
  float S[2];
  uint32_t nz[2];
  if (active) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      float sq[NKS][8];
      uint32_t mag = 0u;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if constexpr (F32) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = xf[tt][ks][e];
            mag |= __float_as_uint(x) & 0x7FFFFFFFu;
            sq[ks][e] = x * x;
          }
        } else {
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const uint32_t wd = av[tt][ks][x];
            mag |= wd & 0x7FFF7FFFu;
            const float lo = __uint_as_float(wd << 16), hi = __uint_as_float(wd & 0xFFFF0000u);
            sq[ks][2 * x] = lo * lo;
            sq[ks][2 * x + 1] = hi * hi;
          }
        }
      }
      float s2[8];
      if constexpr (NKS == 4) {
#pragma unroll
        for (int e = 0; e < 8; ++e) s2[e] = (sq[0][e] + sq[2][e]) + (sq[1][e] + sq[3][e]);
      } else {  // d = 64: pairs (c, c + 32) are k-steps 0 and 1
#pragma unroll
        for (int e = 0; e < 8; ++e) s2[e] = sq[0][e] + sq[1][e];
      }
      // channel 8 g + e: lanes g and g + 2, then g and g + 1
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(s2[e]), __float_as_uint(s2[e]), false, false);
        s2[e] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(s2[e]), __float_as_uint(s2[e]), false, false);
        s2[e] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
      }
      const float s5[4] = {s2[0] + s2[4], s2[1] + s2[5], s2[2] + s2[6], s2[3] + s2[7]};
      S[tt] = (s5[0] + s5[2]) + (s5[1] + s5[3]);
      // tokens with a nonzero magnitude bit (subnormals count), over the four lanes
      const auto p32 = __builtin_amdgcn_permlane32_swap(mag, mag, false, false);
      mag = p32[0] | p32[1];
      const auto p16 = __builtin_amdgcn_permlane16_swap(mag, mag, false, false);
      nz[tt] = p16[0] | p16[1];
    }
  }
  if (active && g == 0) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const float sigma = sqrtf(S[tt] * (1.0f / static_cast<float>(D)));
      const uint16_t s16 = f16_bits(sigma);
      const int t = 16 * tt + nn;
      sig_lds[wave][t] = f16_value(s16);
      eps_lds[wave][t] = nz[tt] != 0u ? eps_c * sqrtf(S[tt]) + 1e-20f : -1.0f;
      v_scale[(static_cast<size_t>(b) * hkv + h) * t_cap + tok0 + t] = s16;
    }
  }
  __syncthreads();

  // ---- rotation on the matrix cores, then the codes.  Lane (nn, g) of channel tile ct holds
  // channel 16 ct + nn of tokens 16 tt + 4 g + i: exactly the codes of its own output words
  // in the window-block layout, so the lane packs them in place.
  uint32_t words[VW];
#pragma unroll
  for (int x = 0; x < VW; ++x) words[x] = 0u;
  uint64_t near_bits = 0u;  // element (ct, tt, i) at bit 8 ct + 4 tt + i
  uint32_t my_tag[2][4];    // modality of this lane's result tokens 16 tt + 4 g + i
  if (active) {
    uint32_t present = 0u;
#pragma unroll
    for (int t = 0; t < kWindow; ++t)
      present |= 1u << min((tw[t >> 2] >> (8 * (t & 3))) & 0xFFu, static_cast<uint32_t>(kMaxModalities - 1));
    // scales, tolerances and (2-bit) thresholds of the lane's result tokens.  A token whose
    // thresholds are not all finite (an infinite scale) gets an infinite tolerance: all its
    // elements take the sequential definition.
    constexpr bool kTwoBit = NB == 3;
    float th[2][4][kTwoBit ? NB : 1], my_sg[2][4], my_ep[2][4];
    float beta[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) beta[j] = boundaries[j];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const uint32_t tword = g == 0 ? tw[4 * tt] : (g == 1 ? tw[4 * tt + 1] : (g == 2 ? tw[4 * tt + 2] : tw[4 * tt + 3]));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        my_tag[tt][i] = min((tword >> (8 * i)) & 0xFFu, static_cast<uint32_t>(kMaxModalities - 1));
        my_sg[tt][i] = sig_lds[wave][16 * tt + 4 * g + i];
        const float ep = eps_lds[wave][16 * tt + 4 * g + i];
        my_ep[tt][i] = __builtin_isfinite(my_sg[tt][i]) ? ep : INFINITY;
        if constexpr (kTwoBit) {
#pragma unroll
          for (int j = 0; j < NB; ++j) th[tt][i][j] = my_sg[tt][i] * beta[j];
        }
      }
    }
    // symmetric 4-bit codebook: the token's magnitude |x| / sigma against the positive
    // boundaries, with a tolerance carried into that scale (below), and the code fields of the
    // lane's all-zero tokens (code 15: every threshold is +-0 there and x = 0)
    constexpr bool kSym4 = !kTwoBit && SYM;
    float rsg[2][4], epy[2][4];
    uint32_t zero_fields = 0u;
    if constexpr (kSym4) {
      const float bmax = beta[NB - 1];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float sg = my_sg[tt][i], ep = my_ep[tt][i];
          // an all-zero token has tolerance -1 (never near); a token whose squares underflow
          // (sigma 0, tolerance 1e-20) gets y = 0 and a positive tolerance: all its elements
          // are near and take the sequential definition, as the signs of their sums decide
          const bool zero = ep < 0.0f;
          rsg[tt][i] = sg > 0.0f ? 1.0f / sg : 0.0f;  // sigma is an fp16 value: 1 / sigma <= 2^24
          epy[tt][i] = zero ? -1.0f
                            : (!__builtin_isfinite(ep) ? INFINITY : ep * rsg[tt][i] * (1.0f + 0x1p-16f) + 0x1p-19f * bmax);
          if (zero) zero_fields |= 0xFu << (VB * (4 * tt + i));
        }
    }
    // symmetric 2-bit codebook, boundaries (-b, 0, b): away from them (the only results this
    // code decides: near ones take the sequential definition) the high bit is x >= 0 and the
    // low bit |x| >= sigma b, flipped for x < 0.  Near: within eps of 0 or of +-sigma b (the
    // two candidates for the nearest boundary); a NaN result counts.  Every test is one
    // comparison's lane mask, combined on the scalar unit with the lane masks `own` of the
    // tokens of the modality, and pushed into the bit fields from element 7 down to 0, so
    // element k = 4 tt + i lands at bits 2k (low) and 2k + 1 (high) of `bits` and at bit k
    // of `nearm`.
    auto classify_sym = [&](const float4_t (&acc)[2], const uint64_t (&own)[2][4], uint32_t& bits, uint32_t& nearm) {
#pragma unroll
      for (int k = 7; k >= 0; --k) {
        const int tt = k >> 2, i = k & 3;
        const float x = acc[tt][i], tb = th[tt][i][kTwoBit ? 2 : 0], ax = fabsf(x), ep = my_ep[tt][i];
        const uint64_t pos = __builtin_amdgcn_ballot_w64(x >= 0.0f);
        const uint64_t outer = __builtin_amdgcn_ballot_w64(ax >= tb);
        const uint64_t near =
            __builtin_amdgcn_ballot_w64(!(ax > ep)) | __builtin_amdgcn_ballot_w64(!(fabsf(ax - tb) > ep));
        bits = push_bit(bits, pos & own[tt][i]);
        bits = push_bit(bits, ~(pos ^ outer) & own[tt][i]);
        nearm = push_bit(nearm, near & own[tt][i]);
      }
    };
    // symmetric 4-bit codebook, boundaries (-b7 .. -b1, 0, b1 .. b7): with m = #{j : y >= b_j},
    // y = |x| / sigma as computed (|x| times the rounded reciprocal), the code is 8 + m for
    // x >= 0 and 7 - m below: (x >= 0 ? 8 : 7) XOR m.  Near: y within epy of 0 or of some
    // b_j.  epy = eps / sigma (1 + 2^-16) + 2^-19 b7 covers the two roundings of y and the
    // rounding of the definition's thresholds sigma b_j (relative 2^-23 and 2^-24 of values
    // at most ~b7 where it matters), so an element outside every band has |x| on the same
    // side of each threshold as y is of b_j, farther than eps.  A NaN result is near; an
    // infinite scale has an infinite tolerance.  `mine` drops the tokens of other modalities.
    // m comes from a three-level binary search over b1 .. b7 (b4, then b2 or b6, then one of
    // b1, b3, b5, b7), its three outcomes the bits of m.  The interval [b_m, b_(m+1)) that
    // holds y is bounded by two of those split points (or by 0 below b1), so the nearest
    // boundary to y is 0 or a split point on y's path: the four distances give the same
    // minimum as all eight.
    static_assert(!kSym4 || NB == 15, "the binary search covers seven positive boundaries");
    auto classify_sym4 = [&](const float4_t (&acc)[2], const bool (&mine)[2][4], const uint64_t (&own)[2][4],
                             uint32_t& bits, uint32_t& nearm) {
      const float b1 = beta[8], b2 = beta[9], b3 = beta[10], b4 = beta[11], b5 = beta[12], b6 = beta[13], b7 = beta[14];
#pragma unroll
      for (int k = 7; k >= 0; --k) {
        const int tt = k >> 2, i = k & 3;
        const float x = acc[tt][i], y = fabsf(x) * rsg[tt][i];
        const bool c1 = y >= b4;
        const float t2 = c1 ? b6 : b2;
        const bool c2 = y >= t2;
        const float t3 = c1 ? (c2 ? b7 : b5) : (c2 ? b3 : b1);
        const bool c3 = y >= t3;
        uint32_t m = push_bit(0u, __builtin_amdgcn_ballot_w64(c1));
        m = push_bit(m, __builtin_amdgcn_ballot_w64(c2));
        m = push_bit(m, __builtin_amdgcn_ballot_w64(c3));
        const float d = fminf(fminf(y, fabsf(y - b4)), fminf(fabsf(y - t2), fabsf(y - t3)));
        const uint32_t code = ((x >= 0.0f) ? 8u : 7u) ^ m;
        bits = (bits << 4) | (mine[tt][i] ? code : 0u);
        nearm = push_bit(nearm, __builtin_amdgcn_ballot_w64(!(d > epy[tt][i])) & own[tt][i]);
      }
    };
    // one channel tile's eight results -> codes (tt, i) at bit VB (4 tt + i) of `bits` and
    // near-threshold flags at bit 4 tt + i of `nearm`, for the tokens of modality m
    auto classify = [&](const float4_t (&acc)[2], uint32_t m, bool mixed, uint32_t& bits, uint32_t& nearm) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = acc[tt][i];
          const bool mine = !mixed || my_tag[tt][i] == m;
          const int sh = VB * (4 * tt + i);
          uint32_t code;
          bool near;
          if constexpr (kTwoBit) {
            // the thresholds rise (finite scale), so the three comparisons form a
            // thermometer: code = c0 + c1 + c2 has high bit c1 and low bit c0 ^ c1 ^ c2
            const bool c0 = x >= th[tt][i][0], c1 = x >= th[tt][i][1], c2 = x >= th[tt][i][2];
            code = (c1 ? 2u : 0u) | ((c0 ^ c1 ^ c2) ? 1u : 0u);
            // a NaN distance (NaN sum) stays NaN through the min and counts as near
            const float dmin = fminf(fminf(fabsf(x - th[tt][i][0]), fabsf(x - th[tt][i][1])), fabsf(x - th[tt][i][2]));
            near = !(dmin > my_ep[tt][i]);
          } else {
            code = 0u;
            near = false;
#pragma unroll
            for (int j = 0; j < NB; ++j) {
              const float thj = my_sg[tt][i] * beta[j];
              code += (x >= thj) ? 1u : 0u;
              near = near || !(fabsf(x - thj) > my_ep[tt][i]);  // NaN or infinite sums count
            }
          }
          bits |= (mine ? code : 0u) << sh;
          nearm |= (near && mine ? 1u : 0u) << (4 * tt + i);
        }
    };
#pragma unroll
    for (int m = 0; m < kMaxModalities; ++m) {
      if (!(present & (1u << m))) continue;
      const bool mixed = present != (1u << m);  // wave-uniform
      uint64_t own[2][4];  // lanes whose token (tt, i) has modality m
      bool mine[2][4];
      uint32_t mine_fields = 0u;  // (4-bit) code fields of this lane's tokens of modality m
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          mine[tt][i] = !mixed || my_tag[tt][i] == static_cast<uint32_t>(m);
          own[tt][i] = mixed ? __builtin_amdgcn_ballot_w64(my_tag[tt][i] == m) : ~uint64_t{0};
          if (mine[tt][i]) mine_fields |= 0xFu << (VB * (4 * tt + i));
        }
      const uint4_t* B = rot_b16 + static_cast<size_t>(m) * 3 * NCT * NKS * 64 + lane;
      // U_m's tiles come from L2: all eight of a channel tile are requested before its
      // products (a barrier keeps the scheduler from sinking each load to its use)
#pragma unroll 1
      for (int ct = 0; ct < NCT; ++ct) {
        uint4_t bv[2][NKS];
#pragma unroll
        for (int part = 0; part < 2; ++part)
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) bv[part][ks] = B[((part * NCT + ct) * NKS + ks) * 64];
        __builtin_amdgcn_sched_barrier(0);
        float4_t acc[2] = {float4_t{0.f, 0.f, 0.f, 0.f}, float4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int part = 0; part < 2; ++part)
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
              acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[tt][ks]),
                                                                __builtin_bit_cast(bf16x8_t, bv[part][ks]), acc[tt], 0, 0, 0);
              if constexpr (F32)
                acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, al[tt][ks]),
                                                                  __builtin_bit_cast(bf16x8_t, bv[part][ks]), acc[tt], 0, 0, 0);
            }
        uint32_t bits = 0u, nearm = 0u;
        if constexpr (kTwoBit && SYM) {
          classify_sym(acc, own, bits, nearm);
        } else if constexpr (kSym4) {
          classify_sym4(acc, mine, own, bits, nearm);
          bits |= zero_fields & mine_fields;
        } else {
          if (kTwoBit && !mixed)  // (a copy without the modality test for the common case)
            classify(acc, static_cast<uint32_t>(m), false, bits, nearm);
          else
            classify(acc, static_cast<uint32_t>(m), mixed, bits, nearm);
        }
        // token pair p = 4 ct + 2 tt + (i >> 1) goes to word p / PPW at bit 2 VB (p % PPW) +
        // VB (i & 1) = 8 VB (ct % TPW) + VB (4 tt + i), TPW = PPW / 4 tiles per word
        if constexpr (VB == 2 && VW == 4) {
          // tile ct's 16 bits go to bits 16 ct .. 16 ct + 15 of the 128-bit word queue: each
          // tile turns the queue right by 16 bits and ORs its bits into the top, so after a
          // pass's eight tiles every earlier bit is back in place and tile ct's bits sit at 16 ct
          const uint32_t w0 = words[0];
          words[0] = __builtin_amdgcn_alignbit(words[1], words[0], 16);
          words[1] = __builtin_amdgcn_alignbit(words[2], words[1], 16);
          words[2] = __builtin_amdgcn_alignbit(words[3], words[2], 16);
          words[3] = __builtin_amdgcn_alignbit(w0, words[3], 16) | (bits << 16);
        } else {
          words[ct / TPW] |= bits << (8 * VB * (ct % TPW));
        }
        near_bits |= static_cast<uint64_t>(nearm) << (8 * ct);
      }
    }
  }

  // ---- the sequential definition for the elements near a threshold (rare), wave by wave.
  // The wave lists its flagged elements in LDS.  For each batch of listed elements, lane L
  // loads terms 2L and 2L + 1 of every element's dot product (coalesced rows of U_m^T and
  // of the token) and forms their fp32 products; one lane per element then adds its 128
  // products in the definition's order.  A listed element costs the wave two loads and a
  // few instructions, and its 128-term sum runs beside the batch's others; no other wave
  // waits for it.  Elements past the list's room are computed by their own lane, alone.
  auto exact_code = [&](int t, int c, uint32_t tg) -> uint32_t {
    const float* ut = rot_t + (static_cast<size_t>(tg) * D + c) * D;
    float s = 0.0f;
    for (int k0 = 0; k0 < D; k0 += 8) {
      const float4 u0 = *reinterpret_cast<const float4*>(ut + k0);
      const float4 u1 = *reinterpret_cast<const float4*>(ut + k0 + 4);
      const float uu[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
      float xv[8];
      if constexpr (F32) {
        const float* vr = vf + row0 + t * rstride;
        const float4 a0 = *reinterpret_cast<const float4*>(vr + k0);
        const float4 a1 = *reinterpret_cast<const float4*>(vr + k0 + 4);
        xv[0] = a0.x; xv[1] = a0.y; xv[2] = a0.z; xv[3] = a0.w;
        xv[4] = a1.x; xv[5] = a1.y; xv[6] = a1.z; xv[7] = a1.w;
      } else {
        const uint4_t vb = *reinterpret_cast<const uint4_t*>(v + row0 + t * rstride + k0);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) xv[kk] = __uint_as_float(((vb[kk >> 1] >> (16 * (kk & 1))) & 0xFFFFu) << 16);
      }
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) s = s + uu[kk] * xv[kk];
    }
    const float sg = sig_lds[wave][t];
    uint32_t code = 0;
    for (int j = 0; j < NB; ++j) code += (s >= sg * boundaries[j]) ? 1u : 0u;
    return code;
  };
  // the modality of this lane's element (tt, i) (selects over the unrolled indices keep
  // the array in registers)
  auto tag_of = [&](int tt, int i) {
    uint32_t tg = 0u;
#pragma unroll
    for (int x = 0; x < 8; ++x)
      if (x == 4 * tt + i) tg = my_tag[x >> 2][x & 3];
    return tg;
  };
  if (active) {
    // Slots: pass j gives each lane's j-th flagged element (lowest bit first) the next free
    // slot, lanes in order.  The same passes run again for the patching below, so each lane
    // finds its elements' slots without storing them.
    uint32_t listed = 0u;  // wave-uniform
    {
      uint64_t todo = near_bits;
      for (;;) {
        const uint64_t has = __builtin_amdgcn_ballot_w64(todo != 0u);
        if (has == 0u) break;
        if (todo != 0u) {
          const uint32_t slot = listed + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(has >> 32),
                                                                  __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(has), 0u));
          const int k = __builtin_ctzll(todo);
          todo &= todo - 1u;
          const int ct = k >> 3, tt = (k >> 2) & 1, i = k & 3;
          if (slot < static_cast<uint32_t>(kNearList))
            near_entry[wave][slot] = (static_cast<uint32_t>(16 * tt + 4 * g + i) << 9) |
                                     (static_cast<uint32_t>(16 * ct + nn) << 2) | tag_of(tt, i);
        }
        listed += static_cast<uint32_t>(__builtin_popcountll(has));
      }
    }
    const int n = static_cast<int>(min(listed, static_cast<uint32_t>(kNearList)));
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    for (int e0 = 0; e0 < n; e0 += kNearBatch) {
      // every lane's two terms of each element of the batch, all requested before any use
      // (the bf16 pairs stay packed until every load is issued: unpacked at the load, each
      // would wait for its own load before the next is requested)
      float2 uu[kNearBatch];
      float2 vf2[F32 ? kNearBatch : 1];
      uint32_t vv[F32 ? 1 : kNearBatch];
      const bool terms = 2 * lane < D;
#pragma unroll
      for (int j = 0; j < kNearBatch; ++j) {
        uu[j] = make_float2(0.0f, 0.0f);
        if constexpr (F32) vf2[j] = make_float2(0.0f, 0.0f);
        else vv[j] = 0u;
        if (e0 + j < n && terms) {
          const uint32_t en = near_entry[wave][e0 + j];
          const int et = static_cast<int>(en >> 9), ec = static_cast<int>((en >> 2) & 127u);
          uu[j] = *reinterpret_cast<const float2*>(rot_t + (static_cast<size_t>(en & 3u) * D + ec) * D + 2 * lane);
          if constexpr (F32) vf2[j] = *reinterpret_cast<const float2*>(vf + row0 + et * rstride + 2 * lane);
          else vv[j] = *reinterpret_cast<const uint32_t*>(v + row0 + et * rstride + 2 * lane);
        }
      }
#pragma unroll
      for (int j = 0; j < kNearBatch; ++j)
        if (e0 + j < n && terms) {
          float2 x;
          if constexpr (F32) x = vf2[j];
          else x = make_float2(__uint_as_float(vv[j] << 16), __uint_as_float(vv[j] & 0xFFFF0000u));
          *reinterpret_cast<float2*>(&near_prod[wave][j][2 * lane]) = make_float2(uu[j].x * x.x, uu[j].y * x.y);
        }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      if (lane < kNearBatch && e0 + lane < n) {
        const float* pr = near_prod[wave][lane];
        float s = 0.0f;
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += 4) {
          const float4 q = *reinterpret_cast<const float4*>(pr + k0);
          s = s + q.x;
          s = s + q.y;
          s = s + q.z;
          s = s + q.w;
        }
        const uint32_t en = near_entry[wave][e0 + lane];
        const float sg = sig_lds[wave][en >> 9];
        uint32_t code = 0;
        for (int j = 0; j < NB; ++j) code += (s >= sg * boundaries[j]) ? 1u : 0u;
        near_code[wave][e0 + lane] = static_cast<uint8_t>(code);
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    }
    // patch: the same slot passes
    {
      uint64_t todo = near_bits;
      listed = 0u;
      for (;;) {
        const uint64_t has = __builtin_amdgcn_ballot_w64(todo != 0u);
        if (has == 0u) break;
        if (todo != 0u) {
          const uint32_t slot = listed + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(has >> 32),
                                                                  __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(has), 0u));
          const int k = __builtin_ctzll(todo);
          todo &= todo - 1u;
          const int ct = k >> 3, tt = (k >> 2) & 1, i = k & 3;
          const int t = 16 * tt + 4 * g + i, c = 16 * ct + nn;
          const uint32_t code = slot < static_cast<uint32_t>(kNearList) ? near_code[wave][slot] : exact_code(t, c, tag_of(tt, i));
          const int bit = 8 * VB * (ct % TPW) + 4 * VB * tt + VB * i;
#pragma unroll
          for (int x = 0; x < VW; ++x)
            if (x == ct / TPW) words[x] = (words[x] & ~(((1u << VB) - 1u) << bit)) | (code << bit);
        }
        listed += static_cast<uint32_t>(__builtin_popcountll(has));
      }
    }
    uint32_t* dst = v_codes + blk * (D * VB) + lane * VW;
#pragma unroll
    for (int x = 0; x < VW; x += 2) *reinterpret_cast<uint2*>(dst + x) = make_uint2(words[x], words[x + 1]);
  }
}

// The tolerance eps_t = eps ||v_t||_2 between the matrix-core value and the sequential
// definition, eps = value_eps_unit * (largest column norm of U_m) + 1.02 * (largest column
// norm of the third bf16 part of U_m, which the matrix cores leave out: its dot product
// with v is at most that times ||v||_2).  value_eps_unit counts, in units of the sum of
// |terms| of one dot product: matrix cores, 2 d/32 instructions per output, each adding 32
// exact bf16 products to the accumulator with an error of at most 34 x 2^-23 of (|acc| +
// those products), in case the unit aligns the addends by truncation; sequential, d
// products and d sums, each rounded to nearest.  The two bf16 parts of U_m sum in
// magnitude to at most 1.01 |U_m|, and a 2% margin covers the rounding of ||v||_2 =
// sqrt(S) and of |v' - theta|.
template <int D>
constexpr double value_eps_unit() {
  return 1.02 * 1.01 * (68.0 * (2 * (D / 32) + 1) + (2 * D + 2)) / 16777216.0;
}
// The same for fp32 values (split_bf16): twice the matrix-core instructions per output, the
// terms' magnitudes at most (1 + 2^-7) those of the definition (one more 1.01), and the
// remainder v - hi - lo, at most 2^-15 |v| per value, whose dot product with a column of
// U_m is at most 2^-15 ||U_m column|| ||v||_2 (the last term, in units of the column norm).
template <int D>
constexpr double value_eps_unit_f32() {
  return 1.02 * 1.01 * 1.01 * (68.0 * (4 * (D / 32) + 1) + (2 * D + 2)) / 16777216.0 + 1.02 / 32768.0;
}

template <int D, int VB>
hipError_t launch_vb(const DeviceTables& tb, const void* v, bool bf16, const uint8_t* mod, int hkv,
                     int batch, const WindowSource& src, int64_t t_cap, uint32_t* vc, uint16_t* vs,
                     hipStream_t stream) {
  const int64_t tasks = static_cast<int64_t>(batch) * hkv * src.windows_per_sequence();
  if (tasks > kMaxWindowTasks) return hipErrorInvalidConfiguration;  // the task indices are 32-bit
  const dim3 grid(static_cast<unsigned>((tasks + kWaves - 1) / kWaves));
  if (tb.rot_bf16 != nullptr) {
    // matrix cores, bf16 values as they come or fp32 values as two bf16 parts each
    const double unit = bf16 ? value_eps_unit<D>() : value_eps_unit_f32<D>();
    const float eps = static_cast<float>(unit * tb.rot_col_norm + 1.02 * tb.rot_lo_col_norm);
    const uint4_t* rb = reinterpret_cast<const uint4_t*>(tb.rot_bf16);
    if (bf16 && tb.value_sym)
      quantize_values_mfma_kernel<D, VB, true, false><<<grid, 256, 0, stream>>>(
          v, mod, hkv, src, t_cap, tasks, rb, tb.rotations_t, tb.boundaries, eps, vc, vs);
    else if (bf16)
      quantize_values_mfma_kernel<D, VB, false, false><<<grid, 256, 0, stream>>>(
          v, mod, hkv, src, t_cap, tasks, rb, tb.rotations_t, tb.boundaries, eps, vc, vs);
    else if (tb.value_sym)
      quantize_values_mfma_kernel<D, VB, true, true><<<grid, 256, 0, stream>>>(
          v, mod, hkv, src, t_cap, tasks, rb, tb.rotations_t, tb.boundaries, eps, vc, vs);
    else
      quantize_values_mfma_kernel<D, VB, false, true><<<grid, 256, 0, stream>>>(
          v, mod, hkv, src, t_cap, tasks, rb, tb.rotations_t, tb.boundaries, eps, vc, vs);
  } else if (bf16) {
    quantize_values_kernel<D, VB, true><<<grid, 256, 0, stream>>>(v, mod, hkv, src, t_cap, tasks, tb.rotations,
                                                                  tb.boundaries, vc, vs);
  } else {
    quantize_values_kernel<D, VB, false><<<grid, 256, 0, stream>>>(v, mod, hkv, src, t_cap, tasks, tb.rotations,
                                                                   tb.boundaries, vc, vs);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_values(const Shape& sh, const DeviceTables& tb, const void* v, bool bf16,
                                  const uint8_t* modality, int batch, const WindowSource& src,
                                  int64_t t_cap, uint32_t* vc, uint16_t* vs, hipStream_t stream) {
  if (sh.d == 128 && sh.vbits == 2) return launch_vb<128, 2>(tb, v, bf16, modality, sh.hkv, batch, src, t_cap, vc, vs, stream);
  if (sh.d == 128 && sh.vbits == 4) return launch_vb<128, 4>(tb, v, bf16, modality, sh.hkv, batch, src, t_cap, vc, vs, stream);
  if (sh.d == 64 && sh.vbits == 2) return launch_vb<64, 2>(tb, v, bf16, modality, sh.hkv, batch, src, t_cap, vc, vs, stream);
  return launch_vb<64, 4>(tb, v, bf16, modality, sh.hkv, batch, src, t_cap, vc, vs, stream);
}

}  // namespace omnikv
