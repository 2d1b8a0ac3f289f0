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
    const void* __restrict__ v, const uint8_t* __restrict__ modality, int hkv, int64_t n,
    int64_t t0, int64_t t_cap, int64_t tasks, const float* __restrict__ rot,
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

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t task = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
  const bool active = task < tasks;
  const int64_t nw = n / kWindow;
  const int64_t b = active ? task / (nw * hkv) : 0;
  const int64_t w = active ? (task / hkv) % nw : 0;
  const int h = active ? static_cast<int>(task % hkv) : 0;
  const int64_t tok0 = t0 + w * kWindow;                       // absolute token of the window
  const size_t blk = (static_cast<size_t>(b) * hkv + h) * (t_cap / kWindow) + tok0 / kWindow;

  if (active) {
#pragma unroll 4
    for (int t = 0; t < kWindow; ++t) {
      const size_t row = ((static_cast<size_t>(b) * n + w * kWindow + t) * hkv + h) * D;
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

constexpr int kMaxFlags = 512;  // near-threshold elements per window handled one by one

template <int D, int VB>
__global__ __launch_bounds__(256) void quantize_values_mfma_kernel(
    const uint16_t* __restrict__ v, const uint8_t* __restrict__ modality, int hkv, int64_t n,
    int64_t t0, int64_t t_cap, int64_t tasks, const uint4_t* __restrict__ rot_b16,
    const float* __restrict__ rot_t, const float* __restrict__ boundaries, float eps_c,
    uint32_t* __restrict__ v_codes, uint16_t* __restrict__ v_scale) {
  constexpr int NC = D / 64;
  constexpr int NCT = D / 16;                 // channel tiles
  constexpr int NKS = D / 32;                 // k-steps
  constexpr int NB = (1 << VB) - 1;           // boundaries
  constexpr int VW = D * VB / 64;             // output words per lane
  constexpr int PPW = 16 / VB;                // code pairs per word
  constexpr int ROW = D + 8;
  __shared__ uint8_t codes_lds[kWaves][kWindow][ROW];
  __shared__ float sig_lds[kWaves][kWindow];
  __shared__ float eps_lds[kWaves][kWindow];
  __shared__ uint8_t tag_lds[kWaves][kWindow];
  __shared__ uint16_t flag_lds[kWaves][kMaxFlags];
  __shared__ int nflag_lds[kWaves];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t task = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
  const bool active = task < tasks;
  const int64_t nw = n / kWindow;
  const int64_t b = active ? task / (nw * hkv) : 0;
  const int64_t w = active ? (task / hkv) % nw : 0;
  const int h = active ? static_cast<int>(task % hkv) : 0;
  const int64_t tok0 = t0 + w * kWindow;
  const size_t blk = (static_cast<size_t>(b) * hkv + h) * (t_cap / kWindow) + tok0 / kWindow;
  const size_t row0 = ((static_cast<size_t>(b) * n + w * kWindow) * hkv + h) * D;  // element of token 0
  const size_t rstride = static_cast<size_t>(hkv) * D;                             // elements per token

  if (active) {
    // ---- tags
    const uint8_t* tagp = modality + static_cast<size_t>(b) * t_cap + tok0;
    uint32_t present = 0u;
    {
      uint32_t tw[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) tw[x] = reinterpret_cast<const uint32_t*>(tagp)[x];
#pragma unroll
      for (int t = 0; t < kWindow; ++t) {
        const uint32_t tg = min((tw[t >> 2] >> (8 * (t & 3))) & 0xFFu, static_cast<uint32_t>(kMaxModalities - 1));
        present |= 1u << tg;
      }
      if (lane < kWindow)
        tag_lds[wave][lane] = static_cast<uint8_t>(
            min((tw[lane >> 2] >> (8 * (lane & 3))) & 0xFFu, static_cast<uint32_t>(kMaxModalities - 1)));
    }
    if (lane == 0) nflag_lds[wave] = 0;

    // ---- per-token scale: stride-halving tree of squares (lane l holds channels l, l + 64).
    // The 32 trees run as one reduce-scatter: the stage across lane bit b (b = 5 .. 1) adds
    // the partner's partial sums for half of the lane's tokens and leaves the other half to
    // the partner, so after five stages lane l holds token l >> 1 alone, and the last stage
    // (bit 0) completes it in both lanes of the pair.  Every sum is the tree's own (each
    // stage adds the same two partial sums as the stride-halving definition), so the result
    // is the definition's exactly; no stage waits on another token's shuffles.
    {
      float x[kWindow][NC];
#pragma unroll
      for (int t = 0; t < kWindow; ++t)
#pragma unroll
        for (int c = 0; c < NC; ++c)
          x[t][c] = __uint_as_float(static_cast<uint32_t>(v[row0 + t * rstride + lane + 64 * c]) << 16);
      float part[kWindow];
      uint32_t nzbits = 0u;  // tokens with a nonzero magnitude bit in this lane (subnormals count)
#pragma unroll
      for (int t = 0; t < kWindow; ++t) {
        part[t] = (NC == 2) ? (x[t][0] * x[t][0] + x[t][1] * x[t][1]) : x[t][0] * x[t][0];
        uint32_t mag = 0u;
#pragma unroll
        for (int c = 0; c < NC; ++c) mag |= __float_as_uint(x[t][c]) & 0x7FFFFFFFu;
        nzbits |= (mag != 0u ? 1u : 0u) << t;
      }
#pragma unroll
      for (int hh = 32; hh >= 1; hh >>= 1) nzbits |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(nzbits), hh, 64));
      // reduce-scatter over lane bits 5 .. 1; part[k] is then the partial sum of token base + k
      int base = 0;
      auto stage = [&](auto st_c) {
        constexpr int st = decltype(st_c)::value, cnt = 1 << (st - 1);
        const bool up = (lane >> st) & 1;
#pragma unroll
        for (int k = 0; k < cnt; ++k) {
          const float give = up ? part[k] : part[cnt + k];
          const float keep = up ? part[cnt + k] : part[k];
          part[k] = keep + __shfl_xor(give, 1 << st, 64);
        }
        base += up ? cnt : 0;
      };
      stage(std::integral_constant<int, 5>{});
      stage(std::integral_constant<int, 4>{});
      stage(std::integral_constant<int, 3>{});
      stage(std::integral_constant<int, 2>{});
      stage(std::integral_constant<int, 1>{});
      const float S = part[0] + __shfl_xor(part[0], 1, 64);  // token base = lane >> 1
      const float sigma = sqrtf(S * (1.0f / static_cast<float>(D)));
      const uint16_t s16 = f16_bits(sigma);
      if ((lane & 1) == 0) {
        const int t = base;
        sig_lds[wave][t] = f16_value(s16);
        eps_lds[wave][t] = ((nzbits >> t) & 1u) ? eps_c * sqrtf(S) + 1e-20f : -1.0f;
        v_scale[(static_cast<size_t>(b) * hkv + h) * t_cap + tok0 + t] = s16;
      }
    }

    // ---- the window as matrix-core A operands: token 16 tt + n, channels 32 ks + 8 g ..
    const int nn = lane & 15, g = lane >> 4;
    uint4_t av[2][NKS];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        av[tt][ks] = *reinterpret_cast<const uint4_t*>(v + row0 + (16 * tt + nn) * rstride + 32 * ks + 8 * g);
    float beta[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) beta[j] = boundaries[j];
    // this lane's result tokens (16 tt + 4 g + i) and their modalities
    uint32_t my_tag[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) my_tag[tt][i] = tag_lds[wave][16 * tt + 4 * g + i];
    // and their scales and tolerances, read once for all channel tiles
    float my_sg[2][4], my_ep[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        my_sg[tt][i] = sig_lds[wave][16 * tt + 4 * g + i];
        my_ep[tt][i] = eps_lds[wave][16 * tt + 4 * g + i];
      }

    // ---- one pass per modality present
#pragma unroll
    for (int m = 0; m < kMaxModalities; ++m) {
      if (!(present & (1u << m))) continue;
      const uint4_t* B = rot_b16 + static_cast<size_t>(m) * 3 * NCT * NKS * 64 + lane;
#pragma unroll 2
      for (int ct = 0; ct < NCT; ++ct) {
        uint4_t bv[2][NKS];
#pragma unroll
        for (int part = 0; part < 2; ++part)
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) bv[part][ks] = B[((part * NCT + ct) * NKS + ks) * 64];
        float4_t acc[2] = {float4_t{0.f, 0.f, 0.f, 0.f}, float4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int part = 0; part < 2; ++part)
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
              acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[tt][ks]),
                                                                __builtin_bit_cast(bf16x8_t, bv[part][ks]), acc[tt], 0, 0, 0);
        const int c = 16 * ct + nn;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (my_tag[tt][i] != static_cast<uint32_t>(m)) continue;
            const int t = 16 * tt + 4 * g + i;
            const float x = acc[tt][i];
            const float sg = my_sg[tt][i], e = my_ep[tt][i];
            int code = 0;
            bool near = false;
#pragma unroll
            for (int j = 0; j < NB; ++j) {
              const float th = sg * beta[j];
              code += (x >= th) ? 1 : 0;
              near = near || !(fabsf(x - th) > e);  // NaN or infinite sums count as near
            }
            codes_lds[wave][t][c] = static_cast<uint8_t>(code);
            if (near) {
              const int idx = atomicAdd(&nflag_lds[wave], 1);
              if (idx < kMaxFlags) flag_lds[wave][idx] = static_cast<uint16_t>((t << 8) | c);
            }
          }
      }
    }

    // ---- the sequential definition for the elements near a threshold
    auto exact_code = [&](int t, int c) {
      const float* ut = rot_t + (static_cast<size_t>(tag_lds[wave][t]) * D + c) * D;
      const uint16_t* vr = v + row0 + t * rstride;
      float s = 0.0f;
      for (int k0 = 0; k0 < D; k0 += 8) {
        const float4 u0 = *reinterpret_cast<const float4*>(ut + k0);
        const float4 u1 = *reinterpret_cast<const float4*>(ut + k0 + 4);
        const uint4_t vb = *reinterpret_cast<const uint4_t*>(vr + k0);
        const float uu[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const uint32_t half = (vb[kk >> 1] >> (16 * (kk & 1))) & 0xFFFFu;
          s = s + uu[kk] * __uint_as_float(half << 16);
        }
      }
      const float sg = sig_lds[wave][t];
      int code = 0;
#pragma unroll
      for (int j = 0; j < NB; ++j) code += (s >= sg * beta[j]) ? 1 : 0;
      codes_lds[wave][t][c] = static_cast<uint8_t>(code);
    };
    const int nf = nflag_lds[wave];
    if (nf <= kMaxFlags) {
      for (int f = lane; f < nf; f += 64) {
        const uint32_t e = flag_lds[wave][f];
        exact_code(static_cast<int>(e >> 8), static_cast<int>(e & 0xFFu));
      }
    } else {
      // too many elements near a threshold (all-zero tokens, say): the whole window by the
      // definition
      for (int e = lane; e < kWindow * D; e += 64) exact_code(e / D, e % D);
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

template <int D, int VB>
hipError_t launch_vb(const DeviceTables& tb, const void* v, bool bf16, const uint8_t* mod, int hkv,
                     int batch, int64_t t0, int64_t n, int64_t t_cap, uint32_t* vc, uint16_t* vs,
                     hipStream_t stream) {
  const int64_t tasks = static_cast<int64_t>(batch) * hkv * (n / kWindow);
  const dim3 grid(static_cast<unsigned>((tasks + kWaves - 1) / kWaves));
  if (bf16 && tb.rot_bf16 != nullptr)
    quantize_values_mfma_kernel<D, VB><<<grid, 256, 0, stream>>>(
        static_cast<const uint16_t*>(v), mod, hkv, n, t0, t_cap, tasks, reinterpret_cast<const uint4_t*>(tb.rot_bf16),
        tb.rotations_t, tb.boundaries,
        static_cast<float>(value_eps_unit<D>() * tb.rot_col_norm + 1.02 * tb.rot_lo_col_norm), vc, vs);
  else if (bf16)
    quantize_values_kernel<D, VB, true><<<grid, 256, 0, stream>>>(v, mod, hkv, n, t0, t_cap, tasks, tb.rotations,
                                                                  tb.boundaries, vc, vs);
  else
    quantize_values_kernel<D, VB, false><<<grid, 256, 0, stream>>>(v, mod, hkv, n, t0, t_cap, tasks, tb.rotations,
                                                                   tb.boundaries, vc, vs);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_values(const Shape& sh, const DeviceTables& tb, const void* v, bool bf16,
                                  const uint8_t* modality, int batch, int64_t t0, int64_t n,
                                  int64_t t_cap, uint32_t* vc, uint16_t* vs, hipStream_t stream) {
  if (sh.d == 128 && sh.vbits == 2) return launch_vb<128, 2>(tb, v, bf16, modality, sh.hkv, batch, t0, n, t_cap, vc, vs, stream);
  if (sh.d == 128 && sh.vbits == 4) return launch_vb<128, 4>(tb, v, bf16, modality, sh.hkv, batch, t0, n, t_cap, vc, vs, stream);
  if (sh.d == 64 && sh.vbits == 2) return launch_vb<64, 2>(tb, v, bf16, modality, sh.hkv, batch, t0, n, t_cap, vc, vs, stream);
  return launch_vb<64, 4>(tb, v, bf16, modality, sh.hkv, batch, t0, n, t_cap, vc, vs, stream);
}

}  // namespace omnikv
