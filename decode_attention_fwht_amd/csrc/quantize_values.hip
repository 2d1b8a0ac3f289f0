// Value write path: per-token RMS scale, rotation by the basis U_m of the
// token's modality ([paper] "OmniKVQuant: KV Cache Quantization for Omni-LLMs",
// §2.3 "Modality-aware value rotation"), then the fixed Lloyd-Max codebook.
//
// One 64-lane wave owns one 32-token window of one (sequence, KV head); lane l
// computes rotated channels l and l + 64 of every token.  The rotation is the
// plain dot product accumulated in index order with every product and sum
// rounded to fp32, so the codes are bit-identical to any implementation of the
// same definition.
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
  __shared__ float vals[kWaves][kWindow][D];
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
      for (int c = 0; c < NC; ++c) vals[wave][t][lane + 64 * c] = load_elem<BF16>(v, row + lane + 64 * c);
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
    for (int t = 0; t < kWindow; ++t) tag[t] = (tw[t >> 2] >> (8 * (t & 3))) & 0xFF;
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
        const float x = vals[wave][t][lane + 64 * c];
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
    if (uniform) {
      const float* U = rot + static_cast<size_t>(tag[0]) * D * D;
      for (int kk = 0; kk < D; ++kk) {
        float u[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) u[c] = U[kk * D + lane + 64 * c];
#pragma unroll
        for (int t = 0; t < kWindow; ++t) {
          const float x = vals[wave][t][kk];
#pragma unroll
          for (int c = 0; c < NC; ++c) acc[t][c] = acc[t][c] + u[c] * x;
        }
      }
    } else {
      for (int kk = 0; kk < D; ++kk) {
        float u[kMaxModalities][NC];
#pragma unroll
        for (int m = 0; m < kMaxModalities; ++m)
#pragma unroll
          for (int c = 0; c < NC; ++c) u[m][c] = rot[(static_cast<size_t>(m) * D + kk) * D + lane + 64 * c];
#pragma unroll
        for (int t = 0; t < kWindow; ++t) {
          const float x = vals[wave][t][kk];
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            const float um = tag[t] == 0 ? u[0][c] : (tag[t] == 1 ? u[1][c] : u[2][c]);
            acc[t][c] = acc[t][c] + um * x;
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

template <int D, int VB>
hipError_t launch_vb(const DeviceTables& tb, const void* v, bool bf16, const uint8_t* mod, int hkv,
                     int batch, int64_t t0, int64_t n, int64_t t_cap, uint32_t* vc, uint16_t* vs,
                     hipStream_t stream) {
  const int64_t tasks = static_cast<int64_t>(batch) * hkv * (n / kWindow);
  const dim3 grid(static_cast<unsigned>((tasks + kWaves - 1) / kWaves));
  if (bf16)
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
