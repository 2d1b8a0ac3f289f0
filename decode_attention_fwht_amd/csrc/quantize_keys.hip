// Key write path: shared randomized Hadamard rotation, then one min-max range
// per (KV head, 32-token window, rotated channel) mapped onto the fixed uniform
// codebook {0, ..., 2^bits - 1}.
//   [paper] "OmniKVQuant: KV Cache Quantization for Omni-LLMs", §1 Introduction
//   (TurboQuant's rotation; temporal key drift), §3.1 Implementation details
//   (32-token groups), §3.3 Error comparison (m_gc, s_gc in FP16).
//
// One 64-lane wave owns one window of one (sequence, KV head).  Lane l holds
// channels l and l + 64 of every token, so the per-channel min/max over the
// window never leaves the lane; the Hadamard stages h < 64 cross lanes.  The
// fp32 operations follow the documented order exactly, so codes and metadata
// are bit-identical to any implementation of the same definition.
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

template <int D, int KB, bool BF16>
__global__ __launch_bounds__(256) void quantize_keys_kernel(
    const void* __restrict__ k, int hkv, int64_t n, int64_t w0, int64_t nwin_cap,
    int64_t tasks, const float* __restrict__ signs, uint32_t* __restrict__ k_codes,
    uint16_t* __restrict__ k_min, uint16_t* __restrict__ k_scale) {
  constexpr int NC = D / 64;                 // channels per lane
  constexpr int L = (1 << KB) - 1;           // largest code
  constexpr int KW = D * KB / 64;            // output words per lane
  constexpr int NS = D / 32;                 // K-steps of the decode operand
  constexpr int ROW = D + 8;                 // padded LDS row (bytes)
  __shared__ uint8_t codes_lds[kWavesPerBlock][kWindow][ROW];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t task = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave;
  const bool active = task < tasks;
  const int64_t nw = n / kWindow;
  // task -> (b, window, head), heads fastest so a block reads adjacent token rows
  const int64_t b = active ? task / (nw * hkv) : 0;
  const int64_t w = active ? (task / hkv) % nw : 0;
  const int h = active ? static_cast<int>(task % hkv) : 0;
  const size_t blk = (static_cast<size_t>(b) * hkv + h) * nwin_cap + w0 + w;

  if (active) {
    float sg[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) sg[c] = signs[lane + 64 * c];
    float y[kWindow][NC];
    float mn[NC], mx[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      mn[c] = INFINITY;
      mx[c] = -INFINITY;
    }
#pragma unroll
    for (int t = 0; t < kWindow; ++t) {
      const size_t row = ((static_cast<size_t>(b) * n + w * kWindow + t) * hkv + h) * D;
      float z[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) z[c] = load_elem<BF16>(k, row + lane + 64 * c) * sg[c];
      // butterfly stages h = 1 .. 32 across lanes: lower index keeps a + b, upper gets a - b
#pragma unroll
      for (int hh = 1; hh < 64; hh <<= 1) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const float p = __shfl_xor(z[c], hh, 64);
          z[c] = (lane & hh) ? (p - z[c]) : (z[c] + p);
        }
      }
      if constexpr (NC == 2) {  // stage h = 64 inside the lane
        const float a0 = z[0] + z[1];
        const float a1 = z[0] - z[1];
        z[0] = a0;
        z[1] = a1;
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const float yy = z[c] * RhtConst<D>::value;
        y[t][c] = yy;
        mn[c] = fminf(mn[c], yy);
        mx[c] = fmaxf(mx[c], yy);
      }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const float lo = mn[c] + 0.0f;  // a zero extreme is +0
      const float hi = mx[c] + 0.0f;
      const float step = (hi - lo) / static_cast<float>(L);
      const uint16_t m16 = f16_bits(lo), s16 = f16_bits(step);
      k_min[blk * D + lane + 64 * c] = m16;
      k_scale[blk * D + lane + 64 * c] = s16;
      const float mf = f16_value(m16), sf = f16_value(s16);
      float th[L];
#pragma unroll
      for (int j = 0; j < L; ++j) th[j] = mf + sf * (static_cast<float>(j) + 0.5f);
#pragma unroll
      for (int t = 0; t < kWindow; ++t) {
        int code = 0;
#pragma unroll
        for (int j = 0; j < L; ++j) code += (y[t][c] >= th[j]) ? 1 : 0;
        codes_lds[wave][t][lane + 64 * c] = static_cast<uint8_t>(code);
      }
    }
  }
  __syncthreads();
  if (!active) return;
  // pack: lane = 16 g + rho holds tokens rho, rho + 16 of channels g*D/4 + 8 s + j
  const int rho = lane & 15, g = lane >> 4;
  uint32_t words[KW];
#pragma unroll
  for (int x = 0; x < KW; ++x) words[x] = 0u;
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint2 eight = *reinterpret_cast<const uint2*>(&codes_lds[wave][16 * tau + rho][g * (D / 4) + 8 * s]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t code = ((j < 4 ? eight.x : eight.y) >> (8 * (j & 3))) & 0xFFu;
        int lw, bit;
        key_slot<D, KB>(tau, s, j, lw, bit);
        words[lw] |= code << bit;
      }
    }
  }
  uint32_t* dst = k_codes + blk * (D * KB) + lane * KW;
#pragma unroll
  for (int x = 0; x < KW; x += 2) *reinterpret_cast<uint2*>(dst + x) = make_uint2(words[x], words[x + 1]);
}

template <int D, int KB>
hipError_t launch_kb(const DeviceTables& tb, const void* k, bool bf16, int hkv, int batch, int64_t t0,
                     int64_t n, int64_t t_cap, uint32_t* kc, uint16_t* km, uint16_t* ks,
                     hipStream_t stream) {
  const int64_t tasks = static_cast<int64_t>(batch) * hkv * (n / kWindow);
  const dim3 grid(static_cast<unsigned>((tasks + kWavesPerBlock - 1) / kWavesPerBlock));
  if (bf16)
    quantize_keys_kernel<D, KB, true><<<grid, 256, 0, stream>>>(k, hkv, n, t0 / kWindow, t_cap / kWindow,
                                                                tasks, tb.signs, kc, km, ks);
  else
    quantize_keys_kernel<D, KB, false><<<grid, 256, 0, stream>>>(k, hkv, n, t0 / kWindow, t_cap / kWindow,
                                                                 tasks, tb.signs, kc, km, ks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_keys(const Shape& sh, const DeviceTables& tb, const void* k, bool bf16,
                                int batch, int64_t t0, int64_t n, int64_t t_cap, uint32_t* kc,
                                uint16_t* km, uint16_t* ks, hipStream_t stream) {
  if (sh.d == 128 && sh.kbits == 2) return launch_kb<128, 2>(tb, k, bf16, sh.hkv, batch, t0, n, t_cap, kc, km, ks, stream);
  if (sh.d == 128 && sh.kbits == 4) return launch_kb<128, 4>(tb, k, bf16, sh.hkv, batch, t0, n, t_cap, kc, km, ks, stream);
  if (sh.d == 64 && sh.kbits == 2) return launch_kb<64, 2>(tb, k, bf16, sh.hkv, batch, t0, n, t_cap, kc, km, ks, stream);
  return launch_kb<64, 4>(tb, k, bf16, sh.hkv, batch, t0, n, t_cap, kc, km, ks, stream);
}

}  // namespace omnikv
