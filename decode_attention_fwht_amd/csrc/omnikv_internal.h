// Internal declarations shared by the HIP translation units of libomnikv.
// Not part of the public ABI (include/omnikv.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "omnikv.h"

namespace omnikv {

constexpr int kWindow = 32;
constexpr int kMaxGroup = 8;       // query heads per KV head handled by one wave
constexpr int kMaxModalities = 3;

// Device-resident, immutable tables owned by a context.
struct DeviceTables {
  float* signs = nullptr;          // [d] +-1.0f, the diagonal D of R = c_d H D
  float* rotations = nullptr;      // [M][d][d] row-major U_m
  float* rotations_t = nullptr;    // [M][d][d] U_m transposed (Ut[m][k][c] = U[m][c][k])
  float* boundaries = nullptr;     // [2^vb - 1] fp32 midpoints of fp16 levels
  uint32_t* pair_table = nullptr;  // [4^vb] fp16 level pairs: (l[lo code], l[hi code])
  // U_m as three bf16 parts (hi + mid + lo == U_m exactly), in the matrix-core operand
  // order of the value quantizer: [3 modalities][3 parts][d/16 channel tiles][d/32 k-steps]
  // [64 lanes][8] (lane 16 g + n: channel 16 ct + n, rows k = 32 ks + 8 g .. + 7)
  // (null when some U_m does not split exactly; the sequential kernel is used then)
  uint16_t* rot_bf16 = nullptr;
  // host value: the largest column norm max_{m,c} ||U_m e_c||_2, which bounds the sum of
  // |U_m[k][c] v_k| over k by that times ||v||_2
  float rot_col_norm = 1.0f;
};

struct Shape {
  int d, hq, hkv, group, kbits, vbits, modalities;
};

// ---- launchers (return hipSuccess or the launch error) -----------------------------------
hipError_t launch_quantize_keys(const Shape& sh, const DeviceTables& tb, const void* k, bool bf16,
                                int batch, int64_t t0, int64_t n, int64_t t_cap, uint32_t* k_codes,
                                uint16_t* k_min, uint16_t* k_scale, hipStream_t stream);

hipError_t launch_quantize_values(const Shape& sh, const DeviceTables& tb, const void* v, bool bf16,
                                  const uint8_t* modality, int batch, int64_t t0, int64_t n,
                                  int64_t t_cap, uint32_t* v_codes, uint16_t* v_scale,
                                  hipStream_t stream);

// Split-KV decode: partial results per (sequence, KV head, split) followed by the
// log-sum-exp merge and the batched inverse value rotation.
struct DecodePlan {
  int splits;            // splits (one workgroup each) per (sequence, KV head)
  int windows_per_wave;  // consecutive 32-token windows per wave of a split
  size_t workspace_bytes;
};

DecodePlan plan_decode(const Shape& sh, int batch, int64_t max_len, int requested_splits);

hipError_t launch_decode_partial(const Shape& sh, const DeviceTables& tb, const DecodePlan& plan,
                                 const float* q, const int32_t* seq_lens, int batch, int64_t max_len,
                                 const uint32_t* k_codes, const uint16_t* k_min, const uint16_t* k_scale,
                                 const uint32_t* v_codes, const uint16_t* v_scale, const uint8_t* modality,
                                 int64_t t_cap, float softmax_scale, void* workspace, hipStream_t stream);

hipError_t launch_decode_combine(const Shape& sh, const DeviceTables& tb, const DecodePlan& plan,
                                 const int32_t* seq_lens, int batch, const void* workspace, float* out,
                                 hipStream_t stream);

}  // namespace omnikv
