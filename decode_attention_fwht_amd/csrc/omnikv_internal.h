// Internal declarations shared by the HIP translation units of libomnikv.
// Not part of the public ABI (include/omnikv.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

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
  // host value: the same for the third bf16 part alone (the part the value quantizer's
  // matrix-core pass leaves out), rounded up
  float rot_lo_col_norm = 0.0f;
  // host value: 2-bit values whose boundaries are (-b, 0, b) exactly (the built-in Gaussian
  // codebook is symmetric); the value quantizer then classifies by sign and magnitude
  bool value_sym = false;  // value boundaries symmetric about 0 (0 in the middle)
};

// Streaming schedule ([paper] §3.1 Implementation details, captioning): after n
// streamed tokens, keys are quantized for the first 128 floor(n / 128) tokens (every
// 128 tokens, in 32-token groups); values stay in a sliding window of the 128 most
// recent tokens and are quantized per 32-token window once all of it has left.
__host__ __device__ inline int64_t stream_key_packed(int64_t n) { return (n / 128) * 128; }
__host__ __device__ inline int64_t stream_value_packed(int64_t n) {
  return (n > 128 ? (n - 128) / kWindow : 0) * kWindow;
}
constexpr int kStreamRecent = 128;  // tokens of the sliding value window
constexpr int kMaxRingCap = 512;    // largest ring of recent tokens

struct Shape {
  int d, hq, hkv, group, kbits, vbits, modalities;
  int mx = 0;  // key range metadata: 0 fp16 vectors, 1 MXFP4 records
};

// Bytes of one MXFP4 metadata record (one vector of one window): d/2 bytes of E2M1
// codes, d/32 exponent bytes, zero padding to a multiple of 16.
__host__ __device__ constexpr int mx_record_bytes(int d) { return (d / 2 + d / 32 + 15) / 16 * 16; }
// Value of MXFP4 element code c (E2M1, sign in bit 3) times 2^e, exact in fp32: codes 0
// and 1 are 0 and 0.5 (subnormal), codes 2..7 are 2^(c/2 - 1) (1 + (c & 1) / 2).
__device__ __forceinline__ float mx_decode(uint32_t c, int e) {
  const uint32_t m = c & 7u;
  const float mag = m < 2u ? 0.5f * static_cast<float>(m)
                           : ldexpf(1.0f + 0.5f * static_cast<float>(m & 1u), static_cast<int>(m >> 1) - 1);
  const float v = ldexpf(mag, e);
  return (c & 8u) ? -v : v;
}
// The fp32 scale 2^(x - 127) of an E8M0 exponent byte x in 0..254 (x = 0: 2^-127).
__device__ __forceinline__ float mx_scale(uint32_t x) {
  return __uint_as_float(x ? (x << 23) : 0x00400000u);
}
// Bytes of k_min (or k_scale) per window in the shape's format.
inline size_t key_meta_bytes(const Shape& sh) {
  return sh.mx ? static_cast<size_t>(mx_record_bytes(sh.d)) : static_cast<size_t>(2 * sh.d);
}

// ---- which window a quantizer task (one wave: one window of one (sequence, KV head))
// takes, and where its tokens come from.  Source tokens are rows of [rows][Hkv][d].
//   dense chunk: the source is [batch][n][Hkv][d]; window w of sequence b covers cache
//     tokens t0 + 32 w .. of b, read from source rows b n + 32 w ..
//   streaming flush: the source is the rings [batch][ring_cap][Hkv][d]; lens[b] (device)
//     is sequence b's length n before an append, and the windows are those the append
//     moves past the schedule (keys: the 4 windows of [kp(n), kp(n + 1)) when it grows;
//     values: the window [vp(n), vp(n + 1)) when it grows), at ring rows t % ring_cap
//     (a 32-token window never wraps: ring_cap is a multiple of 128).  Tasks of sequences
//     that do not flush are inactive.
struct WindowSource {
  const int32_t* flush_lens = nullptr;  // null: dense chunk
  int flush_keys = 0;                   // flush mode: 1 keys, 0 values
  int ring_cap = 0;
  int64_t n = 0, t0 = 0;                // dense chunk
  __host__ __device__ int64_t windows_per_sequence() const {
    return flush_lens ? (flush_keys ? 128 / kWindow : 1) : n / kWindow;
  }
};
struct WindowTask {
  bool active;
  int64_t b;        // sequence
  int h;            // KV head
  int64_t src_row;  // source row of the window's first token
  int64_t tok0;     // cache position of the window's first token
};
// The launchers keep `tasks` below 2^32 (kMaxWindowTasks), so the task's indices come from two
// 32-bit divisions (64-bit ones expand to some 600 scalar instructions ahead of the wave's
// first load; measured, that prologue did not bound the launch).
constexpr int64_t kMaxWindowTasks = int64_t{0xFFFFFFFF};
__device__ inline WindowTask map_window_task(const WindowSource& s, int64_t task, int64_t tasks, int hkv) {
  WindowTask r{task < tasks, 0, 0, 0, 0};
  if (!r.active) return r;
  const uint32_t t = static_cast<uint32_t>(task), H = static_cast<uint32_t>(hkv);
  const uint32_t per = static_cast<uint32_t>(s.windows_per_sequence());
  const uint32_t th = t / H;           // task / hkv
  const uint32_t b = th / per;         // task / (hkv per)
  r.b = b;
  const int64_t w = th - b * per;      // (task / hkv) % per
  r.h = static_cast<int>(t - th * H);  // task % hkv
  if (!s.flush_lens) {
    r.src_row = r.b * s.n + w * kWindow;
    r.tok0 = s.t0 + w * kWindow;
    return r;
  }
  const int64_t n0 = s.flush_lens[r.b];
  const int64_t p0 = s.flush_keys ? stream_key_packed(n0) : stream_value_packed(n0);
  const int64_t p1 = s.flush_keys ? stream_key_packed(n0 + 1) : stream_value_packed(n0 + 1);
  r.active = p1 > p0;
  r.tok0 = p0 + w * kWindow;
  r.src_row = r.b * s.ring_cap + r.tok0 % s.ring_cap;
  return r;
}

// ---- launchers (return hipSuccess or the launch error) -----------------------------------
// src.n and src.t0 describe a dense chunk (batch sequences of src.n tokens from cache
// position src.t0); src.flush_lens selects the streaming flush of `batch` sequences.
hipError_t launch_quantize_keys(const Shape& sh, const DeviceTables& tb, const void* k, bool bf16,
                                int batch, const WindowSource& src, int64_t t_cap, uint32_t* k_codes,
                                uint16_t* k_min, uint16_t* k_scale, hipStream_t stream);

hipError_t launch_quantize_values(const Shape& sh, const DeviceTables& tb, const void* v, bool bf16,
                                  const uint8_t* modality, int batch, const WindowSource& src,
                                  int64_t t_cap, uint32_t* v_codes, uint16_t* v_scale,
                                  hipStream_t stream);

// Split-KV decode: partial results per (sequence, KV head, split) followed by the
// log-sum-exp merge and the batched inverse value rotation.
struct DecodePlan {
  int splits;            // splits (one workgroup each) per (sequence, KV head)
  int windows_per_wave;  // consecutive 32-token windows per wave of a split (splits below split_old)
  size_t workspace_bytes;
  int split_old = 0;     // splits [split_old, splits) take wpw_young windows per wave
  int wpw_young = 0;
};

// stream: the plan of omnikv_decode_attention_streaming (one workgroup per (sequence, KV
// head) more, for the recent tokens)
DecodePlan plan_decode(const Shape& sh, int batch, int64_t max_len, int requested_splits, bool stream = false);

// The recent (unquantized) tokens of streamed sequences: keys of tokens
// [stream_key_packed(n), n) and values of [stream_value_packed(n), n) come from the rings
// (token t at row t % ring_cap); older keys of the recent span come from the packed cache.
struct StreamTail {
  const void* k_ring = nullptr;      // [B][ring_cap][Hkv][d], bf16 or fp32
  const void* v_ring = nullptr;
  bool ring_f32 = false;
  int ring_cap = 0;
};

// tail != nullptr: each sequence's seq_lens value is a streamed length n; the split
// workgroups attend over its value-packed prefix (tokens below stream_value_packed(n)) and
// one more workgroup per (sequence, KV head) over the recent tokens.
hipError_t launch_decode_partial(const Shape& sh, const DeviceTables& tb, const DecodePlan& plan,
                                 const float* q, const int32_t* seq_lens, int batch, int64_t max_len,
                                 const uint32_t* k_codes, const uint16_t* k_min, const uint16_t* k_scale,
                                 const uint32_t* v_codes, const uint16_t* v_scale, const uint8_t* modality,
                                 int64_t t_cap, float softmax_scale, void* workspace, const StreamTail* tail,
                                 hipStream_t stream_handle);

// tail != nullptr: the recent tokens' partial (written by the partial launch) joins the merge.
hipError_t launch_decode_combine(const Shape& sh, const DeviceTables& tb, const DecodePlan& plan,
                                 const int32_t* seq_lens, int batch, const void* workspace, float* out,
                                 const StreamTail* tail, hipStream_t stream);

// Appends one token per sequence to the rings (row lens[b] % ring_cap) and writes its
// modality tag at modality[b][lens[b]]; lens (device) are the lengths before the append.
hipError_t launch_stream_append(const Shape& sh, const void* k_new, const void* v_new, bool f32,
                                const uint8_t* tags_new, const int32_t* lens, int batch, void* k_ring,
                                void* v_ring, int ring_cap, uint8_t* modality, int64_t t_cap, hipStream_t stream);

// U_m from calibration values [n][d] (fp32 or bf16, device) and optional weights [n]
// (device); writes u_out (host, [d][d] row-major) and returns "" or an error text.
// Offline: allocates scratch and synchronizes `stream`.
std::string calibrate_value_rotation(const void* values, bool bf16, const float* weights, int64_t n, int d,
                                     float* u_out, hipStream_t stream);

}  // namespace omnikv
