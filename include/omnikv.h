/*
 * omnikv.h -- C ABI of the MI355X (gfx950) OmniKVQuant hot path.
 *
 * OmniKVQuant is a training-free 2-bit KV-cache codec for caches that mix
 * text, audio and video tokens, with a fused decode attention that reads the
 * packed cache directly.  Sources, cited by page title and section:
 *   [paper]    "OmniKVQuant: KV Cache Quantization for Omni-LLMs" (paper text)
 *   [abstract] arXiv listing of the same paper (arXiv:2609.11582), Abstract
 *   [digest]   "OmniKVQuant：面向 Omni-LLM 的 KV 缓存量化" (digest of the paper)
 *
 * Three operations, as the pages state the problem:
 *   omnikv_quantize_keys     keys: randomized Hadamard rotation shared by all
 *                            modalities, then a min-max range per 32-token
 *                            window and rotated channel mapped onto a fixed
 *                            uniform codebook ([abstract] (i); [paper] §1,
 *                            §3.1 Implementation details, §3.3 Error comparison;
 *                            [digest] 方法概览).
 *   omnikv_quantize_values   values: a per-modality orthogonal basis U_m
 *                            ([paper] §2.3 "Modality-aware value rotation"),
 *                            then a fixed Lloyd-Max codebook with a per-token
 *                            scale (the codebook and scale are not printed; see
 *                            the value-codec notes below).
 *   omnikv_decode_attention  one decode step over the packed cache: rotate each
 *                            query once per head, unpack codes in registers,
 *                            online softmax in FlashAttention order, value
 *                            accumulators per modality in rotated space, one
 *                            batched inverse value rotation per head output; no
 *                            dense FP16 cache is built ([paper] §1 and Fig. 1(d);
 *                            [abstract]).
 *
 * Conventions for every call
 *   - Pointers marked "device" are HIP device memory owned by the caller; the
 *     library never frees or retains them.  "host" pointers are read during
 *     the call only.  Device pointers must be 16-byte aligned.
 *   - Every compute call enqueues kernels on `stream` and returns without
 *     synchronizing the host.  Faults inside a kernel surface at the caller's
 *     next synchronization (HIP semantics).
 *   - Argument errors return OMNIKV_EINVAL (or OMNIKV_EUNSUPPORTED for a shape
 *     the kernels do not implement) with a message from omnikv_last_error(),
 *     and launch nothing.  A failed launch returns OMNIKV_EHIP.  NaN or Inf
 *     inputs give undefined codes; they are not checked on the hot path.
 *   - No C++ exception crosses this interface.
 *   - A context is immutable after omnikv_create, so calls on different streams
 *     may run concurrently when their outputs do not overlap.
 *
 * Shapes: B = batch, Hq / Hkv = query / KV heads (G = Hq / Hkv query heads per
 * KV head; query head h reads KV head h / G), d = head dim, T_cap = cache
 * capacity in tokens (a multiple of 32), W = 32 = window.
 *
 * Packed cache (all arrays device, caller-allocated, indexed by absolute
 * token position t in [0, T_cap)):
 *   k_codes  uint32 [B][Hkv][T_cap/32][d*key_bits]     key window blocks
 *   k_min    uint16 [B][Hkv][T_cap/32][d]              fp16 m_gc (bit patterns)
 *   k_scale  uint16 [B][Hkv][T_cap/32][d]              fp16 s_gc
 *            (with key_meta = OMNIKV_META_MXFP4 both are byte records instead,
 *            [B][Hkv][T_cap/32][R], R = omnikv_key_meta_bytes(); see below)
 *   v_codes  uint32 [B][Hkv][T_cap/32][d*value_bits]   value window blocks
 *   v_scale  uint16 [B][Hkv][T_cap]                    fp16 per-token scale
 *   modality uint8  [B][T_cap]                         0 text, 1 audio, 2 video
 *
 * Window-block layouts (the code of window token t in [0,32) and channel c;
 * "bits" is the code width; a block is read by one 64-lane wave, lane
 * l = 16 g + rho owning d*bits/64 consecutive uint32 words):
 *   keys:   tau = t / 16, rho = t % 16, g = c / (d/4), s = (c % (d/4)) / 8,
 *           j = c % 8, i = j / 2, e = j % 2;
 *           (d,bits) = (128,2): word i,          slot 4 tau + s
 *                      (128,4): word 4 tau + i,  slot s
 *                      (64,2):  word i % 2,      slot 4 (i / 2) + 2 tau + s
 *                      (64,4):  word i,          slot 2 tau + s
 *           bit = 16 e + bits * slot inside the lane's word.
 *   values: u = c / 16, rho = c % 16; t < 16: g = t / 4, j = t % 4;
 *           t >= 16: g = (t - 16) / 4, j = 4 + t % 4; pair p = 4 u + j / 2;
 *           word p / (16 / bits), bit 2*bits*(p % (16/bits)) + bits * (j % 2).
 *   These orders put every code where the decode kernel's matrix-core operand
 *   expects it, so unpacking is a mask (keys) or one table read per code pair
 *   (values).
 *
 * Key codec (fp32, fixed order; bit-exact across implementations):
 *   y = c_d * FWHT(D x): z = D x (D = diag(key_signs)); butterfly stages
 *   h = 1, 2, ..., d/2, each (z_i, z_{i+h}) -> (z_i + z_{i+h}, z_i - z_{i+h}) for
 *   i with bit h clear; then one multiply by c_d = fp32(1/sqrt(d)).
 *   Per (b, kv head, window, channel): mn = min_t y + 0, mx = max_t y + 0 (the
 *   "+ 0" makes a zero extreme +0); m = fp16(mn); s = fp16((mx - mn) / L),
 *   L = 2^key_bits - 1, IEEE division, fp16 round-to-nearest-even.
 *   code = #{ j < L : y >= m + s * (j + 1/2) }, the product and the sum each
 *   rounded to fp32 (no fused multiply-add).
 *   Dequantized key: x_hat = R^{-1}(m + s * code), R = c_d H D.
 *
 * MXFP4 key metadata (key_meta = OMNIKV_META_MXFP4; the pages' default format,
 * [paper] §3.1 Implementation details; the fp16 form above is the variant of
 * [paper] §3.3).  The window's vectors mn and (mx - mn) / L (fp32, as above) are
 * each cut into blocks of 32 consecutive channels, OCP microscaling style: a
 * block keeps one E8M0 exponent e = floor(log2 max|x|) - 2, clamped to
 * [-127, 127] (-127 for an all-zero block), stored as the byte e + 127, and 32
 * E2M1 codes, x * 2^-e rounded to the nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6 with
 * ties to the even code (larger magnitudes take 6), the sign of x in bit 3.
 * m and s are the decoded values (E2M1 value * 2^e, exact in fp32); codes and
 * the dequantized key follow from them by the rules above.  One record per
 * (b, kv head, window) and vector: d/2 bytes of codes (channel 2i in the low
 * nibble of byte i), d/32 exponent bytes, zero bytes up to R = 16 *
 * ceil((d/2 + d/32) / 16) (80 bytes at d = 128, 48 at d = 64).  Reading: the
 * pages name the format only; blocks run over the channels of one window.
 * The decode kernel takes m and s as fp16: their decoded values must lie within
 * fp16 range (|x| <= 65504); smaller than 2^-24 they count as zero there.
 *
 * Value codec (fp32, fixed order):
 *   sigma = sqrt(S / d) with S the stride-halving tree sum of v_i^2 (pairs
 *   (i, i + d/2), then (i, i + d/4), ...), stored as fp16 (RNE);
 *   v'_i = sum_k U_m[k][i] v_k for k = 0, 1, ..., d-1, every product and partial
 *   sum rounded to fp32 (U_m of the token's modality m; v' = U_m^T v);
 *   code = #{ j : v' >= fp32(sigma_fp16) * beta_j }, beta_j the fp32 midpoint of
 *   fp16 codebook levels l_j, l_{j+1}.
 *   Dequantized value: v_hat = U_m (sigma_fp16 * l[code]).
 *   A token whose RMS exceeds fp16's largest finite value (65504) gets an infinite
 *   scale; the decode's result over such a token is undefined.  Every finite scale,
 *   subnormals included, is within the decode's range: it keeps each probability
 *   times scale inside fp16's normal range for the tokens that dominate the sums.
 */
#ifndef OMNIKV_H_
#define OMNIKV_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct omnikv_ctx omnikv_ctx;

typedef enum {
  OMNIKV_OK = 0,
  OMNIKV_EINVAL = 1,       /* bad argument: shape, alignment, range, NULL */
  OMNIKV_EUNSUPPORTED = 2, /* valid but not implemented: d, bits, G */
  OMNIKV_EHIP = 3,         /* a HIP runtime call or launch failed */
  OMNIKV_ENOMEM = 4        /* device allocation at create time failed */
} omnikv_status;

typedef enum { OMNIKV_F32 = 0, OMNIKV_BF16 = 1 } omnikv_dtype;

typedef struct {
  int32_t head_dim;       /* d: 64 or 128 */
  int32_t num_q_heads;    /* Hq: a multiple of Hkv, Hq/Hkv <= 8 */
  int32_t num_kv_heads;   /* Hkv >= 1 */
  int32_t key_bits;       /* 2 or 4 */
  int32_t value_bits;     /* 2 or 4 */
  int32_t window;         /* 32 (the key-range group g of [paper] §3.1) */
  int32_t num_modalities; /* M in 1..3: one value rotation per modality */
  int32_t key_meta;       /* OMNIKV_META_FP16 (0) or OMNIKV_META_MXFP4 (1) */
} omnikv_config;

/* Storage of the key range metadata m_gc, s_gc. */
enum { OMNIKV_META_FP16 = 0, OMNIKV_META_MXFP4 = 1 };

/* Create a context.  cfg (host) as above.
 * key_signs (host, int8 [d], each +1 or -1): the diagonal D of the shared
 *   randomized Hadamard rotation R = c_d H D ([paper] §1; [digest] 关联工作).
 * value_rotations (host, fp32 [M][d][d] row-major): U_m, each with orthonormal
 *   columns (max |U^T U - I| <= 1e-3, else OMNIKV_EINVAL); v' = U_m^T v.
 *   Their calibration is offline ([paper] §2.3, §3.1).
 * value_codebook (host, uint16 [2^value_bits] fp16 bit patterns, strictly
 *   ascending) or NULL for the built-in Lloyd-Max levels of N(0,1) rounded to
 *   fp16.
 * On success *out owns device copies of these tables (freed by destroy). */
omnikv_status omnikv_create(const omnikv_config* cfg, const int8_t* key_signs,
                            const float* value_rotations, const uint16_t* value_codebook,
                            omnikv_ctx** out);

/* Destroy a context (NULL is accepted).  The caller must have synchronized
 * every stream that used it. */
omnikv_status omnikv_destroy(omnikv_ctx* ctx);

/* Copy the context's fp16 value codebook (2^value_bits entries) to host memory. */
omnikv_status omnikv_value_codebook(const omnikv_ctx* ctx, uint16_t* levels /* host */);

/* Bytes of k_min (and of k_scale) per (sequence, KV head, window) in the
 * context's metadata format: 2 d for fp16, R for MXFP4 (see above). */
omnikv_status omnikv_key_meta_bytes(const omnikv_ctx* ctx, size_t* bytes /* host */);

/* Quantize keys of tokens [t0, t0+n) of every sequence ([paper] §3.1: 32-token
 * groups; [paper] §3.3: FP16 m_gc and s_gc, or the MXFP4 records of §3.1).
 * k (device): [B][n][Hkv][d] of dtype dt (fp32 or bf16), token-major.
 * t0 % 32 == 0, n % 32 == 0, n > 0, t0 + n <= t_cap, t_cap % 32 == 0, and at
 * most 2^32 - 1 windows per call (batch x Hkv x n / 32; more: OMNIKV_EINVAL).
 * Writes k_codes / k_min / k_scale for windows t0/32 .. (t0+n)/32 - 1 only. */
omnikv_status omnikv_quantize_keys(const omnikv_ctx* ctx, const void* k, omnikv_dtype dt,
                                   int32_t batch, int64_t t0, int64_t n, int64_t t_cap,
                                   uint32_t* k_codes, uint16_t* k_min, uint16_t* k_scale,
                                   hipStream_t stream);

/* Quantize values of tokens [t0, t0+n) ([paper] §2.3: rotation by the basis of
 * the token's modality).  v (device): [B][n][Hkv][d] of dtype dt.
 * modality (device): uint8 [B][t_cap]; entries [t0, t0+n) are read and must be
 * < num_modalities.  Same alignment rules as omnikv_quantize_keys.
 * Writes v_codes for windows t0/32 .. and v_scale for tokens [t0, t0+n). */
omnikv_status omnikv_quantize_values(const omnikv_ctx* ctx, const void* v, omnikv_dtype dt,
                                     const uint8_t* modality, int32_t batch, int64_t t0,
                                     int64_t n, int64_t t_cap, uint32_t* v_codes,
                                     uint16_t* v_scale, hipStream_t stream);

/* Bytes of device workspace omnikv_decode_attention needs for (batch, max_len,
 * num_splits).  num_splits: how many splits of consecutive 32-token windows each
 * (sequence, KV head) is cut into, one partial result each; 0 = the library's
 * choice; larger requests are clamped to what the window count allows (the plan
 * may use fewer).  bytes: host out. */
omnikv_status omnikv_decode_workspace_size(const omnikv_ctx* ctx, int32_t batch, int64_t max_len,
                                           int32_t num_splits, size_t* bytes);

/* One decode step: out[b][h] = sum_t softmax_t(scale * q[b][h] . k_hat_t) v_hat_t
 * over tokens t in [0, seq_lens[b]) of the packed cache, computed in the
 * rotated domains ([paper] §1, Fig. 1(d)); fp32 accumulation.
 * q (device): fp32 [B][Hq][d], post-RoPE queries.
 * seq_lens (device): int32 [B], 0 <= seq_lens[b] <= max_len <= t_cap; every
 *   window touched must hold quantized data.  seq_lens[b] == 0 gives zeros.
 * max_len (host): an upper bound of seq_lens; it sizes the launch.
 * softmax_scale: 0 selects 1/sqrt(d).
 * workspace (device): at least omnikv_decode_workspace_size(..) bytes; its
 *   contents on entry are ignored.  num_splits as for the size query.
 * out (device): fp32 [B][Hq][d]. */
omnikv_status omnikv_decode_attention(const omnikv_ctx* ctx, const float* q, const int32_t* seq_lens,
                                      int32_t batch, int64_t max_len, const uint32_t* k_codes,
                                      const uint16_t* k_min, const uint16_t* k_scale,
                                      const uint32_t* v_codes, const uint16_t* v_scale,
                                      const uint8_t* modality, int64_t t_cap, float softmax_scale,
                                      int32_t num_splits, void* workspace, size_t workspace_bytes,
                                      float* out, hipStream_t stream);

/* The two halves of omnikv_decode_attention, with the same arguments and
 * rules.  omnikv_decode_partial runs the split-KV pass: for every (sequence,
 * KV head, split of consecutive 32-token windows) it writes the running max,
 * the softmax sum and one value accumulator per modality, in rotated space,
 * into the workspace.  omnikv_decode_combine merges those partials with the
 * log-sum-exp rule and applies the batched inverse value rotation
 * out = sum_m U_m A_m ([paper] §1, Fig. 1(d)).  Calling partial then combine on
 * one stream with the same (batch, max_len, num_splits, workspace) gives the
 * result of omnikv_decode_attention; the split lets a caller time, overlap or
 * exchange the partials (they are linear in the inverse rotation). */
omnikv_status omnikv_decode_partial(const omnikv_ctx* ctx, const float* q, const int32_t* seq_lens,
                                    int32_t batch, int64_t max_len, const uint32_t* k_codes,
                                    const uint16_t* k_min, const uint16_t* k_scale,
                                    const uint32_t* v_codes, const uint16_t* v_scale,
                                    const uint8_t* modality, int64_t t_cap, float softmax_scale,
                                    int32_t num_splits, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);
omnikv_status omnikv_decode_combine(const omnikv_ctx* ctx, const int32_t* seq_lens, int32_t batch,
                                    int64_t max_len, int32_t num_splits, const void* workspace,
                                    size_t workspace_bytes, float* out, hipStream_t stream);

/* omnikv_decode_attention for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments without the workspace, which is a static array of the library instead,
 * 12 MiB per GPU, held from the first omnikv_create on that GPU until the process ends.
 * The call allocates nothing.  Steps whose plan needs more workspace than that
 * (omnikv_decode_workspace_size(..) > 12 MiB) return OMNIKV_EINVAL and launch nothing;
 * with the library's default split count (num_splits = 0) every step of at most 512
 * (sequence, KV head) units fits (at most 512 partials of 12 KiB, d = 128).  All calls
 * on one GPU share the array: calls that overlap in time on one GPU
 * (different streams, or different contexts) race and must be ordered by the caller.
 * The array's contents between calls are scratch (nothing is carried over). */
omnikv_status omnikv_decode_attention_noalloc(const omnikv_ctx* ctx, const float* q, const int32_t* seq_lens,
                                              int32_t batch, int64_t max_len, const uint32_t* k_codes,
                                              const uint16_t* k_min, const uint16_t* k_scale,
                                              const uint32_t* v_codes, const uint16_t* v_scale,
                                              const uint8_t* modality, int64_t t_cap, float softmax_scale,
                                              int32_t num_splits, float* out, hipStream_t stream);

/* ---- Streaming generation ([paper] §3.1 Implementation details, captioning:
 * keys are quantized every 128 tokens in groups of 32; values keep a 128-token
 * sliding FP16 window before quantization).
 *
 * A streamed sequence of n tokens is held as the packed cache above plus two
 * rings of recent tokens, k_ring and v_ring [B][ring_cap][Hkv][d] (device, caller-
 * allocated, dtype F32 or BF16, token t at row t % ring_cap, stored as given):
 *   keys   of tokens [0, kp) are packed, kp = 128 * floor(n / 128);
 *   values of tokens [0, vp) are packed, vp = 32 * floor(max(0, n - 128) / 32)
 *   (a value window is quantized once all of its 32 tokens have left the
 *   128-token window; reading: the pages do not say how the sliding window meets
 *   the 32-token packing).  Always vp <= kp <= n and n - vp < 160.
 * ring_cap must be a multiple of 128 in [256, 512]. */

/* kp and vp for a stream of n >= 0 tokens (host arithmetic, no device work). */
omnikv_status omnikv_stream_packed_lengths(int64_t n, int64_t* key_packed, int64_t* value_packed);

/* Appends one token to every sequence of the batch: k_new, v_new (device,
 * [B][Hkv][d] of dtype dt) go to ring row lens[b] % ring_cap, tags_new[b]
 * (device, uint8 [B]) to modality[b][lens[b]].  lens (device int32 [B]) and
 * lens_host (host int64 [B]) both give each sequence's length before the append
 * and must agree; lens_host[b] + 1 <= t_cap.  tags_new and lens need no
 * alignment (the other device pointers do, as everywhere).  Every key group and value window
 * that the new length moves past the schedule's thresholds is then quantized
 * from the rings into the packed cache, with the codes omnikv_quantize_keys /
 * _values give for those rows: one launch appends the tokens, one more launch
 * quantizes the key groups of every sequence that crosses a 128-token threshold,
 * and one more the value windows of every sequence whose value window moves (each
 * made only when some sequence needs it; the kernels read each sequence's length
 * from lens), all on `stream`, so at most three launches per call whatever the
 * batch.  The caller advances its lengths by one afterwards.  Errors as for
 * omnikv_quantize_keys; nothing is launched on an argument error. */
omnikv_status omnikv_stream_append(const omnikv_ctx* ctx, const void* k_new, const void* v_new, omnikv_dtype dt,
                                   const uint8_t* tags_new, const int32_t* lens, const int64_t* lens_host,
                                   int32_t batch, void* k_ring, void* v_ring, int32_t ring_cap, uint32_t* k_codes,
                                   uint16_t* k_min, uint16_t* k_scale, uint32_t* v_codes, uint16_t* v_scale,
                                   uint8_t* modality, int64_t t_cap, hipStream_t stream);

/* Decode attention of streamed sequences: as omnikv_decode_attention over all n =
 * seq_lens[b] tokens, where token t attends with its packed key when t < kp and
 * with its ring key otherwise, and with its packed value when t < vp and its ring
 * value otherwise (ring tokens are not quantized; their values enter in the
 * original space).  The packed prefix [0, vp) runs through the split-KV pass; the
 * recent tokens [vp, n) are scored by one more workgroup per (sequence, KV head) of
 * the same launch, and the second launch merges their partial with the splits'
 * and adds their values after the inverse rotation.  Arguments as for
 * omnikv_decode_attention, plus the rings (ring_dtype F32 or BF16, ring_cap as
 * above, each sequence's recent tokens present in its ring); the workspace size
 * is the one omnikv_decode_workspace_size gives for (batch, max_len,
 * num_splits). */
omnikv_status omnikv_decode_attention_streaming(const omnikv_ctx* ctx, const float* q, const int32_t* seq_lens,
                                                int32_t batch, int64_t max_len, const uint32_t* k_codes,
                                                const uint16_t* k_min, const uint16_t* k_scale,
                                                const uint32_t* v_codes, const uint16_t* v_scale,
                                                const uint8_t* modality, int64_t t_cap, const void* k_ring,
                                                const void* v_ring, omnikv_dtype ring_dtype, int32_t ring_cap,
                                                float softmax_scale, int32_t num_splits, void* workspace,
                                                size_t workspace_bytes, float* out, hipStream_t stream);

/* ---- Calibration of a modality's value basis U_m ([paper] §2.3 "Modality-aware
 * value rotation"; [digest] 方法概览: an attention-contribution-weighted covariance,
 * eigendecomposed).  From one modality's calibration values v_t (device, [n][d] of
 * dtype dt, 16-byte aligned) and optional weights w_t (device fp32 [n], e.g. each
 * token's mean attention probability; NULL = 1):
 *   C = sum_t w_t v_t v_t^T / sum_t w_t, accumulated in float64 on the GPU;
 *   E = its eigenvectors (cyclic Jacobi, float64, host), columns in descending
 *       eigenvalue order, each column's first largest-magnitude entry positive;
 *   U_m = E H_d / sqrt(d), H_d the Sylvester Hadamard matrix (reading of the pages'
 *       "modality-aware correction of the Hadamard rotation"),
 * written to u_out (host, fp32 [d][d] row-major) in the layout omnikv_create takes.
 * Offline: it allocates scratch device memory and synchronizes `stream` before it
 * returns.  OMNIKV_EHIP if the weights sum to zero or a HIP call fails. */
omnikv_status omnikv_calibrate_value_rotation(const void* values, omnikv_dtype dt, const float* weights, int64_t n,
                                              int32_t head_dim, float* u_out, hipStream_t stream);

/* Thread-local text describing the last non-OK status of this thread. */
const char* omnikv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* OMNIKV_H_ */
