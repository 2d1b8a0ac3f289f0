// C ABI of libomnikv: contexts, argument validation, built-in codebook, launches.
// The public contract (shapes, layouts, arithmetic, errors) is in include/omnikv.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <string>
#include <vector>

#include <climits>
#include <mutex>

#include "omnikv_internal.h"

// Decode workspace of omnikv_decode_attention_noalloc, for callers that cannot allocate:
// one array per GPU, held until the process ends.  In host code `scratch` only names the
// symbol; its device address comes from hipGetSymbolAddress (per device, kept in
// g_scratch_ptr) and is the only form ever passed to a kernel or runtime call.
constexpr size_t kScratchBytes = size_t{12} << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

struct omnikv_ctx {
  omnikv::Shape sh{};
  omnikv::DeviceTables tb{};
  std::vector<uint16_t> levels;  // fp16 value codebook
  int device = 0;
  void* scratch = nullptr;       // device address of `scratch` on `device`
};

namespace {

thread_local std::string g_error;

omnikv_status fail(omnikv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

omnikv_status hip_fail(hipError_t e, const char* what) {
  return fail(OMNIKV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Device address of `scratch` on `device` (the current device), looked up once per device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_address(int device, void** out) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[device] = p;
  }
  *out = g_scratch_ptr[device];
  return hipSuccess;
}

// Lloyd-Max quantizer of a unit Gaussian with n levels: alternate the midpoint
// condition for the thresholds and the centroid condition for the levels, the
// centroid of N(0,1) on (a, b) being (phi(a) - phi(b)) / (Phi(b) - Phi(a)).
std::vector<double> gaussian_lloyd_max(int n) {
  auto pdf = [](double x) { return std::isinf(x) ? 0.0 : exp(-0.5 * x * x) * 0.3989422804014327; };
  auto cdf = [](double x) { return std::isinf(x) ? (x > 0 ? 1.0 : 0.0) : 0.5 * erfc(-x * 0.7071067811865476); };
  std::vector<double> lv(n), th(n + 1);
  for (int i = 0; i < n; ++i) lv[i] = -2.0 + 4.0 * i / (n - 1);
  for (int it = 0; it < 20000; ++it) {
    th[0] = -INFINITY;
    th[n] = INFINITY;
    for (int i = 1; i < n; ++i) th[i] = 0.5 * (lv[i - 1] + lv[i]);
    double change = 0.0;
    for (int i = 0; i < n; ++i) {
      const double c = (pdf(th[i]) - pdf(th[i + 1])) / (cdf(th[i + 1]) - cdf(th[i]));
      change = std::max(change, fabs(c - lv[i]));
      lv[i] = c;
    }
    if (change < 1e-15) break;
  }
  return lv;
}

uint16_t host_f16_bits(float x) { return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x)); }
float host_f16_value(uint16_t b) { return static_cast<float>(__builtin_bit_cast(_Float16, b)); }

template <typename T>
omnikv_status upload(T** dst, const T* src, size_t count) {
  hipError_t e = hipMalloc(reinterpret_cast<void**>(dst), count * sizeof(T));
  if (e != hipSuccess) return fail(OMNIKV_ENOMEM, "hipMalloc(%zu bytes): %s", count * sizeof(T), hipGetErrorString(e));
  e = hipMemcpy(*dst, src, count * sizeof(T), hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy");
  return OMNIKV_OK;
}

// bf16 of a finite fp32, round to nearest even, and back
uint16_t host_bf16_bits(float x) {
  uint32_t u;
  std::memcpy(&u, &x, sizeof(u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
float host_bf16_value(uint16_t b) {
  const uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, sizeof(f));
  return f;
}

void free_tables(omnikv::DeviceTables& tb) {
  if (tb.signs) (void)hipFree(tb.signs);
  if (tb.rotations) (void)hipFree(tb.rotations);
  if (tb.rotations_t) (void)hipFree(tb.rotations_t);
  if (tb.boundaries) (void)hipFree(tb.boundaries);
  if (tb.pair_table) (void)hipFree(tb.pair_table);
  if (tb.rot_bf16) (void)hipFree(tb.rot_bf16);
  tb = omnikv::DeviceTables{};
}

omnikv_status check_ctx(const omnikv_ctx* ctx) {
  if (!ctx) return fail(OMNIKV_EINVAL, "context is NULL");
  return OMNIKV_OK;
}

omnikv_status check_chunk(int32_t batch, int64_t t0, int64_t n, int64_t t_cap) {
  if (batch <= 0) return fail(OMNIKV_EINVAL, "batch must be positive (got %d)", batch);
  if (t_cap <= 0 || t_cap % omnikv::kWindow) return fail(OMNIKV_EINVAL, "t_cap must be a positive multiple of 32 (got %lld)", (long long)t_cap);
  if (t0 < 0 || t0 % omnikv::kWindow) return fail(OMNIKV_EINVAL, "t0 must be a non-negative multiple of 32 (got %lld)", (long long)t0);
  if (n <= 0 || n % omnikv::kWindow) return fail(OMNIKV_EINVAL, "n must be a positive multiple of 32 (got %lld)", (long long)n);
  if (t0 + n > t_cap) return fail(OMNIKV_EINVAL, "t0 + n = %lld exceeds t_cap = %lld", (long long)(t0 + n), (long long)t_cap);
  return OMNIKV_OK;
}

}  // namespace

extern "C" {

omnikv_status omnikv_create(const omnikv_config* cfg, const int8_t* key_signs, const float* value_rotations,
                            const uint16_t* value_codebook, omnikv_ctx** out) {
  if (!out) return fail(OMNIKV_EINVAL, "out is NULL");
  *out = nullptr;
  if (!cfg || !key_signs || !value_rotations) return fail(OMNIKV_EINVAL, "cfg, key_signs and value_rotations are required");
  const int d = cfg->head_dim;
  if (cfg->window != omnikv::kWindow) return fail(OMNIKV_EUNSUPPORTED, "window must be 32 (got %d)", cfg->window);
  if (d != 64 && d != 128) return fail(OMNIKV_EUNSUPPORTED, "head_dim must be 64 or 128 (got %d)", d);
  if ((cfg->key_bits != 2 && cfg->key_bits != 4) || (cfg->value_bits != 2 && cfg->value_bits != 4))
    return fail(OMNIKV_EUNSUPPORTED, "key_bits and value_bits must be 2 or 4 (got %d, %d)", cfg->key_bits, cfg->value_bits);
  if (cfg->num_kv_heads <= 0 || cfg->num_q_heads <= 0 || cfg->num_q_heads % cfg->num_kv_heads)
    return fail(OMNIKV_EINVAL, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)", cfg->num_q_heads, cfg->num_kv_heads);
  const int group = cfg->num_q_heads / cfg->num_kv_heads;
  if (group > omnikv::kMaxGroup) return fail(OMNIKV_EUNSUPPORTED, "at most 8 query heads per KV head (got %d)", group);
  const int M = cfg->num_modalities;
  if (M < 1 || M > omnikv::kMaxModalities) return fail(OMNIKV_EINVAL, "num_modalities must be 1..3 (got %d)", M);
  if (cfg->key_meta != OMNIKV_META_FP16 && cfg->key_meta != OMNIKV_META_MXFP4)
    return fail(OMNIKV_EINVAL, "key_meta must be OMNIKV_META_FP16 or OMNIKV_META_MXFP4 (got %d)", cfg->key_meta);
  for (int i = 0; i < d; ++i)
    if (key_signs[i] != 1 && key_signs[i] != -1) return fail(OMNIKV_EINVAL, "key_signs[%d] = %d is not +-1", i, key_signs[i]);
  for (int m = 0; m < M; ++m) {
    const float* U = value_rotations + static_cast<size_t>(m) * d * d;
    double worst = 0.0;
    for (int a = 0; a < d; ++a)
      for (int b = a; b < d; ++b) {
        double s = 0.0;
        for (int k = 0; k < d; ++k) s += static_cast<double>(U[k * d + a]) * U[k * d + b];
        worst = std::max(worst, fabs(s - (a == b ? 1.0 : 0.0)));
      }
    if (!(worst <= 1e-3)) return fail(OMNIKV_EINVAL, "value_rotations[%d] is not orthogonal (max |U^T U - I| = %g)", m, worst);
  }
  const int nl = 1 << cfg->value_bits;
  std::vector<uint16_t> levels(nl);
  if (value_codebook) {
    for (int i = 0; i < nl; ++i) levels[i] = value_codebook[i];
    for (int i = 0; i < nl; ++i)
      if (!std::isfinite(host_f16_value(levels[i]))) return fail(OMNIKV_EINVAL, "value_codebook[%d] is not finite", i);
    for (int i = 1; i < nl; ++i)
      if (!(host_f16_value(levels[i]) > host_f16_value(levels[i - 1])))
        return fail(OMNIKV_EINVAL, "value_codebook must be strictly ascending (entry %d)", i);
  } else {
    const std::vector<double> lv = gaussian_lloyd_max(nl);
    for (int i = 0; i < nl; ++i) levels[i] = host_f16_bits(static_cast<float>(lv[i]));
  }

  auto* ctx = new (std::nothrow) omnikv_ctx();
  if (!ctx) return fail(OMNIKV_ENOMEM, "out of host memory");
  ctx->sh = omnikv::Shape{d, cfg->num_q_heads, cfg->num_kv_heads, group, cfg->key_bits, cfg->value_bits, M,
                          cfg->key_meta == OMNIKV_META_MXFP4 ? 1 : 0};
  ctx->levels = levels;
  if (const hipError_t e = hipGetDevice(&ctx->device); e != hipSuccess) {
    delete ctx;
    return hip_fail(e, "hipGetDevice");
  }
  if (const hipError_t e = scratch_address(ctx->device, &ctx->scratch); e != hipSuccess) {
    delete ctx;
    return hip_fail(e, "hipGetSymbolAddress(scratch)");
  }

  std::vector<float> sg(d);
  for (int i = 0; i < d; ++i) sg[i] = static_cast<float>(key_signs[i]);
  // all three rotation slots exist on the device; unused ones repeat U_0
  std::vector<float> rot(static_cast<size_t>(omnikv::kMaxModalities) * d * d);
  for (int m = 0; m < omnikv::kMaxModalities; ++m)
    std::copy(value_rotations + static_cast<size_t>(m < M ? m : 0) * d * d,
              value_rotations + static_cast<size_t>((m < M ? m : 0) + 1) * d * d, rot.begin() + static_cast<size_t>(m) * d * d);
  std::vector<float> rot_t(rot.size());
  for (int m = 0; m < omnikv::kMaxModalities; ++m)
    for (int r = 0; r < d; ++r)
      for (int c = 0; c < d; ++c)
        rot_t[(static_cast<size_t>(m) * d + c) * d + r] = rot[(static_cast<size_t>(m) * d + r) * d + c];
  std::vector<float> bnd(nl - 1);
  for (int j = 0; j + 1 < nl; ++j) bnd[j] = (host_f16_value(levels[j]) + host_f16_value(levels[j + 1])) / 2.0f;
  const int np = 1 << (2 * cfg->value_bits);
  std::vector<uint32_t> pairs(np);
  for (int idx = 0; idx < np; ++idx)
    pairs[idx] = static_cast<uint32_t>(levels[idx & (nl - 1)]) | (static_cast<uint32_t>(levels[idx >> cfg->value_bits]) << 16);

  // three-part bf16 split of every U_m in the value quantizer's operand order
  // (exact for every entry that is zero or of magnitude above 2^-100: each part keeps the
  // next 8 significant bits, and the residuals are fp32-exact; checked below, and a
  // split with a remainder or a subnormal part disables it)
  const int nct = d / 16, nks = d / 32;
  std::vector<uint16_t> rb16(static_cast<size_t>(omnikv::kMaxModalities) * 3 * nct * nks * 64 * 8);
  bool split_exact = true;
  for (int m = 0; m < omnikv::kMaxModalities; ++m)
    for (int ct = 0; ct < nct; ++ct)
      for (int ks = 0; ks < nks; ++ks)
        for (int lane = 0; lane < 64; ++lane)
          for (int i = 0; i < 8; ++i) {
            const int c = 16 * ct + (lane & 15), k = 32 * ks + 8 * (lane >> 4) + i;
            float r = rot[(static_cast<size_t>(m) * d + k) * d + c];
            for (int part = 0; part < 3; ++part) {
              const uint16_t bits = host_bf16_bits(r);
              const bool subnormal = (bits & 0x7F80u) == 0 && (bits & 0x7Fu) != 0;
              if (subnormal || (bits & 0x7F80u) == 0x7F80u) split_exact = false;
              r = r - host_bf16_value(bits);
              rb16[(((((static_cast<size_t>(m) * 3 + part) * nct + ct) * nks + ks) * 64 + lane) * 8) + i] = bits;
            }
            if (r != 0.0f) split_exact = false;
          }
  double col_norm = 0.0;
  for (int m = 0; m < omnikv::kMaxModalities; ++m)
    for (int c = 0; c < d; ++c) {
      double s2 = 0.0;
      for (int k = 0; k < d; ++k) {
        const double u = rot[(static_cast<size_t>(m) * d + k) * d + c];
        s2 += u * u;
      }
      col_norm = std::max(col_norm, std::sqrt(s2));
    }
  if (!std::isfinite(col_norm)) split_exact = false;
  ctx->tb.rot_col_norm = static_cast<float>(col_norm * (1.0 + 1e-6));
  double lo_norm = 0.0;  // largest column norm of the third part
  for (int m = 0; m < omnikv::kMaxModalities; ++m)
    for (int ct = 0; ct < nct; ++ct)
      for (int n = 0; n < 16; ++n) {
        double s2 = 0.0;
        for (int ks = 0; ks < nks; ++ks)
          for (int g = 0; g < 4; ++g)
            for (int i = 0; i < 8; ++i) {
              const double u = host_bf16_value(rb16[(((((static_cast<size_t>(m) * 3 + 2) * nct + ct) * nks + ks) * 64 + 16 * g + n) * 8) + i]);
              s2 += u * u;
            }
        lo_norm = std::max(lo_norm, std::sqrt(s2));
      }
  ctx->tb.rot_lo_col_norm = static_cast<float>(lo_norm * (1.0 + 1e-6));
  // a symmetric codebook (boundaries -b_k .. -b_1, 0, b_1 .. b_k, as the built-in Lloyd-Max
  // tables are) lets the value quantizer classify by sign and magnitude
  {
    const int nb = nl - 1, mid = nb / 2;
    bool sym = bnd[mid] == 0.0f;
    for (int j = 1; j <= mid; ++j) sym = sym && bnd[mid - j] == -bnd[mid + j];
    ctx->tb.value_sym = sym;
  }

  omnikv_status st;
  if ((st = upload(&ctx->tb.signs, sg.data(), sg.size())) != OMNIKV_OK ||
      (split_exact && (st = upload(&ctx->tb.rot_bf16, rb16.data(), rb16.size())) != OMNIKV_OK) ||
      (st = upload(&ctx->tb.rotations, rot.data(), rot.size())) != OMNIKV_OK ||
      (st = upload(&ctx->tb.rotations_t, rot_t.data(), rot_t.size())) != OMNIKV_OK ||
      (st = upload(&ctx->tb.boundaries, bnd.data(), bnd.size())) != OMNIKV_OK ||
      (st = upload(&ctx->tb.pair_table, pairs.data(), pairs.size())) != OMNIKV_OK) {
    free_tables(ctx->tb);
    delete ctx;
    return st;
  }
  *out = ctx;
  return OMNIKV_OK;
}

omnikv_status omnikv_destroy(omnikv_ctx* ctx) {
  if (!ctx) return OMNIKV_OK;
  free_tables(ctx->tb);
  delete ctx;
  return OMNIKV_OK;
}

omnikv_status omnikv_value_codebook(const omnikv_ctx* ctx, uint16_t* levels) {
  if (check_ctx(ctx) != OMNIKV_OK) return OMNIKV_EINVAL;
  if (!levels) return fail(OMNIKV_EINVAL, "levels is NULL");
  std::copy(ctx->levels.begin(), ctx->levels.end(), levels);
  return OMNIKV_OK;
}

omnikv_status omnikv_key_meta_bytes(const omnikv_ctx* ctx, size_t* bytes) {
  omnikv_status st;
  if ((st = check_ctx(ctx)) != OMNIKV_OK) return st;
  if (!bytes) return fail(OMNIKV_EINVAL, "key_meta_bytes: bytes is NULL");
  *bytes = omnikv::key_meta_bytes(ctx->sh);
  return OMNIKV_OK;
}

omnikv_status omnikv_quantize_keys(const omnikv_ctx* ctx, const void* k, omnikv_dtype dt, int32_t batch,
                                   int64_t t0, int64_t n, int64_t t_cap, uint32_t* k_codes, uint16_t* k_min,
                                   uint16_t* k_scale, hipStream_t stream) {
  omnikv_status st;
  if ((st = check_ctx(ctx)) != OMNIKV_OK) return st;
  if (!k || !k_codes || !k_min || !k_scale) return fail(OMNIKV_EINVAL, "quantize_keys: NULL device pointer");
  if (!aligned16(k) || !aligned16(k_codes) || !aligned16(k_min) || !aligned16(k_scale))
    return fail(OMNIKV_EINVAL, "quantize_keys: device pointers must be 16-byte aligned");
  if (dt != OMNIKV_F32 && dt != OMNIKV_BF16) return fail(OMNIKV_EINVAL, "quantize_keys: dtype must be F32 or BF16");
  if ((st = check_chunk(batch, t0, n, t_cap)) != OMNIKV_OK) return st;
  if (static_cast<int64_t>(batch) * ctx->sh.hkv * (n / omnikv::kWindow) > omnikv::kMaxWindowTasks)
    return fail(OMNIKV_EINVAL, "quantize_keys: one call covers at most 2^32 - 1 windows (batch x KV heads x n / 32)");
  omnikv::WindowSource src;
  src.n = n;
  src.t0 = t0;
  const hipError_t e = omnikv::launch_quantize_keys(ctx->sh, ctx->tb, k, dt == OMNIKV_BF16, batch, src, t_cap,
                                                    k_codes, k_min, k_scale, stream);
  if (e != hipSuccess) return hip_fail(e, "quantize_keys launch");
  return OMNIKV_OK;
}

omnikv_status omnikv_quantize_values(const omnikv_ctx* ctx, const void* v, omnikv_dtype dt, const uint8_t* modality,
                                     int32_t batch, int64_t t0, int64_t n, int64_t t_cap, uint32_t* v_codes,
                                     uint16_t* v_scale, hipStream_t stream) {
  omnikv_status st;
  if ((st = check_ctx(ctx)) != OMNIKV_OK) return st;
  if (!v || !modality || !v_codes || !v_scale) return fail(OMNIKV_EINVAL, "quantize_values: NULL device pointer");
  if (!aligned16(v) || !aligned16(modality) || !aligned16(v_codes) || !aligned16(v_scale))
    return fail(OMNIKV_EINVAL, "quantize_values: device pointers must be 16-byte aligned");
  if (dt != OMNIKV_F32 && dt != OMNIKV_BF16) return fail(OMNIKV_EINVAL, "quantize_values: dtype must be F32 or BF16");
  if ((st = check_chunk(batch, t0, n, t_cap)) != OMNIKV_OK) return st;
  if (static_cast<int64_t>(batch) * ctx->sh.hkv * (n / omnikv::kWindow) > omnikv::kMaxWindowTasks)
    return fail(OMNIKV_EINVAL, "quantize_values: one call covers at most 2^32 - 1 windows (batch x KV heads x n / 32)");
  omnikv::WindowSource src;
  src.n = n;
  src.t0 = t0;
  const hipError_t e = omnikv::launch_quantize_values(ctx->sh, ctx->tb, v, dt == OMNIKV_BF16, modality, batch, src,
                                                      t_cap, v_codes, v_scale, stream);
  if (e != hipSuccess) return hip_fail(e, "quantize_values launch");
  return OMNIKV_OK;
}

omnikv_status omnikv_decode_workspace_size(const omnikv_ctx* ctx, int32_t batch, int64_t max_len, int32_t num_splits,
                                           size_t* bytes) {
  omnikv_status st;
  if ((st = check_ctx(ctx)) != OMNIKV_OK) return st;
  if (!bytes) return fail(OMNIKV_EINVAL, "bytes is NULL");
  if (batch <= 0) return fail(OMNIKV_EINVAL, "batch must be positive (got %d)", batch);
  if (max_len < 0) return fail(OMNIKV_EINVAL, "max_len must be >= 0");
  if (num_splits < 0) return fail(OMNIKV_EINVAL, "num_splits must be >= 0");
  *bytes = omnikv::plan_decode(ctx->sh, batch, max_len, num_splits).workspace_bytes;
  return OMNIKV_OK;
}

}  // extern "C"

namespace {

omnikv_status check_decode(const omnikv_ctx* ctx, int32_t batch, int64_t max_len, int64_t t_cap, int32_t num_splits,
                           size_t workspace_bytes, omnikv::DecodePlan* plan, bool stream = false) {
  if (batch <= 0) return fail(OMNIKV_EINVAL, "batch must be positive (got %d)", batch);
  if (t_cap <= 0 || t_cap % omnikv::kWindow) return fail(OMNIKV_EINVAL, "t_cap must be a positive multiple of 32");
  if (max_len < 0 || max_len > t_cap) return fail(OMNIKV_EINVAL, "max_len must be in [0, t_cap] (got %lld)", (long long)max_len);
  if (num_splits < 0) return fail(OMNIKV_EINVAL, "num_splits must be >= 0");
  {
    // the decode kernel addresses a (sequence, KV head)'s code blocks with 32-bit offsets
    const int64_t bits = ctx->sh.kbits > ctx->sh.vbits ? ctx->sh.kbits : ctx->sh.vbits;
    if (t_cap / omnikv::kWindow * (4 * static_cast<int64_t>(ctx->sh.d) * bits) > INT32_MAX)
      return fail(OMNIKV_EUNSUPPORTED, "t_cap %lld too large: one KV head's code blocks must stay below 2 GiB",
                  (long long)t_cap);
  }
  *plan = omnikv::plan_decode(ctx->sh, batch, max_len, num_splits, stream);
  if (workspace_bytes < plan->workspace_bytes)
    return fail(OMNIKV_EINVAL, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, plan->workspace_bytes);
  return OMNIKV_OK;
}

omnikv_status decode_partial(const omnikv_ctx* ctx, const float* q, const int32_t* seq_lens, int32_t batch,
                             int64_t max_len, const uint32_t* k_codes, const uint16_t* k_min, const uint16_t* k_scale,
                             const uint32_t* v_codes, const uint16_t* v_scale, const uint8_t* modality, int64_t t_cap,
                             float softmax_scale, int32_t num_splits, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  omnikv_status st;
  if ((st = check_ctx(ctx)) != OMNIKV_OK) return st;
  if (!q || !seq_lens || !k_codes || !k_min || !k_scale || !v_codes || !v_scale || !modality || !workspace)
    return fail(OMNIKV_EINVAL, "decode: NULL device pointer");
  const void* ptrs[] = {q, seq_lens, k_codes, k_min, k_scale, v_codes, v_scale, modality, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(OMNIKV_EINVAL, "decode: device pointers must be 16-byte aligned");
  if (!(softmax_scale >= 0.0f) || std::isinf(softmax_scale)) return fail(OMNIKV_EINVAL, "softmax_scale must be finite and >= 0");
  omnikv::DecodePlan plan;
  if ((st = check_decode(ctx, batch, max_len, t_cap, num_splits, workspace_bytes, &plan)) != OMNIKV_OK) return st;
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf(static_cast<float>(ctx->sh.d));
  const hipError_t e = omnikv::launch_decode_partial(ctx->sh, ctx->tb, plan, q, seq_lens, batch, max_len, k_codes, k_min,
                                                     k_scale, v_codes, v_scale, modality, t_cap, scale, workspace,
                                                     nullptr, stream);
  if (e != hipSuccess) return hip_fail(e, "decode_partial launch");
  return OMNIKV_OK;
}

omnikv_status decode_combine(const omnikv_ctx* ctx, const int32_t* seq_lens, int32_t batch, int64_t max_len,
                             int32_t num_splits, const void* workspace, size_t workspace_bytes, float* out,
                             hipStream_t stream) {
  omnikv_status st;
  if ((st = check_ctx(ctx)) != OMNIKV_OK) return st;
  if (!seq_lens || !workspace || !out) return fail(OMNIKV_EINVAL, "decode_combine: NULL device pointer");
  if (!aligned16(seq_lens) || !aligned16(workspace) || !aligned16(out))
    return fail(OMNIKV_EINVAL, "decode_combine: device pointers must be 16-byte aligned");
  omnikv::DecodePlan plan;
  if ((st = check_decode(ctx, batch, max_len, max_len > 0 ? ((max_len + 31) / 32) * 32 : 32, num_splits,
                         workspace_bytes, &plan)) != OMNIKV_OK)
    return st;
  const hipError_t e =
      omnikv::launch_decode_combine(ctx->sh, ctx->tb, plan, seq_lens, batch, workspace, out, nullptr, stream);
  if (e != hipSuccess) return hip_fail(e, "decode_combine launch");
  return OMNIKV_OK;
}

}  // namespace

extern "C" {

omnikv_status omnikv_decode_partial(const omnikv_ctx* ctx, const float* q, const int32_t* seq_lens, int32_t batch,
                                    int64_t max_len, const uint32_t* k_codes, const uint16_t* k_min,
                                    const uint16_t* k_scale, const uint32_t* v_codes, const uint16_t* v_scale,
                                    const uint8_t* modality, int64_t t_cap, float softmax_scale, int32_t num_splits,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_partial(ctx, q, seq_lens, batch, max_len, k_codes, k_min, k_scale, v_codes, v_scale, modality, t_cap,
                        softmax_scale, num_splits, workspace, workspace_bytes, stream);
}

omnikv_status omnikv_decode_combine(const omnikv_ctx* ctx, const int32_t* seq_lens, int32_t batch, int64_t max_len,
                                    int32_t num_splits, const void* workspace, size_t workspace_bytes, float* out,
                                    hipStream_t stream) {
  return decode_combine(ctx, seq_lens, batch, max_len, num_splits, workspace, workspace_bytes, out, stream);
}

omnikv_status omnikv_decode_attention(const omnikv_ctx* ctx, const float* q, const int32_t* seq_lens, int32_t batch,
                                      int64_t max_len, const uint32_t* k_codes, const uint16_t* k_min,
                                      const uint16_t* k_scale, const uint32_t* v_codes, const uint16_t* v_scale,
                                      const uint8_t* modality, int64_t t_cap, float softmax_scale, int32_t num_splits,
                                      void* workspace, size_t workspace_bytes, float* out, hipStream_t stream) {
  if (!out) return fail(OMNIKV_EINVAL, "decode_attention: NULL device pointer");
  if (!aligned16(out)) return fail(OMNIKV_EINVAL, "decode_attention: device pointers must be 16-byte aligned");
  const omnikv_status st = decode_partial(ctx, q, seq_lens, batch, max_len, k_codes, k_min, k_scale, v_codes, v_scale,
                                          modality, t_cap, softmax_scale, num_splits, workspace, workspace_bytes, stream);
  if (st != OMNIKV_OK) return st;
  return decode_combine(ctx, seq_lens, batch, max_len, num_splits, workspace, workspace_bytes, out, stream);
}

omnikv_status omnikv_stream_packed_lengths(int64_t n, int64_t* key_packed, int64_t* value_packed) {
  if (n < 0) return fail(OMNIKV_EINVAL, "stream length must be >= 0 (got %lld)", (long long)n);
  if (!key_packed || !value_packed) return fail(OMNIKV_EINVAL, "stream_packed_lengths: NULL output");
  *key_packed = omnikv::stream_key_packed(n);
  *value_packed = omnikv::stream_value_packed(n);
  return OMNIKV_OK;
}

omnikv_status omnikv_stream_append(const omnikv_ctx* ctx, const void* k_new, const void* v_new, omnikv_dtype dt,
                                   const uint8_t* tags_new, const int32_t* lens, const int64_t* lens_host,
                                   int32_t batch, void* k_ring, void* v_ring, int32_t ring_cap, uint32_t* k_codes,
                                   uint16_t* k_min, uint16_t* k_scale, uint32_t* v_codes, uint16_t* v_scale,
                                   uint8_t* modality, int64_t t_cap, hipStream_t stream) {
  omnikv_status st;
  if ((st = check_ctx(ctx)) != OMNIKV_OK) return st;
  if (dt != OMNIKV_F32 && dt != OMNIKV_BF16) return fail(OMNIKV_EINVAL, "stream_append: dtype must be F32 or BF16");
  if (batch <= 0) return fail(OMNIKV_EINVAL, "batch must be positive (got %d)", batch);
  if (!k_new || !v_new || !tags_new || !lens || !lens_host || !k_ring || !v_ring || !k_codes || !k_min || !k_scale ||
      !v_codes || !v_scale || !modality)
    return fail(OMNIKV_EINVAL, "stream_append: NULL pointer");
  // (tags_new and lens are read one element per sequence and need no alignment)
  const void* ptrs[] = {k_new, v_new, k_ring, v_ring, k_codes, k_min, k_scale, v_codes, v_scale, modality};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(OMNIKV_EINVAL, "stream_append: device pointers must be 16-byte aligned");
  if (ring_cap < omnikv::kStreamRecent + omnikv::kWindow || ring_cap % omnikv::kStreamRecent || ring_cap > omnikv::kMaxRingCap)
    return fail(OMNIKV_EINVAL, "ring_cap must be a multiple of 128 in [256, 512] (got %d)", ring_cap);
  if (t_cap <= 0 || t_cap % omnikv::kWindow) return fail(OMNIKV_EINVAL, "t_cap must be a positive multiple of 32");
  for (int32_t b = 0; b < batch; ++b)
    if (lens_host[b] < 0 || lens_host[b] + 1 > t_cap)
      return fail(OMNIKV_EINVAL, "stream_append: sequence %d has %lld tokens; the cache holds %lld", b,
                  (long long)lens_host[b], (long long)t_cap);
  const omnikv::Shape& sh = ctx->sh;
  const bool f32 = dt == OMNIKV_F32;
  hipError_t e = omnikv::launch_stream_append(sh, k_new, v_new, f32, tags_new, lens, batch, k_ring, v_ring, ring_cap,
                                              modality, t_cap, stream);
  if (e != hipSuccess) return hip_fail(e, "stream_append launch");
  // the key groups and value windows this append moves past the schedule's thresholds are
  // quantized from the rings: one launch for every sequence's keys and one for every
  // sequence's values (the kernels read each sequence's length from `lens` and leave the
  // sequences that do not flush alone), each launched only if some sequence flushes
  bool any_k = false, any_v = false;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t n0 = lens_host[b];
    any_k = any_k || omnikv::stream_key_packed(n0 + 1) > omnikv::stream_key_packed(n0);
    any_v = any_v || omnikv::stream_value_packed(n0 + 1) > omnikv::stream_value_packed(n0);
  }
  omnikv::WindowSource src;
  src.flush_lens = lens;
  src.ring_cap = ring_cap;
  if (any_k) {
    src.flush_keys = 1;
    e = omnikv::launch_quantize_keys(sh, ctx->tb, k_ring, !f32, batch, src, t_cap, k_codes, k_min, k_scale, stream);
    if (e != hipSuccess) return hip_fail(e, "stream_append key flush");
  }
  if (any_v) {
    src.flush_keys = 0;
    e = omnikv::launch_quantize_values(sh, ctx->tb, v_ring, !f32, modality, batch, src, t_cap, v_codes, v_scale,
                                       stream);
    if (e != hipSuccess) return hip_fail(e, "stream_append value flush");
  }
  return OMNIKV_OK;
}

omnikv_status omnikv_decode_attention_noalloc(const omnikv_ctx* ctx, const float* q, const int32_t* seq_lens,
                                              int32_t batch, int64_t max_len, const uint32_t* k_codes,
                                              const uint16_t* k_min, const uint16_t* k_scale, const uint32_t* v_codes,
                                              const uint16_t* v_scale, const uint8_t* modality, int64_t t_cap,
                                              float softmax_scale, int32_t num_splits, float* out, hipStream_t stream) {
  omnikv_status st;
  if ((st = check_ctx(ctx)) != OMNIKV_OK) return st;
  if (!ctx->scratch) return fail(OMNIKV_EHIP, "decode_attention_noalloc: no scratch address for device %d", ctx->device);
  if (batch <= 0) return fail(OMNIKV_EINVAL, "batch must be positive (got %d)", batch);
  if (max_len < 0) return fail(OMNIKV_EINVAL, "max_len must be >= 0 (got %lld)", (long long)max_len);
  if (num_splits < 0) return fail(OMNIKV_EINVAL, "num_splits must be >= 0");
  const size_t need = omnikv::plan_decode(ctx->sh, batch, max_len, num_splits).workspace_bytes;
  if (need > kScratchBytes)
    return fail(OMNIKV_EINVAL,
                "decode_attention_noalloc: this step needs %zu bytes of workspace, the static scratch holds %zu; "
                "use omnikv_decode_attention with a caller workspace (or fewer splits)",
                need, kScratchBytes);
  return omnikv_decode_attention(ctx, q, seq_lens, batch, max_len, k_codes, k_min, k_scale, v_codes, v_scale, modality,
                                 t_cap, softmax_scale, num_splits, ctx->scratch, kScratchBytes, out, stream);
}

omnikv_status omnikv_decode_attention_streaming(const omnikv_ctx* ctx, const float* q, const int32_t* seq_lens,
                                                int32_t batch, int64_t max_len, const uint32_t* k_codes,
                                                const uint16_t* k_min, const uint16_t* k_scale,
                                                const uint32_t* v_codes, const uint16_t* v_scale,
                                                const uint8_t* modality, int64_t t_cap, const void* k_ring,
                                                const void* v_ring, omnikv_dtype ring_dtype, int32_t ring_cap,
                                                float softmax_scale, int32_t num_splits, void* workspace,
                                                size_t workspace_bytes, float* out, hipStream_t stream) {
  omnikv_status st;
  if ((st = check_ctx(ctx)) != OMNIKV_OK) return st;
  if (!q || !seq_lens || !k_codes || !k_min || !k_scale || !v_codes || !v_scale || !modality || !k_ring || !v_ring ||
      !workspace || !out)
    return fail(OMNIKV_EINVAL, "decode_attention_streaming: NULL device pointer");
  const void* ptrs[] = {q, seq_lens, k_codes, k_min, k_scale, v_codes, v_scale, modality, k_ring, v_ring, workspace, out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(OMNIKV_EINVAL, "decode_attention_streaming: device pointers must be 16-byte aligned");
  if (ring_dtype != OMNIKV_F32 && ring_dtype != OMNIKV_BF16)
    return fail(OMNIKV_EINVAL, "decode_attention_streaming: ring dtype must be F32 or BF16");
  if (ring_cap < omnikv::kStreamRecent + omnikv::kWindow || ring_cap % omnikv::kStreamRecent || ring_cap > omnikv::kMaxRingCap)
    return fail(OMNIKV_EINVAL, "ring_cap must be a multiple of 128 in [256, 512] (got %d)", ring_cap);
  if (!(softmax_scale >= 0.0f) || std::isinf(softmax_scale)) return fail(OMNIKV_EINVAL, "softmax_scale must be finite and >= 0");
  omnikv::DecodePlan plan;
  if ((st = check_decode(ctx, batch, max_len, t_cap, num_splits, workspace_bytes, &plan, true)) != OMNIKV_OK) return st;
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf(static_cast<float>(ctx->sh.d));
  omnikv::StreamTail tail;
  tail.k_ring = k_ring;
  tail.v_ring = v_ring;
  tail.ring_f32 = ring_dtype == OMNIKV_F32;
  tail.ring_cap = ring_cap;
  hipError_t e = omnikv::launch_decode_partial(ctx->sh, ctx->tb, plan, q, seq_lens, batch, max_len, k_codes, k_min,
                                               k_scale, v_codes, v_scale, modality, t_cap, scale, workspace, &tail,
                                               stream);
  if (e != hipSuccess) return hip_fail(e, "decode_partial launch");
  e = omnikv::launch_decode_combine(ctx->sh, ctx->tb, plan, seq_lens, batch, workspace, out, &tail, stream);
  if (e != hipSuccess) return hip_fail(e, "decode_combine launch");
  return OMNIKV_OK;
}

omnikv_status omnikv_calibrate_value_rotation(const void* values, omnikv_dtype dt, const float* weights, int64_t n,
                                              int32_t head_dim, float* u_out, hipStream_t stream) {
  if (head_dim != 64 && head_dim != 128) return fail(OMNIKV_EUNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  if (dt != OMNIKV_F32 && dt != OMNIKV_BF16) return fail(OMNIKV_EINVAL, "calibrate: dtype must be F32 or BF16");
  if (n <= 0) return fail(OMNIKV_EINVAL, "calibrate: n must be positive (got %lld)", (long long)n);
  if (!values || !u_out) return fail(OMNIKV_EINVAL, "calibrate: NULL pointer");
  if (!aligned16(values)) return fail(OMNIKV_EINVAL, "calibrate: values must be 16-byte aligned");
  const std::string err = omnikv::calibrate_value_rotation(values, dt == OMNIKV_BF16, weights, n, head_dim, u_out, stream);
  if (!err.empty()) return fail(OMNIKV_EHIP, "calibrate: %s", err.c_str());
  return OMNIKV_OK;
}

const char* omnikv_last_error(void) { return g_error.c_str(); }

}  // extern "C"
