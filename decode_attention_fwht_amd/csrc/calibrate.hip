// Host calibration of a modality's value basis U_m ([paper] "OmniKVQuant: KV Cache
// Quantization for Omni-LLMs", §2.3 "Modality-aware value rotation"; [digest]
// "OmniKVQuant：面向 Omni-LLM 的 KV 缓存量化", 方法概览: an attention-contribution-weighted
// covariance, eigendecomposed).
//
//   C = sum_t w_t v_t v_t^T / sum_t w_t      (float64, on the GPU: one partial sum per
//                                             block of tokens, added in block order)
//   C = E diag(lambda) E^T                   (cyclic Jacobi on the host, float64)
//   E: columns in descending eigenvalue order, each column's first largest-magnitude
//      entry made positive
//   U_m = E H_d / sqrt(d)                    (H_d the Sylvester Hadamard matrix)
//
// Offline and blocking: it allocates its partial sums and waits for them.
#include <math.h>
#include <stdio.h>

#include <algorithm>
#include <numeric>
#include <string>
#include <vector>

#include "omnikv_internal.h"

namespace {

constexpr int kCalTokens = 256;   // tokens per block
constexpr int kCalThreads = 256;

// Block x: tokens [x * kCalTokens, ...); thread (i, jg) owns row i and columns jg, jg + 16,
// ... of the block's partial sum, and the weight sum goes to the last slot.
template <int D, typename T>
__global__ __launch_bounds__(kCalThreads) void second_moment_kernel(const T* __restrict__ v,
                                                                    const float* __restrict__ w, int64_t n,
                                                                    double* __restrict__ partial) {
  constexpr int JPT = D * D / kCalThreads;  // entries per thread
  constexpr int JG = kCalThreads / D;       // column groups
  __shared__ double tile[32][D];
  __shared__ double wt[32];
  const int tid = threadIdx.x;
  const int i = tid % D, jg = tid / D;
  double acc[JPT];
#pragma unroll
  for (int x = 0; x < JPT; ++x) acc[x] = 0.0;
  double wsum = 0.0;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kCalTokens;
  for (int c0 = 0; c0 < kCalTokens; c0 += 32) {
    __syncthreads();
    for (int e = tid; e < 32 * D; e += kCalThreads) {
      const int tt = e / D, c = e % D;
      const int64_t t = t0 + c0 + tt;
      double x = 0.0;
      if (t < n) {
        if constexpr (sizeof(T) == 2)
          x = static_cast<double>(__uint_as_float(static_cast<uint32_t>(v[t * D + c]) << 16));
        else
          x = static_cast<double>(v[t * D + c]);
      }
      tile[tt][c] = x;
    }
    if (tid < 32) {
      const int64_t t = t0 + c0 + tid;
      wt[tid] = t < n ? (w ? static_cast<double>(w[t]) : 1.0) : 0.0;
    }
    __syncthreads();
    for (int tt = 0; tt < 32; ++tt) {
      const double a = wt[tt] * tile[tt][i];
#pragma unroll
      for (int x = 0; x < JPT; ++x) acc[x] = fma(a, tile[tt][jg + JG * x], acc[x]);
      if (tid == 0) wsum += wt[tt];
    }
  }
  double* out = partial + static_cast<size_t>(blockIdx.x) * (D * D + 1);
#pragma unroll
  for (int x = 0; x < JPT; ++x) out[i * D + jg + JG * x] = acc[x];
  if (tid == 0) out[D * D] = wsum;
}

// Cyclic Jacobi eigenvalue iteration for a symmetric matrix (Golub & Van Loan, Matrix
// Computations, "The classical Jacobi algorithm" / cyclic-by-row variant): each (p, q)
// rotation zeroes a[p][q]; sweeps repeat until the off-diagonal mass is negligible.
void jacobi_eigen(std::vector<double>& a, int d, std::vector<double>& vecs, std::vector<double>& vals) {
  vecs.assign(static_cast<size_t>(d) * d, 0.0);
  for (int i = 0; i < d; ++i) vecs[static_cast<size_t>(i) * d + i] = 1.0;
  auto A = [&](int r, int c) -> double& { return a[static_cast<size_t>(r) * d + c]; };
  auto V = [&](int r, int c) -> double& { return vecs[static_cast<size_t>(r) * d + c]; };
  double total = 0.0;
  for (double x : a) total += x * x;
  for (int sweep = 0; sweep < 100; ++sweep) {
    double off = 0.0;
    for (int p = 0; p < d; ++p)
      for (int q = p + 1; q < d; ++q) off += A(p, q) * A(p, q);
    if (off <= 1e-30 * total) break;
    for (int p = 0; p < d; ++p)
      for (int q = p + 1; q < d; ++q) {
        const double apq = A(p, q);
        if (apq == 0.0) continue;
        const double theta = (A(q, q) - A(p, p)) / (2.0 * apq);
        const double t = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
        const double c = 1.0 / sqrt(t * t + 1.0), s = t * c;
        for (int k = 0; k < d; ++k) {  // columns p, q of A
          const double akp = A(k, p), akq = A(k, q);
          A(k, p) = c * akp - s * akq;
          A(k, q) = s * akp + c * akq;
        }
        for (int k = 0; k < d; ++k) {  // rows p, q of A
          const double apk = A(p, k), aqk = A(q, k);
          A(p, k) = c * apk - s * aqk;
          A(q, k) = s * apk + c * aqk;
        }
        for (int k = 0; k < d; ++k) {  // eigenvector columns
          const double vkp = V(k, p), vkq = V(k, q);
          V(k, p) = c * vkp - s * vkq;
          V(k, q) = s * vkp + c * vkq;
        }
      }
  }
  vals.resize(d);
  for (int i = 0; i < d; ++i) vals[i] = A(i, i);
}

}  // namespace

namespace omnikv {

// Declared in omnikv_internal.h's consumer (api.hip); returns "" or an error text.
std::string calibrate_value_rotation(const void* values, bool bf16, const float* weights, int64_t n, int d,
                                     float* u_out, hipStream_t stream) {
  const int64_t blocks = (n + kCalTokens - 1) / kCalTokens;
  const size_t per = static_cast<size_t>(d) * d + 1;
  double* partial = nullptr;
  hipError_t e = hipMalloc(&partial, static_cast<size_t>(blocks) * per * sizeof(double));
  if (e != hipSuccess) return std::string("hipMalloc: ") + hipGetErrorString(e);
  const dim3 grid(static_cast<unsigned>(blocks));
  if (d == 128) {
    if (bf16)
      second_moment_kernel<128, uint16_t><<<grid, kCalThreads, 0, stream>>>(static_cast<const uint16_t*>(values), weights, n, partial);
    else
      second_moment_kernel<128, float><<<grid, kCalThreads, 0, stream>>>(static_cast<const float*>(values), weights, n, partial);
  } else {
    if (bf16)
      second_moment_kernel<64, uint16_t><<<grid, kCalThreads, 0, stream>>>(static_cast<const uint16_t*>(values), weights, n, partial);
    else
      second_moment_kernel<64, float><<<grid, kCalThreads, 0, stream>>>(static_cast<const float*>(values), weights, n, partial);
  }
  e = hipGetLastError();
  std::vector<double> host(static_cast<size_t>(blocks) * per);
  if (e == hipSuccess)
    e = hipMemcpyAsync(host.data(), partial, host.size() * sizeof(double), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  (void)hipFree(partial);
  if (e != hipSuccess) return std::string("second moment: ") + hipGetErrorString(e);

  std::vector<double> C(static_cast<size_t>(d) * d, 0.0);
  double wsum = 0.0;
  for (int64_t x = 0; x < blocks; ++x) {
    const double* p = host.data() + static_cast<size_t>(x) * per;
    for (size_t k = 0; k < C.size(); ++k) C[k] += p[k];
    wsum += p[static_cast<size_t>(d) * d];
  }
  if (!(wsum > 0.0)) return "the weights sum to zero";
  for (int i = 0; i < d; ++i)  // the kernel wrote row i from thread i: symmetrize exactly
    for (int j = i; j < d; ++j) {
      const double s = 0.5 * (C[static_cast<size_t>(i) * d + j] + C[static_cast<size_t>(j) * d + i]) / wsum;
      C[static_cast<size_t>(i) * d + j] = C[static_cast<size_t>(j) * d + i] = s;
    }
  std::vector<double> E, lam;
  jacobi_eigen(C, d, E, lam);
  std::vector<int> order(d);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return lam[a] > lam[b]; });
  std::vector<double> Es(static_cast<size_t>(d) * d);
  for (int col = 0; col < d; ++col) {
    const int src = order[col];
    int lead = 0;
    for (int r = 1; r < d; ++r)
      if (fabs(E[static_cast<size_t>(r) * d + src]) > fabs(E[static_cast<size_t>(lead) * d + src])) lead = r;
    const double sg = E[static_cast<size_t>(lead) * d + src] < 0.0 ? -1.0 : 1.0;
    for (int r = 0; r < d; ++r) Es[static_cast<size_t>(r) * d + col] = sg * E[static_cast<size_t>(r) * d + src];
  }
  // U = Es H / sqrt(d), H_kj = (-1)^popcount(k & j)
  const double inv = 1.0 / sqrt(static_cast<double>(d));
  for (int r = 0; r < d; ++r)
    for (int j = 0; j < d; ++j) {
      double s = 0.0;
      for (int k = 0; k < d; ++k) s += Es[static_cast<size_t>(r) * d + k] * ((__builtin_popcount(k & j) & 1) ? -1.0 : 1.0);
      u_out[static_cast<size_t>(r) * d + j] = static_cast<float>(s * inv);
    }
  return "";
}

}  // namespace omnikv
