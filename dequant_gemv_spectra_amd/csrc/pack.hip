// SPECTRA packer for gfx950: the kurtosis split, the Group-32 asymmetric
// 4-bit quantizer and the container layout, all as device kernels.
//
// Method: SPECTRA page ("SPECTRA: Sparse-Precision Exact Channel Tensor
// Reconstruction Architecture"), abstract -- saliency from the upstream norm
// gain, a fourth-moment test with threshold 3.0, exact floating-point storage
// for heavy-tailed channels, microscaled Group-32 4-bit codes with bit-packed
// zero points for the rest.  The formulas, rounding and layout are the
// library's own reading and are written out in include/spectra.h.
//
// Built with -ffp-contract=off: every binary64 product and sum below is
// rounded on its own, as the written steps state.
#include "spectra_internal.h"
#include "g32.h"

namespace spectra {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ double h2d(uint16_t b) { return g32_h2d(b); }
__device__ __forceinline__ bool finite16(uint16_t b) { return (b & 0x7C00u) != 0x7C00u; }

// Rows per partial sum: aim for about 2^20 threads over the K x chunks grid.
__host__ __device__ inline int64_t rows_per_chunk(int64_t K, int64_t N) {
  int64_t want_chunks = (int64_t)(1 << 20) / (K > 0 ? K : 1);
  if (want_chunks < 1) want_chunks = 1;
  int64_t max_chunks = (N + 63) / 64;
  if (max_chunks > 65535) max_chunks = 65535;  // grid.y limit
  if (want_chunks > max_chunks) want_chunks = max_chunks;
  if (want_chunks < 1) want_chunks = 1;
  return (N + want_chunks - 1) / want_chunks;
}

// Pass 1: partial sums of s = W[n][k] * gamma[k] over a chunk of rows, in row
// order; flags any non-finite W or gamma.
__global__ __launch_bounds__(kThreads) void k_colsum(const uint16_t* __restrict__ W,
                                                     const uint16_t* __restrict__ gamma,
                                                     int64_t K, int64_t N, int64_t R,
                                                     double* __restrict__ psum,
                                                     uint32_t* __restrict__ status) {
  const int64_t k = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t c = blockIdx.y;
  if (k >= K) return;
  const uint16_t gb = gamma[k];
  bool bad = (c == 0) && !finite16(gb);
  const double g = h2d(gb);
  const int64_t n0 = c * R;
  const int64_t n1 = (n0 + R < N) ? n0 + R : N;
  double acc = 0.0;
  for (int64_t n = n0; n < n1; ++n) {
    const uint16_t wb = W[n * K + k];
    bad |= !finite16(wb);
    acc += h2d(wb) * g;
  }
  psum[c * K + k] = acc;
  if (bad) atomicOr(status, 1u);
}

// Column means from the chunk partials (chunks summed in order).
__global__ __launch_bounds__(kThreads) void k_colmean(const double* __restrict__ psum, int64_t K,
                                                      int64_t N, int64_t chunks,
                                                      double* __restrict__ mean) {
  const int64_t k = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (k >= K) return;
  double acc = 0.0;
  for (int64_t c = 0; c < chunks; ++c) acc += psum[c * K + k];
  mean[k] = acc / (double)N;
}

// Pass 2: partial sums of d^2 and (d^2)^2 with d = s - mean.
__global__ __launch_bounds__(kThreads) void k_colmoments(const uint16_t* __restrict__ W,
                                                         const uint16_t* __restrict__ gamma,
                                                         const double* __restrict__ mean,
                                                         int64_t K, int64_t N, int64_t R,
                                                         double* __restrict__ pm2,
                                                         double* __restrict__ pm4) {
  const int64_t k = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t c = blockIdx.y;
  if (k >= K) return;
  const double g = h2d(gamma[k]);
  const double mu = mean[k];
  const int64_t n0 = c * R;
  const int64_t n1 = (n0 + R < N) ? n0 + R : N;
  double a2 = 0.0, a4 = 0.0;
  for (int64_t n = n0; n < n1; ++n) {
    const double s = h2d(W[n * K + k]) * g;
    const double d = s - mu;
    const double d2 = d * d;
    a2 += d2;
    a4 += d2 * d2;
  }
  pm2[c * K + k] = a2;
  pm4[c * K + k] = a4;
}

// Excess kurtosis and the mask words (one ballot per wave of 64 channels).
__global__ __launch_bounds__(kThreads) void k_colflag(const double* __restrict__ pm2,
                                                      const double* __restrict__ pm4, int64_t K,
                                                      int64_t N, int64_t chunks,
                                                      uint32_t* __restrict__ mask_words) {
  const int64_t k = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  bool flag = false;
  if (k < K) {
    double a2 = 0.0, a4 = 0.0;
    for (int64_t c = 0; c < chunks; ++c) {
      a2 += pm2[c * K + k];
      a4 += pm4[c * K + k];
    }
    const double m2 = a2 / (double)N;
    const double m4 = a4 / (double)N;
    flag = (m2 > 0.0) && (m4 / (m2 * m2) - 3.0 > 3.0);
  }
  const uint64_t bal = __ballot(flag);
  const int lane = threadIdx.x & 63;
  const int64_t base = k - lane;  // first channel of this wave
  if (lane == 0 && base < K) mask_words[base >> 5] = (uint32_t)bal;
  if (lane == 32 && base + 32 < K) mask_words[(base >> 5) + 1] = (uint32_t)(bal >> 32);
}

// perm: bulk channels ascending, then heavy-tailed ascending.  One block; each
// thread owns a contiguous channel range, ranges are offset by a serial scan.
__global__ __launch_bounds__(1024) void k_perm(const uint32_t* __restrict__ mask_words, int64_t K,
                                               int64_t K_b, int32_t* __restrict__ perm) {
  __shared__ int64_t bulk_before[1024];
  const int t = threadIdx.x;
  const int64_t chunk = (K + 1023) / 1024;
  const int64_t k0 = ((int64_t)t * chunk < K) ? (int64_t)t * chunk : K;
  const int64_t k1 = (k0 + chunk < K) ? k0 + chunk : K;
  int64_t nb = 0;
  for (int64_t k = k0; k < k1; ++k) nb += !((mask_words[k >> 5] >> (k & 31)) & 1u);
  bulk_before[t] = nb;
  __syncthreads();
  if (t == 0) {
    int64_t run = 0;
    for (int i = 0; i < 1024; ++i) {
      const int64_t v = bulk_before[i];
      bulk_before[i] = run;
      run += v;
    }
  }
  __syncthreads();
  int64_t bpos = bulk_before[t];
  int64_t opos = K_b + (k0 - bulk_before[t]);
  for (int64_t k = k0; k < k1; ++k) {
    if ((mask_words[k >> 5] >> (k & 31)) & 1u) perm[opos++] = (int32_t)k;
    else perm[bpos++] = (int32_t)k;
  }
}

// Quantize two consecutive flat groups per thread (they share a zero byte).
__global__ __launch_bounds__(kThreads) void k_quantize(const uint16_t* __restrict__ W, int64_t K,
                                                       int64_t NG, int32_t G, int32_t K_b,
                                                       const int32_t* __restrict__ perm,
                                                       uint4* __restrict__ codes,
                                                       uint16_t* __restrict__ scales,
                                                       uint8_t* __restrict__ zeros) {
  const int64_t pr = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (2 * pr >= NG) return;
  uint32_t zbyte = 0;
  for (int h = 0; h < 2; ++h) {
    const int64_t i = 2 * pr + h;
    if (i >= NG) break;
    const int64_t n = i / G;
    const int32_t g = (int32_t)(i - n * G);
    const uint16_t* row = W + n * K;
    const int32_t j0 = g * kGroup;
    const int32_t cnt = (K_b - j0 < kGroup) ? K_b - j0 : kGroup;
    double lo = 0.0, hi = 0.0;
    for (int e = 0; e < cnt; ++e) {
      const double w = h2d(row[perm[j0 + e]]);
      lo = w < lo ? w : lo;
      hi = w > hi ? w : hi;
    }
    const double s = (hi - lo) / 15.0;
    const uint16_t s16 = f64_to_f16_rne(s);
    const double sd = h2d(s16);
    uint32_t z = 0;
    uint32_t words[4] = {0u, 0u, 0u, 0u};
    if (sd > 0.0) {
      double zf = __builtin_rint(-lo / sd);
      if (zf > 15.0) zf = 15.0;
      z = (uint32_t)zf;
      for (int e = 0; e < kGroup; ++e) {
        uint32_t q = z;
        if (e < cnt) {
          double qf = __builtin_rint(h2d(row[perm[j0 + e]]) / sd) + (double)z;
          qf = qf < 0.0 ? 0.0 : (qf > 15.0 ? 15.0 : qf);
          q = (uint32_t)qf;
        }
        words[e >> 3] |= q << member_shift(e);
      }
    }
    codes[i] = make_uint4(words[0], words[1], words[2], words[3]);
    scales[i] = s16;
    zbyte |= z << (4 * h);
  }
  zeros[pr] = (uint8_t)zbyte;
}

__global__ __launch_bounds__(kThreads) void k_outliers(const uint16_t* __restrict__ W, int64_t K,
                                                       int64_t N, int32_t K_b, int32_t n_out,
                                                       const int32_t* __restrict__ perm,
                                                       uint16_t* __restrict__ O) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= N * (int64_t)n_out) return;
  const int64_t n = idx / n_out;
  const int32_t j = (int32_t)(idx - n * n_out);
  O[idx] = W[n * K + perm[K_b + j]];
}

inline unsigned grid1(int64_t work) { return (unsigned)((work + kThreads - 1) / kThreads); }

}  // namespace

uint64_t kurtosis_scratch_bytes(int64_t K, int64_t N) {
  const int64_t R = rows_per_chunk(K, N);
  const int64_t chunks = (N + R - 1) / R;
  return 8ull * (uint64_t)K * (uint64_t)(3 * chunks + 1);
}

hipError_t launch_kurtosis(const uint16_t* W, const uint16_t* gamma, int64_t K, int64_t N,
                           void* scratch, uint32_t* status_out, hipStream_t s) {
  const int64_t R = rows_per_chunk(K, N);
  const int64_t chunks = (N + R - 1) / R;
  double* psum = static_cast<double*>(scratch);
  double* pm2 = psum + chunks * K;
  double* pm4 = pm2 + chunks * K;
  double* mean = pm4 + chunks * K;
  const dim3 g2(grid1(K), (unsigned)chunks);
  hipLaunchKernelGGL(k_colsum, g2, dim3(kThreads), 0, s, W, gamma, K, N, R, psum, status_out);
  hipLaunchKernelGGL(k_colmean, dim3(grid1(K)), dim3(kThreads), 0, s, psum, K, N, chunks, mean);
  hipLaunchKernelGGL(k_colmoments, g2, dim3(kThreads), 0, s, W, gamma, mean, K, N, R, pm2, pm4);
  hipLaunchKernelGGL(k_colflag, dim3(grid1(K)), dim3(kThreads), 0, s, pm2, pm4, K, N, chunks,
                     status_out + 1);
  return hipGetLastError();
}

hipError_t launch_quantize(const uint16_t* W, const spectra_container* c, hipStream_t s) {
  unsigned char* base = c->dev;
  const uint32_t* mask_words = reinterpret_cast<const uint32_t*>(base + c->lay.mask);
  int32_t* perm = reinterpret_cast<int32_t*>(base + c->lay.perm);
  hipLaunchKernelGGL(k_perm, dim3(1), dim3(1024), 0, s, mask_words, c->K, c->K_b, perm);
  const int64_t NG = c->N * c->G;
  if (NG > 0) {
    hipLaunchKernelGGL(k_quantize, dim3(grid1((NG + 1) / 2)), dim3(kThreads), 0, s, W, c->K, NG,
                       (int32_t)c->G, (int32_t)c->K_b, perm,
                       reinterpret_cast<uint4*>(base + c->lay.codes),
                       reinterpret_cast<uint16_t*>(base + c->lay.scales),
                       reinterpret_cast<uint8_t*>(base + c->lay.zeros));
  }
  if (c->n_out > 0) {
    hipLaunchKernelGGL(k_outliers, dim3(grid1(c->N * c->n_out)), dim3(kThreads), 0, s, W, c->K,
                       c->N, (int32_t)c->K_b, (int32_t)c->n_out, perm,
                       reinterpret_cast<uint16_t*>(base + c->lay.outliers));
  }
  return hipGetLastError();
}

}  // namespace spectra
