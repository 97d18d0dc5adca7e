// SPECTRA Group-32 4-bit KV cache for gfx950: quantize on append, attend over
// the quantized cache at decode.
//
// The SPECTRA page (abstract) keeps the key-value cache in microscaled
// Group-32 4-bit form next to the weights.  Each head's key or value vector of
// D = 32G channels is split into G groups of 32 consecutive channels and
// quantized exactly as a bulk weight group: range [min(0, min w), max(0,
// max w)], s16 = fp16((hi - lo) / 15), z = rint(-lo / s16), q = clamp(rint(w /
// s16) + z, 0, 15), all in binary64 on the device, codes in the weight
// container's 16-byte record order.
//
// Device layout of each of the K and V planes, for capacity C tokens and H
// heads: records [C][H][G] (16 bytes), scales [C][H][G] fp16, zero bytes
// [C][H][G/2] (group g's nibble at bits 4 (g % 2)); G is even (D = 64, 128,
// 256), so a byte never spans two vectors.
//
// Attention (one query per head, Hq = rep * H query heads, head h reading
// cache head h / rep), three launches:
//   k_kv_scores  one thread per cached token and cache head: dequantize the
//                key (exact fp16 (q - z) pairs, as in the GEMV), dot it with
//                the rep queries of that head in fp32, times s16 per group,
//                divided by sqrt(D) -> scores [Hq][L] in the workspace;
//   k_kv_pv      per (split of 128 tokens, query head): the split's max m,
//                sum of exp(s - m) and sum_t exp(s_t - m) v_t with
//                lane-per-channel-pair dequantization -> fp32 partials;
//   k_kv_combine rescales the splits to the global max and divides, fp16.
#include "spectra_internal.h"
#include "g32.h"

namespace spectra {
namespace {

constexpr int kGroup32 = 32;
constexpr int kScoreThreads = 256;
constexpr int kPvThreads = 256;
constexpr int kTokensPerSplit = 128;
constexpr int kMaxRep = 16;  // query heads per cache head handled in one pass

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// Quantize the 32 fp16 values at src into one record, its scale and zero.
__device__ void quantize32(const uint16_t* src, uint4& rec, uint16_t& s16, uint32_t& z) {
  uint16_t w[kGroup32];
  const uint4* s4 = reinterpret_cast<const uint4*>(src);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 t = s4[i];
    const uint32_t u[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w[8 * i + 2 * j] = (uint16_t)(u[j] & 0xFFFFu);
      w[8 * i + 2 * j + 1] = (uint16_t)(u[j] >> 16);
    }
  }
  double lo = 0.0, hi = 0.0;
#pragma unroll
  for (int e = 0; e < kGroup32; ++e) {
    const double v = g32_h2d(w[e]);
    lo = v < lo ? v : lo;
    hi = v > hi ? v : hi;
  }
  s16 = f64_to_f16_rne((hi - lo) / 15.0);
  const double sd = g32_h2d(s16);
  uint32_t words[4] = {0u, 0u, 0u, 0u};
  z = 0;
  if (sd > 0.0) {
    double zf = __builtin_rint(-lo / sd);
    if (zf > 15.0) zf = 15.0;
    z = (uint32_t)zf;
#pragma unroll
    for (int e = 0; e < kGroup32; ++e) {
      double qf = __builtin_rint(g32_h2d(w[e]) / sd) + (double)z;
      qf = qf < 0.0 ? 0.0 : (qf > 15.0 ? 15.0 : qf);
      words[e >> 3] |= (uint32_t)qf << member_shift(e);
    }
  }
  rec = make_uint4(words[0], words[1], words[2], words[3]);
}

// One thread per (plane, token, head, pair of groups).
__global__ __launch_bounds__(256) void k_kv_append(const KvView c, const uint16_t* __restrict__ k,
                                                   const uint16_t* __restrict__ v, int64_t T,
                                                   int64_t pos0) {
  const int G = c.G, H = c.H, D = c.D;
  const int64_t pairs = T * H * (G / 2);
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= 2 * pairs) return;
  const int plane = idx >= pairs ? 1 : 0;
  const int64_t r = plane ? idx - pairs : idx;
  const int pr = (int)(r % (G / 2));
  const int64_t th = r / (G / 2);  // token * H + head
  const uint16_t* src = (plane ? v : k) + th * D;
  const KvPlane& pl = plane ? c.v : c.k;
  const int64_t flat0 = (pos0 * H + th) * G + 2 * pr;  // even
  uint32_t zbyte = 0;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    uint4 rec;
    uint16_t s16;
    uint32_t z;
    quantize32(src + (2 * pr + hh) * kGroup32, rec, s16, z);
    pl.codes[flat0 + hh] = rec;
    pl.scales[flat0 + hh] = s16;
    zbyte |= z << (4 * hh);
  }
  pl.zeros[flat0 >> 1] = (uint8_t)zbyte;
}

// Exact fp16 (q - z) pair j (members 2j, 2j + 1 of the word's 8) of code word w.
__device__ __forceinline__ half2_t pair_qz(uint32_t w, int j, uint32_t z) {
  const uint32_t ww = j >= 2 ? w >> 8 : w;
  if (j & 1)
    return as_h2((ww & 0x00F000F0u) | 0x54005400u) - as_h2((0x5400u + (z << 4)) * 0x00010001u);
  return as_h2((ww & 0x000F000Fu) | 0x64006400u) - as_h2((0x6400u + z) * 0x00010001u);
}

// scores[hq][t] = q_hq . k_t / sqrt(D), hq = h * rep + r.
template <int G>
__global__ __launch_bounds__(kScoreThreads) void k_kv_scores(const KvView c, const uint16_t* __restrict__ q,
                                                             int rep, int64_t L, float* __restrict__ scores) {
  constexpr int D = 32 * G;
  __shared__ half2_t qs[kMaxRep][D / 2];
  const int h = blockIdx.y;
  const int H = c.H;
  for (int i = threadIdx.x; i < rep * D / 2; i += blockDim.x) {
    const int rr = i / (D / 2), j = i % (D / 2);
    qs[rr][j] = as_h2(reinterpret_cast<const uint32_t*>(q + (int64_t)(h * rep + rr) * D)[j]);
  }
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= L) return;
  const int64_t flat0 = (t * H + h) * G;
  float acc[kMaxRep];
#pragma unroll
  for (int rr = 0; rr < kMaxRep; ++rr) acc[rr] = 0.f;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint4 rec = c.k.codes[flat0 + g];
    const float sc = h2f(c.k.scales[flat0 + g]);
    const uint32_t z = (c.k.zeros[(flat0 + g) >> 1] >> (4 * (g & 1))) & 0xFu;
    const uint32_t w[4] = {rec.x, rec.y, rec.z, rec.w};
    half2_t wq[16];
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int j = 0; j < 4; ++j) wq[4 * d + j] = pair_qz(w[d], j, z);
#pragma unroll
    for (int rr = 0; rr < kMaxRep; ++rr) {  // unrolled so acc stays in registers
      if (rr < rep) {
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int j = 0; j < 16; j += 2) {
          a0 = __builtin_amdgcn_fdot2(wq[j], qs[rr][16 * g + j], a0, false);
          a1 = __builtin_amdgcn_fdot2(wq[j + 1], qs[rr][16 * g + j + 1], a1, false);
        }
        acc[rr] = __builtin_fmaf(sc, a0 + a1, acc[rr]);
      }
    }
  }
  const float inv_sqrt_d = 1.0f / __builtin_sqrtf((float)D);
#pragma unroll
  for (int rr = 0; rr < kMaxRep; ++rr)
    if (rr < rep) scores[(int64_t)(h * rep + rr) * L + t] = acc[rr] * inv_sqrt_d;
}

__device__ __forceinline__ float block_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float m = red[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) m = fmaxf(m, red[i]);
  return m;
}

__device__ __forceinline__ float block_sum(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) s += red[i];
  return s;
}

// Per (split of the tokens, query head): the split's max score m, l = sum_t
// exp(s_t - m) and the partial sum_t exp(s_t - m) v_t, in fp32.  Lane l of a
// wave owns channel pairs l + 64 i (i < D / 128; lanes < 32 for D = 64); each
// wave takes every WAVES-th token of the split, kUnroll tokens per step with
// all their loads issued before any is used (one step per wave at D <= 128).
template <int G>
__global__ __launch_bounds__(kPvThreads) void k_kv_pv(const KvView c, const float* __restrict__ scores,
                                                      int rep, int64_t L, float* __restrict__ part,
                                                      float* __restrict__ stats) {
  constexpr int D = 32 * G;
  constexpr int NP = D / 2;                   // channel pairs
  constexpr int PL = NP >= 64 ? NP / 64 : 1;  // pairs per lane
  constexpr int WAVES = kPvThreads / 64;
  constexpr int kUnroll = kTokensPerSplit / WAVES / PL;  // 32 tokens per step (16 at D = 256)
  __shared__ float red[WAVES];
  __shared__ float pacc[WAVES][D];
  const int split = blockIdx.x, hq = blockIdx.y;
  const int h = hq / rep, H = c.H;
  const float* srow = scores + (int64_t)hq * L;
  const int64_t t0 = (int64_t)split * kTokensPerSplit;
  const int64_t t1 = t0 + kTokensPerSplit < L ? t0 + kTokensPerSplit : L;
  float m = -INFINITY;
  for (int64_t t = t0 + threadIdx.x; t < t1; t += blockDim.x) m = fmaxf(m, srow[t]);
  m = block_max(m, red);
  float se = 0.f;
  for (int64_t t = t0 + threadIdx.x; t < t1; t += blockDim.x) se += __expf(srow[t] - m);
  se = block_sum(se, red);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float a[PL][2];
#pragma unroll
  for (int i = 0; i < PL; ++i) a[i][0] = a[i][1] = 0.f;
  for (int64_t tb = t0 + wave; tb < t1; tb += (int64_t)WAVES * kUnroll) {
    uint32_t w[kUnroll][PL], zb[kUnroll][PL];
    uint16_t sb[kUnroll][PL];
    float p[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t t = tb + (int64_t)u * WAVES;
      const bool in = t < t1;
      const int64_t flat0 = ((in ? t : t0) * H + h) * G;
      p[u] = in ? srow[t] : -INFINITY;
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int pi = (lane + 64 * i) % NP;  // lanes past NP (D = 64) read a valid pair, unused
        const int g = pi >> 4, e = (2 * pi) & 31;
        w[u][i] = reinterpret_cast<const uint32_t*>(c.v.codes + flat0 + g)[e >> 3];
        sb[u][i] = c.v.scales[flat0 + g];
        zb[u][i] = c.v.zeros[(flat0 + g) >> 1];
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float pu = __expf(p[u] - m);  // 0 for tokens past the split
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int pi = (lane + 64 * i) % NP;
        const int g = pi >> 4, e = (2 * pi) & 31;
        const uint32_t z = (zb[u][i] >> (4 * (g & 1))) & 0xFu;
        const half2_t qz = pair_qz(w[u][i], (e & 7) >> 1, z);
        const float sc = h2f(sb[u][i]);
        a[i][0] = __builtin_fmaf(pu, (float)qz.x * sc, a[i][0]);
        a[i][1] = __builtin_fmaf(pu, (float)qz.y * sc, a[i][1]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const int pi = lane + 64 * i;
    if (pi < NP) {
      pacc[wave][2 * pi] = a[i][0];
      pacc[wave][2 * pi + 1] = a[i][1];
    }
  }
  __syncthreads();
  const int64_t base = (int64_t)split * gridDim.y + hq;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float sum = 0.f;
    for (int w2 = 0; w2 < WAVES; ++w2) sum += pacc[w2][d];
    part[base * D + d] = sum;
  }
  if (threadIdx.x == 0) {
    stats[2 * base] = m;
    stats[2 * base + 1] = se;
  }
}

// out = sum_s exp(m_s - M) O_s / sum_s exp(m_s - M) l_s, M = max_s m_s.  The
// split weights are computed once into LDS; each thread then sums its
// channel over the splits with several loads in flight.
constexpr int kMaxSplits = 4096;
__global__ __launch_bounds__(256) void k_kv_combine(const float* __restrict__ part, const float* __restrict__ stats,
                                                    int splits, int Hq, int D, uint16_t* __restrict__ out) {
  __shared__ float wgt[kMaxSplits];
  __shared__ float red[4];
  const int hq = blockIdx.x;
  float M = -INFINITY;
  for (int sp = threadIdx.x; sp < splits; sp += blockDim.x) M = fmaxf(M, stats[2 * ((int64_t)sp * Hq + hq)]);
  M = block_max(M, red);
  float l = 0.f;
  for (int sp = threadIdx.x; sp < splits; sp += blockDim.x) {
    const int64_t b = (int64_t)sp * Hq + hq;
    const float w = __expf(stats[2 * b] - M);
    wgt[sp] = w;
    l += w * stats[2 * b + 1];
  }
  l = block_sum(l, red);  // its barriers also publish wgt
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int sp = 0;
    for (; sp + 8 <= splits; sp += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[((int64_t)(sp + u) * Hq + hq) * D + d];
#pragma unroll
      for (int u = 0; u < 8; ++u) o[u] = __builtin_fmaf(wgt[sp + u], v[u], o[u]);
    }
    for (; sp < splits; ++sp) o[0] = __builtin_fmaf(wgt[sp], part[((int64_t)sp * Hq + hq) * D + d], o[0]);
    const float tot = ((o[0] + o[1]) + (o[2] + o[3])) + ((o[4] + o[5]) + (o[6] + o[7]));
    out[(int64_t)hq * D + d] = __builtin_bit_cast(uint16_t, (_Float16)(tot / l));
  }
}

int64_t splits_of(int64_t L) { return (L + kTokensPerSplit - 1) / kTokensPerSplit; }

}  // namespace

int64_t kv_max_attend_length() { return (int64_t)kMaxSplits * kTokensPerSplit; }

namespace {

template <int G>
hipError_t attend_g(const KvView& c, const uint16_t* q, int rep, int64_t L, uint16_t* out, void* ws,
                    hipStream_t s) {
  constexpr int D = 32 * G;
  const int Hq = c.H * rep;
  const int64_t splits = splits_of(L);
  float* scores = static_cast<float*>(ws);
  float* part = scores + (size_t)Hq * L;
  float* stats = part + (size_t)splits * Hq * D;
  hipLaunchKernelGGL(k_kv_scores<G>, dim3((unsigned)((L + kScoreThreads - 1) / kScoreThreads), (unsigned)c.H),
                     dim3(kScoreThreads), 0, s, c, q, rep, L, scores);
  hipLaunchKernelGGL(k_kv_pv<G>, dim3((unsigned)splits, (unsigned)Hq), dim3(kPvThreads), 0, s, c, scores, rep, L,
                     part, stats);
  hipLaunchKernelGGL(k_kv_combine, dim3((unsigned)Hq), dim3(D < 256 ? D : 256), 0, s, part, stats, (int)splits,
                     Hq, D, out);
  return hipGetLastError();
}

}  // namespace

size_t kv_attend_workspace_bytes(const KvView& c, int rep, int64_t L) {
  const int64_t Hq = (int64_t)c.H * rep;
  return 4 * (size_t)(Hq * L + splits_of(L) * Hq * (c.D + 2));
}

bool kv_shape_supported(int64_t heads, int64_t head_dim) {
  return heads >= 1 && heads <= 1024 && (head_dim == 64 || head_dim == 128 || head_dim == 256);
}

int kv_max_rep() { return kMaxRep; }

hipError_t launch_kv_append(const KvView& c, const uint16_t* k, const uint16_t* v, int64_t T, int64_t pos0,
                            hipStream_t s) {
  const int64_t threads = 2 * T * c.H * (c.G / 2);
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(k_kv_append, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, c, k, v, T, pos0);
  return hipGetLastError();
}

hipError_t launch_kv_attend(const KvView& c, const uint16_t* q, int rep, int64_t L, uint16_t* out, void* ws,
                            hipStream_t s) {
  switch (c.G) {
    case 2: return attend_g<2>(c, q, rep, L, out, ws, s);
    case 4: return attend_g<4>(c, q, rep, L, out, ws, s);
    case 8: return attend_g<8>(c, q, rep, L, out, ws, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace spectra
