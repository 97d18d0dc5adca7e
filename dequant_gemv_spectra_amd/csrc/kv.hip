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
// cache head h / rep), two launches:
//   k_kv_split   per (split of 128 tokens, cache head): scores of the rep
//                query heads from keys dequantized to exact fp16 (q - z)
//                pairs (as in the GEMV), the split's max m and sum of
//                exp(s - m), and sum_t exp(s_t - m) v_t with lane-per-channel-
//                pair dequantization of the values -> fp32 partials;
//   k_kv_combine rescales the splits to the global max and divides, fp16.
#include "spectra_internal.h"
#include "g32.h"

namespace spectra {
namespace {

constexpr int kGroup32 = 32;
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

// One block per (split of kTokensPerSplit tokens, cache head h), serving the
// rep query heads that read h:
//   1. the value records, scales and zero bytes of the split are requested
//      first, 16 bytes of records per thread and load (as many small
//      per-lane loads cost 3 % more); they are stored to LDS once the scores
//      are done;
//   2. two adjacent threads per token, G / 2 groups each: dequantize the
//      key's groups (exact fp16 (q - z) pairs), dot them with the rep queries
//      in fp32, times s16 per group; the pair adds its halves with one lane
//      swap, over sqrt(D) -> scores in LDS;
//   3. per query head the split's max m and l = sum exp(s - m); the scores
//      become p = exp(s - m);
//   4. sum_t p_t v_t per query head in registers (lane-per-channel-pair:
//      lane l owns pairs l + 64 i, each wave every WAVES-th token, values
//      dequantized from LDS), reduced across the waves -> fp32 partials and
//      (m, l) per (split, query head).
// The keys and values of the split are read once for all rep query heads.
// REP is the build's bound on the query heads per cache head; rep_rt <= REP
// is the call's (heads past rep_rt score a zero query and write nothing).
template <int G, int REP>
__global__ __launch_bounds__(kPvThreads) void k_kv_split(const KvView c, const uint16_t* __restrict__ q,
                                                         int64_t L, float* __restrict__ part,
                                                         float* __restrict__ stats, const int rep_rt) {
  const int rep = rep_rt;
  constexpr int D = 32 * G;
  constexpr int NP = D / 2;                   // channel pairs
  constexpr int PL = NP >= 64 ? NP / 64 : 1;  // pairs per lane
  constexpr int WAVES = kPvThreads / 64;
  constexpr int TS = kTokensPerSplit;
  constexpr int UN = TS / WAVES;              // tokens per wave
  constexpr int RPT = TS * G / kPvThreads;    // value records per thread
  __shared__ half2_t qs[REP][D / 2];
  __shared__ float sc[REP][TS];
  __shared__ float mst[REP], lst[REP];
  // all query heads' wave partials at once (one barrier) where they fit in
  // 32 KiB, else one query head at a time
  constexpr bool ALL = REP * D <= 2048;
  __shared__ float pacc[WAVES][ALL ? REP : 1][D];
  const int split = blockIdx.x, h = blockIdx.y;
  const int H = c.H, Hq = H * rep;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t t0 = (int64_t)split * TS;
  for (int i = threadIdx.x; i < REP * D / 2; i += blockDim.x) {
    const int rr = i / (D / 2), j = i % (D / 2);
    qs[rr][j] = rr < rep ? as_h2(reinterpret_cast<const uint32_t*>(q + (int64_t)(h * rep + rr) * D)[j])
                         : as_h2(0u);
  }

  // 1. the split's value records, scales and zero bytes, a few wide loads per
  //    thread (tokens past L read token t0's); they go to LDS after the scores
  __shared__ u32x4 vrec[TS * G];
  __shared__ uint16_t vscl[TS * G];
  __shared__ uint8_t vzb[TS * G / 2];
  u32x4 vr[RPT];
  uint32_t vsr[RPT], vzr[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int idx = threadIdx.x + kPvThreads * i, tl = idx / G, g = idx % G;
    const int64_t t = t0 + tl;
    const int64_t flat = ((t < L ? t : t0) * H + h) * G + g;
    vr[i] = *reinterpret_cast<const u32x4*>(c.v.codes + flat);
    vsr[i] = c.v.scales[flat];
    vzr[i] = c.v.zeros[flat >> 1];  // the byte of groups g, g + 1 (flat and g have the same parity)
  }
  __syncthreads();  // qs ready

  // 2. scores: two threads per token (adjacent lanes), G / 2 groups each
  static_assert(2 * TS == kPvThreads, "two threads per token");
  {
    constexpr int GH = G / 2;
    const int tl = threadIdx.x >> 1, hf = threadIdx.x & 1;
    const int64_t t = t0 + tl;
    const int64_t flat0 = ((t < L ? t : t0) * H + h) * G + hf * GH;
    uint4 krec[GH];
    uint16_t ksc[GH];
    uint8_t kzb[GH];
#pragma unroll
    for (int g = 0; g < GH; ++g) {
      krec[g] = c.k.codes[flat0 + g];
      ksc[g] = c.k.scales[flat0 + g];
      kzb[g] = c.k.zeros[(flat0 + g) >> 1];
    }
    float acc[REP];
#pragma unroll
    for (int rr = 0; rr < REP; ++rr) acc[rr] = 0.f;
#pragma unroll
    for (int gg = 0; gg < GH; ++gg) {
      const int g = hf * GH + gg;
      const float s16 = h2f(ksc[gg]);
      const uint32_t z = ((uint32_t)kzb[gg] >> (4 * (g & 1))) & 0xFu;
      const uint32_t w[4] = {krec[gg].x, krec[gg].y, krec[gg].z, krec[gg].w};
      half2_t wq[16];
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int j = 0; j < 4; ++j) wq[4 * d + j] = pair_qz(w[d], j, z);
#pragma unroll
      for (int rr = 0; rr < REP; ++rr) {
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int j = 0; j < 16; j += 2) {
          a0 = __builtin_amdgcn_fdot2(wq[j], qs[rr][16 * g + j], a0, false);
          a1 = __builtin_amdgcn_fdot2(wq[j + 1], qs[rr][16 * g + j + 1], a1, false);
        }
        acc[rr] = __builtin_fmaf(s16, a0 + a1, acc[rr]);
      }
    }
#pragma unroll
    for (int rr = 0; rr < REP; ++rr) acc[rr] += __shfl_xor(acc[rr], 1);
    const float inv_sqrt_d = 1.0f / __builtin_sqrtf((float)D);
    if (hf == 0) {
#pragma unroll
      for (int rr = 0; rr < REP; ++rr) sc[rr][tl] = t < L ? acc[rr] * inv_sqrt_d : -INFINITY;
    }
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int idx = threadIdx.x + kPvThreads * i;
    vrec[idx] = vr[i];
    vscl[idx] = (uint16_t)vsr[i];
    if ((idx & 1) == 0) vzb[idx >> 1] = (uint8_t)vzr[i];
  }
  __syncthreads();

  // 3. split max and exp sums, one query head per wave at a time
  for (int rr = wave; rr < rep; rr += WAVES) {
    float m = -INFINITY;
    for (int j = lane; j < TS; j += 64) m = fmaxf(m, sc[rr][j]);
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    float l = 0.f;
    for (int j = lane; j < TS; j += 64) {
      const float p = __expf(sc[rr][j] - m);  // 0 for tokens past L
      sc[rr][j] = p;
      l += p;
    }
    for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o);
    if (lane == 0) {
      mst[rr] = m;
      lst[rr] = l;
    }
  }
  __syncthreads();

  // 4. values
  float a[REP][PL][2];
#pragma unroll
  for (int rr = 0; rr < REP; ++rr)
#pragma unroll
    for (int i = 0; i < PL; ++i) a[rr][i][0] = a[rr][i][1] = 0.f;
#pragma unroll 2
  for (int u = 0; u < UN; ++u) {
    const int tl = wave + WAVES * u;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int pi = (lane + 64 * i) % NP;  // lanes past NP (D = 64) take a valid pair, unused
      const int g = pi >> 4, e = (2 * pi) & 31;
      const int idx = tl * G + g;
      const uint32_t w = reinterpret_cast<const uint32_t*>(vrec)[4 * idx + (e >> 3)];
      const uint32_t z = ((uint32_t)vzb[idx >> 1] >> (4 * (g & 1))) & 0xFu;
      const half2_t qz = pair_qz(w, (e & 7) >> 1, z);
      const float s16 = h2f(vscl[idx]);
      const float v0 = (float)qz.x * s16, v1 = (float)qz.y * s16;
#pragma unroll
      for (int rr = 0; rr < REP; ++rr) {
        const float p = sc[rr][tl];
        a[rr][i][0] = __builtin_fmaf(p, v0, a[rr][i][0]);
        a[rr][i][1] = __builtin_fmaf(p, v1, a[rr][i][1]);
      }
    }
  }
  if constexpr (ALL) {
#pragma unroll
    for (int rr = 0; rr < REP; ++rr)
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int pi = lane + 64 * i;
        if (pi < NP) {
          pacc[wave][rr][2 * pi] = a[rr][i][0];
          pacc[wave][rr][2 * pi + 1] = a[rr][i][1];
        }
      }
    __syncthreads();
    for (int j = threadIdx.x; j < rep * D; j += blockDim.x) {
      const int rr = j / D, d = j % D;
      float sum = 0.f;
      for (int w2 = 0; w2 < WAVES; ++w2) sum += pacc[w2][rr][d];
      part[((int64_t)split * Hq + h * rep + rr) * D + d] = sum;
    }
    if (threadIdx.x < rep) {
      const int64_t base = (int64_t)split * Hq + h * rep + threadIdx.x;
      stats[2 * base] = mst[threadIdx.x];
      stats[2 * base + 1] = lst[threadIdx.x];
    }
  } else {
#pragma unroll
    for (int rr = 0; rr < REP; ++rr) {
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int pi = lane + 64 * i;
        if (pi < NP) {
          pacc[wave][0][2 * pi] = a[rr][i][0];
          pacc[wave][0][2 * pi + 1] = a[rr][i][1];
        }
      }
      __syncthreads();
      const int64_t base = (int64_t)split * Hq + h * rep + rr;
      for (int d = threadIdx.x; d < D && rr < rep; d += blockDim.x) {
        float sum = 0.f;
        for (int w2 = 0; w2 < WAVES; ++w2) sum += pacc[w2][0][d];
        part[base * D + d] = sum;
      }
      if (threadIdx.x == 0 && rr < rep) {
        stats[2 * base] = mst[rr];
        stats[2 * base + 1] = lst[rr];
      }
      __syncthreads();
    }
  }
}

// out = sum_s exp(m_s - M) O_s / sum_s exp(m_s - M) l_s, M = max_s m_s.  The
// split weights are computed once into LDS; each thread then sums its
// channel over the splits with several loads in flight.
constexpr int kMaxSplits = 4096;
constexpr int kCombThreads = 256;
constexpr int kCombFirst = 32;  // partials per thread requested with the stats, in one round trip
// One block per query head hq.  Thread t owns channel d = t % D and the
// splits sp = t / D (mod R), R = 256 / D threads per channel.  The stats of
// every split and the thread's first kCombFirst partials are requested
// together (the partials do not depend on the weights), so a call over up to
// R * kCombFirst splits waits for one round of loads: global max, weights
// exp(m - M) in LDS, sum of weights times exp sums, weighted partial sums,
// the R threads of a channel added in LDS, divided, fp16.
__global__ __launch_bounds__(kCombThreads) void k_kv_combine(const float* __restrict__ part,
                                                            const float* __restrict__ stats, int splits, int Hq,
                                                            int D, uint16_t* __restrict__ out) {
  __shared__ float wgt[kMaxSplits];
  __shared__ float osum[kCombThreads];
  __shared__ float red[kCombThreads / 64];
  const int hq = blockIdx.x, t = threadIdx.x;
  const int R = kCombThreads / D, d = t % D, r = t / D;
  float pv[kCombFirst];
#pragma unroll
  for (int i = 0; i < kCombFirst; ++i) {
    const int sp = r + R * i;
    pv[i] = sp < splits ? part[((int64_t)sp * Hq + hq) * D + d] : 0.f;
  }
  float M = -INFINITY;
  for (int sp = t; sp < splits; sp += kCombThreads) {
    const float m = stats[2 * ((int64_t)sp * Hq + hq)];
    wgt[sp] = m;
    M = fmaxf(M, m);
  }
  M = block_max(M, red);  // its barriers also publish the maxima in wgt
  float l = 0.f;
  for (int sp = t; sp < splits; sp += kCombThreads) {
    const float w = __expf(wgt[sp] - M);
    wgt[sp] = w;
    l += w * stats[2 * ((int64_t)sp * Hq + hq) + 1];
  }
  l = block_sum(l, red);  // its barriers also publish the weights
  float o0 = 0.f, o1 = 0.f;
#pragma unroll
  for (int i = 0; i < kCombFirst; i += 2) {
    const int sp = r + R * i;
    if (sp < splits) o0 = __builtin_fmaf(wgt[sp], pv[i], o0);
    if (sp + R < splits) o1 = __builtin_fmaf(wgt[sp + R], pv[i + 1], o1);
  }
  for (int sp = r + R * kCombFirst; sp < splits; sp += R)  // long contexts: the rest
    o0 = __builtin_fmaf(wgt[sp], part[((int64_t)sp * Hq + hq) * D + d], o0);
  osum[t] = o0 + o1;
  __syncthreads();
  if (r == 0) {
    float tot = osum[d];
    for (int rr = 1; rr < R; ++rr) tot += osum[d + rr * D];
    out[(int64_t)hq * D + d] = __builtin_bit_cast(uint16_t, (_Float16)(tot / l));
  }
}

int64_t splits_of(int64_t L) { return (L + kTokensPerSplit - 1) / kTokensPerSplit; }

}  // namespace

int64_t kv_max_attend_length() { return (int64_t)kMaxSplits * kTokensPerSplit; }

namespace {

template <int G, int REP>
hipError_t attend_gr(const KvView& c, const uint16_t* q, int rep, int64_t L, uint16_t* out, void* ws,
                     hipStream_t s) {
  constexpr int D = 32 * G;
  const int Hq = c.H * rep;
  const int64_t splits = splits_of(L);
  float* part = static_cast<float*>(ws);
  float* stats = part + (size_t)splits * Hq * D;
  hipLaunchKernelGGL((k_kv_split<G, REP>), dim3((unsigned)splits, (unsigned)c.H), dim3(kPvThreads), 0, s, c, q, L,
                     part, stats, rep);
  hipLaunchKernelGGL(k_kv_combine, dim3((unsigned)Hq), dim3(kCombThreads), 0, s, part, stats, (int)splits, Hq, D,
                     out);
  return hipGetLastError();
}

template <int G>
hipError_t attend_g(const KvView& c, const uint16_t* q, int rep, int64_t L, uint16_t* out, void* ws,
                    hipStream_t s) {
  // every ratio 1 .. 16 runs on the build for the next power of two
  if (rep < 1 || rep > 16) return hipErrorNotSupported;
  if (rep == 1) return attend_gr<G, 1>(c, q, rep, L, out, ws, s);
  if (rep == 2) return attend_gr<G, 2>(c, q, rep, L, out, ws, s);
  if (rep <= 4) return attend_gr<G, 4>(c, q, rep, L, out, ws, s);
  if (rep <= 8) return attend_gr<G, 8>(c, q, rep, L, out, ws, s);
  return attend_gr<G, 16>(c, q, rep, L, out, ws, s);
}

}  // namespace

size_t kv_attend_workspace_bytes(const KvView& c, int rep, int64_t L) {
  const int64_t Hq = (int64_t)c.H * rep;
  return 4 * (size_t)(splits_of(L) * Hq * (c.D + 2));
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
