// SPECTRA dequant-GEMV for gfx950 at M = 1 (decode): y = x W_hat^T.
//
// The SPECTRA page (abstract; highlight 4 on its fused kernels) describes
// dequantization fused into the product so that only the packed weights cross
// DRAM; the decode product is bound by weight bytes (the techfi24 summary,
// "Contexte materiel": every token re-reads all weights).  This kernel is a
// gfx950 design of that idea, not a port: the page's kernels target a laptop
// Ampere GPU.
//
// Mapping.  A team of L lanes (L = 16, 32 or 64) owns one output row at a
// time; lane t of a team owns the groups g = t + L*p (p < P) of every row it
// visits, so each of its x slices (32 fp16 values per group) is loaded from
// LDS into registers once per block and reused for every row.  A team's loads
// for slot p cover 16*L contiguous bytes of codes (global_load_dwordx4 per
// lane).  Each block stages x in bulk order (gathered through perm, padded
// with zeros) plus the heavy-tailed x values in LDS, then walks its rows.
//
// Arithmetic.  A code word w yields two members per 16-bit half with
// (w >> 4i) & 0x000F000F; OR-ing 0x6400 into each half makes the fp16 values
// 1024 + q exactly, and subtracting the fp16 pair (1024 + z) gives q - z
// exactly.  v_dot2_f32_f16 multiplies by the matching x pair and accumulates
// in fp32; the group sum is scaled by s16 in fp32.  The heavy-tailed columns
// are a dense fp16 side product in the same pass.  Team partials are reduced
// with DPP inside 16-lane rows and lane swizzles across rows.
#include "spectra_internal.h"

namespace spectra {
namespace {

constexpr int kBlock = 256;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the L lanes of a team; every lane of the team gets the total.
template <int L>
__device__ __forceinline__ float team_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x124>(v);  // row_ror:4
  v += dpp<0x128>(v);  // row_ror:8
  if constexpr (L >= 32) v += __shfl_xor(v, 16);
  if constexpr (L >= 64) v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ float h2f(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}
__device__ __forceinline__ uint16_t f2h(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

// Dot of one 16-byte code record (32 members) with the matching 16 x pairs,
// zero point folded in exactly.  Returns sum_e (q_e - z) * x_e in fp32.
__device__ __forceinline__ float group_dot(const uint4 c, const uint32_t z, const half2_t* xr) {
  const half2_t zp = as_h2((0x6400u + z) * 0x00010001u);
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  float t = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const half2_t q = as_h2(((w[d] >> (4 * i)) & 0x000F000Fu) | 0x64006400u);
      t = __builtin_amdgcn_fdot2(q - zp, xr[4 * d + i], t, false);
    }
  }
  return t;
}

template <int L, int P, int U>
__global__ __launch_bounds__(kBlock) void k_gemv_m1(DeviceView v, const uint16_t* __restrict__ x,
                                                    uint16_t* __restrict__ y,
                                                    int64_t rows_per_block) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int T = kBlock / L;  // teams per block
  const int G = v.G, K_b = v.K_b, n_out = v.n_out;
  const int xs_bytes = (64 * G + 15) & ~15;
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  float* xo = reinterpret_cast<float*>(smem + xs_bytes);
  const int tid = threadIdx.x;

  // Stage x (bulk order, zero padded to 32G) and the heavy-tailed x values.
  for (int j = tid; j < 32 * G; j += kBlock) xs[j] = (j < K_b) ? x[v.perm[j]] : (uint16_t)0;
  for (int j = tid; j < n_out; j += kBlock) xo[j] = h2f(x[v.perm[K_b + j]]);
  __syncthreads();

  const int lt = tid % L;
  const int team = tid / L;
  half2_t xr[P][16];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int g = lt + L * p;
    if (g < G) {
      const uint4* src = reinterpret_cast<const uint4*>(xs + 32 * g);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 u = src[q];
        xr[p][4 * q + 0] = as_h2(u.x);
        xr[p][4 * q + 1] = as_h2(u.y);
        xr[p][4 * q + 2] = as_h2(u.z);
        xr[p][4 * q + 3] = as_h2(u.w);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 16; ++q) xr[p][q] = as_h2(0u);
    }
  }

  const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
  const int64_t r1 = (r0 + rows_per_block < v.N) ? r0 + rows_per_block : v.N;
  for (int64_t tile = r0; tile < r1; tile += (int64_t)T * U) {
    uint4 c[U][P];
    uint16_t sc[U][P];
    uint8_t zb[U][P];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t n = tile + team + (int64_t)u * T;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int g = lt + L * p;
        if (n < r1 && g < G) {
          const int64_t i = n * G + g;
          c[u][p] = v.codes[i];
          sc[u][p] = v.scales[i];
          zb[u][p] = v.zeros[i >> 1];
        } else {
          c[u][p] = make_uint4(0u, 0u, 0u, 0u);
          sc[u][p] = 0;
          zb[u][p] = 0;
        }
      }
    }
    float acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t n = tile + team + (int64_t)u * T;
      float a = 0.f;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int g = lt + L * p;
        const int64_t i = n * G + g;
        const uint32_t z = ((uint32_t)zb[u][p] >> ((uint32_t)(i & 1) * 4u)) & 0xFu;
        a = __builtin_fmaf(h2f(sc[u][p]), group_dot(c[u][p], z, xr[p]), a);
      }
      if (n < r1) {
        const uint16_t* orow = v.outliers + n * n_out;
        for (int j = lt; j < n_out; j += L) a = __builtin_fmaf(xo[j], h2f(orow[j]), a);
      }
      acc[u] = a;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t n = tile + team + (int64_t)u * T;
      const float s = team_sum<L>(acc[u]);
      if (lt == 0 && n < r1) y[n] = f2h(s);
    }
  }
}

struct Variant {
  int L, P;
};

// Pick lanes-per-row L and slots-per-lane P = ceil(G/L) with the best lane use.
Variant pick_variant(int G) {
  Variant best{64, 0};
  double best_eff = -1.0;
  const int Ls[3] = {64, 32, 16};
  for (int li = 0; li < 3; ++li) {
    const int L = Ls[li];
    const int P = G == 0 ? 1 : (G + L - 1) / L;
    if (P > 8) continue;
    const double eff = G == 0 ? 1.0 : (double)G / (double)(L * P);
    if (eff > best_eff + 1e-9 || (eff > best_eff - 1e-9 && P < best.P)) {
      best_eff = eff;
      best = Variant{L, P};
    }
  }
  return best;
}

constexpr int kU = 2;

template <int L, int P>
hipError_t launch_lp(const DeviceView& v, const uint16_t* x, uint16_t* y, hipStream_t s) {
  const int cu = v.cu_count;
  constexpr int T = kBlock / L;
  const int64_t rows_per_tile = (int64_t)T * kU;
  const int64_t tiles = (v.N + rows_per_tile - 1) / rows_per_tile;
  int64_t blocks = tiles < (int64_t)cu * 4 ? tiles : (int64_t)cu * 4;
  if (blocks < 1) blocks = 1;
  const int64_t tiles_per_block = (tiles + blocks - 1) / blocks;
  const int64_t rows_per_block = tiles_per_block * rows_per_tile;
  blocks = (v.N + rows_per_block - 1) / rows_per_block;
  const size_t lds = (size_t)((64 * v.G + 15) & ~15) + 4 * (size_t)v.n_out;
  hipLaunchKernelGGL((k_gemv_m1<L, P, kU>), dim3((unsigned)blocks), dim3(kBlock), lds, s, v, x, y,
                     rows_per_block);
  return hipGetLastError();
}

template <int L>
hipError_t launch_l(int P, const DeviceView& v, const uint16_t* x, uint16_t* y, hipStream_t s) {
  switch (P) {
    case 1: return launch_lp<L, 1>(v, x, y, s);
    case 2: return launch_lp<L, 2>(v, x, y, s);
    case 3: return launch_lp<L, 3>(v, x, y, s);
    case 4: return launch_lp<L, 4>(v, x, y, s);
    case 5: return launch_lp<L, 5>(v, x, y, s);
    case 6: return launch_lp<L, 6>(v, x, y, s);
    case 7: return launch_lp<L, 7>(v, x, y, s);
    case 8: return launch_lp<L, 8>(v, x, y, s);
    default: return hipErrorNotSupported;
  }
}

constexpr size_t kMaxLds = 64 * 1024;

}  // namespace

bool gemv_supports(const DeviceView& v, int64_t M) {
  if (M != 1) return false;
  if (pick_variant(v.G).P == 0) return false;
  const size_t lds = (size_t)((64 * v.G + 15) & ~15) + 4 * (size_t)v.n_out;
  return lds <= kMaxLds;
}

hipError_t launch_gemv(const DeviceView& v, const uint16_t* x, uint16_t* y, int64_t M,
                       hipStream_t s) {
  if (!gemv_supports(v, M)) return hipErrorNotSupported;
  const Variant vr = pick_variant(v.G);
  switch (vr.L) {
    case 16: return launch_l<16>(vr.P, v, x, y, s);
    case 32: return launch_l<32>(vr.P, v, x, y, s);
    default: return launch_l<64>(vr.P, v, x, y, s);
  }
}

hipError_t launch_gemv_grouped(const DeviceView*, int, const uint16_t*, uint16_t* const*,
                               hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace spectra
