// SPECTRA batched product for gfx950: y = x W_hat^T for M >= 2 on the matrix
// cores (v_mfma_f32_16x16x32_f16).
//
// The SPECTRA page reports Tensor-Core prefill next to its decode kernels
// (highlight 4); this is the gfx950 counterpart for batched rows, written for
// 64-wide wavefronts and CDNA4 MFMA rather than from the page's kernels.
//
// Pass 1 (k_xbulk): x is permuted once per call into a workspace row per m:
// bulk order, zero padded to 32G, followed by the heavy-tailed x values
// zero padded to a multiple of 32.
//
// Pass 2 (k_mfma): a block owns BN = 64 output columns and BM = 16*MT input
// rows.  The K loop walks chunks of 4 groups (128 bulk positions):
//   - each thread loads one group record (16 bytes of codes, its scale and
//     zero point) and dequantizes it to 32 exact fp16 values (q - z) with the
//     1024 magic (fp16 integers below 2048 are exact), written to LDS;
//   - the x chunk (BM x 128 halves) is copied to LDS with 16-byte loads;
//   - each wave computes its 16 output columns for every m-subtile: one MFMA
//     per group (K = 32 is exactly one group) into a zero accumulator, then
//     acc += s16 * result in fp32, so weights are never rounded a second time.
// The next chunk's records and x are held in registers while the current
// chunk is multiplied.  The heavy-tailed columns follow as plain MFMA steps
// (fp16 weights, scale 1).  Loads use buffer descriptors: rows past N or M
// and positions past the padded K read as zero.
#include "spectra_internal.h"

namespace spectra {
namespace {

constexpr int kThreads = 256;
constexpr int kBN = 64;        // output columns per block (16 per wave)
constexpr int kChunkG = 4;     // groups per K chunk
constexpr int kChunkK = 128;   // bulk positions per K chunk
constexpr int kRowH = kChunkK + 8;  // LDS row stride in halves (272 bytes: conflict-free 16-byte reads)
constexpr int kRsrcWord3 = 0x00020000;
constexpr uint32_t kOob = 0x80000000u;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint64_t bytes) {
  const int n = bytes >= 0x7FFFFFFFull ? 0x7FFFFFFF : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kRsrcWord3);
}
__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// x (M x K) -> workspace rows of KW = 32G + OP halves: bulk order then the
// heavy-tailed values, zero padded.
__global__ __launch_bounds__(kThreads) void k_xbulk(DeviceView v, const uint16_t* __restrict__ x,
                                                    int64_t M, uint16_t* __restrict__ xw, int KW) {
  const int j = blockIdx.x * kThreads + threadIdx.x;
  if (j >= KW) return;
  const int KP = 32 * v.G;
  int src = -1;  // channel feeding workspace column j
  if (j < KP) {
    if (j < v.K_b) src = v.perm[j];
  } else if (j - KP < v.n_out) {
    src = v.perm[v.K_b + (j - KP)];
  }
  for (int64_t m = blockIdx.y; m < M; m += gridDim.y)
    xw[m * KW + j] = src >= 0 ? x[m * v.K + src] : (uint16_t)0;
}

// One group record -> 32 exact fp16 values (q - z), as four 16-byte rows of
// 8 members each (members 8d .. 8d+7 from code word d).
__device__ __forceinline__ void dequant_record(const u32x4 c, uint32_t z, u32x4 out[4]) {
  const uint32_t zp = (0x6400u + z) * 0x00010001u;  // fp16 pair (1024 + z)
  const half2_t zh = __builtin_bit_cast(half2_t, zp);
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t h = ((w[d] >> (4 * i)) & 0x000F000Fu) | 0x64006400u;  // 1024 + q pair
      r[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, h) - zh);
    }
    out[d] = u32x4{r[0], r[1], r[2], r[3]};
  }
}

template <int MT>
__global__ __launch_bounds__(kThreads) void k_mfma(DeviceView v, const uint16_t* __restrict__ xw,
                                                   int KW, int64_t M, uint16_t* __restrict__ y) {
  constexpr int BM = 16 * MT;
  __shared__ __align__(16) uint16_t As[BM * kRowH];
  __shared__ __align__(16) uint16_t Bs[kBN * kRowH];
  __shared__ float Ss[kBN * kChunkG];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * kBN;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int G = v.G, KP = 32 * G;
  const int64_t rows_n = (v.N - n0) < kBN ? (v.N - n0) : kBN;
  const int64_t rows_m = (M - m0) < BM ? (M - m0) : BM;

  // descriptors rebased on this block's rows
  const int64_t i0 = n0 * G;
  const __amdgpu_buffer_rsrc_t rc = rsrc(v.codes + i0, (uint64_t)rows_n * G * 16);
  const __amdgpu_buffer_rsrc_t rs = rsrc(v.scales + i0, (uint64_t)rows_n * G * 2);
  const int64_t zb0 = i0 >> 1;
  const __amdgpu_buffer_rsrc_t rz = rsrc(v.zeros + zb0, (uint64_t)(((i0 + rows_n * G + 1) >> 1) - zb0));
  const __amdgpu_buffer_rsrc_t rx = rsrc(xw + m0 * KW, (uint64_t)rows_m * KW * 2);

  // loader roles: thread -> one (row, group) record of the chunk, and MT
  // 16-byte x segments (BM rows x 16 segments of 8 halves)
  const int br = tid >> 2, bg = tid & 3;
  float4_t acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};

  const int nchunk = (G + kChunkG - 1) / kChunkG;
  u32x4 pc;
  uint32_t ps, pz;
  u32x4 px[MT];
  auto load_chunk = [&](int ch) {
    const int g = ch * kChunkG + bg;
    const uint32_t local = (uint32_t)(br * G + g);
    const bool ok = g < G;
    pc = __builtin_amdgcn_raw_buffer_load_b128(rc, ok ? local * 16u : kOob, 0, 0);
    ps = __builtin_amdgcn_raw_buffer_load_b16(rs, ok ? local * 2u : kOob, 0, 0);
    const uint32_t zoff = (uint32_t)(((i0 + local) >> 1) - zb0);
    pz = __builtin_amdgcn_raw_buffer_load_b8(rz, ok ? zoff : kOob, 0, 0);
    pz = (pz >> (4u * (uint32_t)((i0 + local) & 1))) & 0xFu;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int seg = tid + kThreads * t;  // < BM * 16
      const int r = seg >> 4, s8 = seg & 15;
      const int col = ch * kChunkK + 8 * s8;
      px[t] = __builtin_amdgcn_raw_buffer_load_b128(
          rx, col < KP ? (uint32_t)(r * KW + col) * 2u : kOob, 0, 0);
    }
  };
  auto store_chunk = [&]() {
    u32x4 q[4];
    dequant_record(pc, pz, q);
#pragma unroll
    for (int d = 0; d < 4; ++d)
      *reinterpret_cast<u32x4*>(Bs + br * kRowH + bg * 32 + 8 * d) = q[d];
    Ss[br * kChunkG + bg] = h2f((uint16_t)ps);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int seg = tid + kThreads * t;
      *reinterpret_cast<u32x4*>(As + (seg >> 4) * kRowH + 8 * (seg & 15)) = px[t];
    }
  };

  const int col_n = wave * 16 + (lane & 15);  // this lane's output column in the block
  const int kq = lane >> 4;                   // which 8-member quarter of a group
  if (nchunk > 0) load_chunk(0);
  for (int ch = 0; ch < nchunk; ++ch) {
    store_chunk();
    __syncthreads();
    if (ch + 1 < nchunk) load_chunk(ch + 1);
#pragma unroll
    for (int g = 0; g < kChunkG; ++g) {
      const half8 b = *reinterpret_cast<const half8*>(Bs + col_n * kRowH + g * 32 + 8 * kq);
      const float s = Ss[col_n * kChunkG + g];
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const half8 a = *reinterpret_cast<const half8*>(As + (16 * t + (lane & 15)) * kRowH + g * 32 + 8 * kq);
        const float4_t p = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        acc[t] += s * p;
      }
    }
    __syncthreads();
  }

  // heavy-tailed columns: fp16 weights as they are, scale 1
  const int n_out = v.n_out;
  if (n_out > 0) {
    const int OP = (n_out + 31) & ~31;
    const __amdgpu_buffer_rsrc_t ro = rsrc(v.outliers + n0 * n_out, (uint64_t)rows_n * n_out * 2);
    for (int o0 = 0; o0 < OP; o0 += 32) {
      // B: 64 rows x 32 values; thread -> row tid/4, 8 values at 8*(tid%4)
      {
        const int r = tid >> 2, c8 = 8 * (tid & 3);
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = o0 + c8 + e;
          h[e] = __builtin_amdgcn_raw_buffer_load_b16(ro, j < n_out ? (uint32_t)(r * n_out + j) * 2u : kOob, 0, 0);
        }
        *reinterpret_cast<u32x4*>(Bs + r * kRowH + c8) =
            u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
      }
      // A: BM rows x 32 heavy-tailed x values (4 segments per row)
      for (int seg = tid; seg < BM * 4; seg += kThreads) {
        const int r = seg >> 2, s8 = seg & 3;
        const int col = KP + o0 + 8 * s8;
        *reinterpret_cast<u32x4*>(As + r * kRowH + 8 * s8) =
            __builtin_amdgcn_raw_buffer_load_b128(rx, (uint32_t)(r * KW + col) * 2u, 0, 0);
      }
      __syncthreads();
      const half8 b = *reinterpret_cast<const half8*>(Bs + col_n * kRowH + 8 * kq);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const half8 a = *reinterpret_cast<const half8*>(As + (16 * t + (lane & 15)) * kRowH + 8 * kq);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[t], 0, 0, 0);
      }
      __syncthreads();
    }
  }

  // D layout: lane holds rows 4*(lane/16) + r of each m-subtile, column lane%16
  const int64_t n = n0 + col_n;
  if (n < v.N) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + 16 * t + 4 * kq + r;
        if (m < M) y[m * v.N + n] = f2h(acc[t][r]);
      }
    }
  }
}

}  // namespace

bool mfma_supports(const DeviceView& v, int64_t M) {
  // workspace row must stay addressable with 32-bit byte offsets per block
  const int64_t KW = 32 * (int64_t)v.G + ((v.n_out + 31) & ~31);
  return M >= 1 && KW * 2 * 128 < 0x7FFFFFFF;
}

size_t mfma_workspace_bytes(const DeviceView& v, int64_t M) {
  const int64_t KW = 32 * (int64_t)v.G + ((v.n_out + 31) & ~31);
  return (size_t)(M * KW * 2);
}

hipError_t launch_mfma_ws(const DeviceView& v, const uint16_t* x, uint16_t* y, int64_t M,
                          void* workspace, hipStream_t s) {
  const int KW = 32 * v.G + ((v.n_out + 31) & ~31);
  uint16_t* xw = static_cast<uint16_t*>(workspace);
  const unsigned gy = (unsigned)(M < 65535 ? M : 65535);
  hipLaunchKernelGGL(k_xbulk, dim3((unsigned)((KW + kThreads - 1) / kThreads), gy),
                     dim3(kThreads), 0, s, v, x, M, xw, KW);
  const unsigned gx = (unsigned)((v.N + kBN - 1) / kBN);
  if (M <= 16) {
    hipLaunchKernelGGL(k_mfma<1>, dim3(gx, (unsigned)((M + 15) / 16)), dim3(kThreads), 0, s, v, xw, KW, M, y);
  } else if (M <= 32) {
    hipLaunchKernelGGL(k_mfma<2>, dim3(gx, (unsigned)((M + 31) / 32)), dim3(kThreads), 0, s, v, xw, KW, M, y);
  } else if (M <= 64) {
    hipLaunchKernelGGL(k_mfma<4>, dim3(gx, (unsigned)((M + 63) / 64)), dim3(kThreads), 0, s, v, xw, KW, M, y);
  } else {
    hipLaunchKernelGGL(k_mfma<8>, dim3(gx, (unsigned)((M + 127) / 128)), dim3(kThreads), 0, s, v, xw, KW, M, y);
  }
  return hipGetLastError();
}

}  // namespace spectra
