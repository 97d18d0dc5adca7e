// SPECTRA batched product for gfx950: y = x W_hat^T on the matrix cores
// (v_mfma_f32_16x16x32_f16), for M >= 5 and the shapes the GEMV declines.
//
// The SPECTRA page reports Tensor-Core prefill next to its decode kernels
// (highlight 4); this is the gfx950 counterpart for batched rows, written for
// 64-wide wavefronts and CDNA4 MFMA rather than from the page's kernels.
//
// Pass 1 (k_xbulk): x is permuted once per call into a workspace row per m:
// bulk order, zero padded to 32G, followed by the heavy-tailed x values
// zero padded to a multiple of 32.
//
// Pass 2 (k_mfma): a wave owns 16 * NT consecutive output rows for the whole
// K loop.  Per chunk of CG groups it loads its code records row-contiguously
// (consecutive lanes on consecutive records of a row: whole cache lines),
// stores them to a small wave-private LDS tile and reads them back in the
// B-operand order of v_mfma_f32_16x16x32_f16: lane (r, c) takes dword r of
// row c's record, members 8r .. 8r + 7 of the group.  The dword is
// dequantized in registers to exact fp16 (q - z): (w & 0x000F000F) | 0x6400
// 6400 holds 1024 + q of two members, (w & 0x00F000F0) | 0x5400 5400 holds
// 64 + q of the next two, and subtracting 1024 + z or 64 + z is exact.  One
// MFMA per group and m-subtile into a zero accumulator, then acc += s16 * D in
// fp32, so the weights are never rounded a second time.  The A operand (x in
// bulk order, 16*MT rows x 32*CG positions per chunk) is staged in LDS once per
// block and chunk; the weights run 4 chunks ahead in registers.  The
// heavy-tailed columns follow as plain MFMA steps (fp16 weights, scale 1).
// Loads use buffer descriptors: rows past N or M and positions past the
// padded K read as zero.
#include "spectra_internal.h"

namespace spectra {
namespace {

constexpr int kThreads = 256;   // k_xbulk
constexpr int kMaxW = 8;        // waves per block (4 .. 8)
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

__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

// (a & m) | o in one VALU op (VOP3 on gfx9 takes no literal, so the compiler
// otherwise splits it into an AND and an OR with literals).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(o));
  return r;
}

// Code word -> its 8 members as exact fp16 (q - z), in member order.  Member
// 8d + i of a record sits in word d at bit 16 (i % 2) + 4 (i / 2).
__device__ __forceinline__ half8 dequant_word(uint32_t w, uint32_t z) {
  const half2_t zl = as_h2((0x6400u + z) * 0x00010001u);  // 1024 + z
  const half2_t zh = as_h2((0x5400u + (z << 4)) * 0x00010001u);  // 64 + z (z in mantissa bits 4..7)
  const uint32_t w8 = w >> 8;
  const half2_t p0 = as_h2(and_or(w, 0x000F000Fu, 0x64006400u)) - zl;   // members 0, 1
  const half2_t p1 = as_h2(and_or(w, 0x00F000F0u, 0x54005400u)) - zh;   // members 2, 3
  const half2_t p2 = as_h2(and_or(w8, 0x000F000Fu, 0x64006400u)) - zl;  // members 4, 5
  const half2_t p3 = as_h2(and_or(w8, 0x00F000F0u, 0x54005400u)) - zh;  // members 6, 7
  return half8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// One chunk of one wave's weights, loaded with consecutive lanes on
// consecutive records of a row (whole cache lines): for load k, lane l takes
// record q = 64 k + l of the 16 x CG block of the tile, i.e. row q / CG and
// group g0 + q % CG, with its scale bits and zero byte.  At compute time the
// wave stores them in its own LDS area and reads them back in MFMA order.
// They stay in separate registers until then: combining them at load time
// would make the compiler wait for the loads right there.
template <int NT, int CR>
struct WFrag {
  u32x4 c[NT][CR];
  uint32_t s[NT][CR], z[NT][CR];
};

// CG groups per K chunk (CR = CG / 4 records per lane and tile).
template <int MT, int NT, int CG>
__global__ __launch_bounds__(64 * kMaxW) void k_mfma(const DeviceView v, const uint16_t* __restrict__ xw,
                                                     int KW, int64_t M, uint16_t* __restrict__ y) {
  constexpr int BM = 16 * MT;
  constexpr int CR = CG / 4;
  constexpr int CK = 32 * CG;       // bulk positions per chunk
  constexpr int RowH = CK + 8;      // LDS row stride in halves (16 bytes of pad: conflict-free reads)
  constexpr int SEG = CK / 8;       // 16-byte x segments per row and chunk
  constexpr int XS = BM * SEG / 256;  // x segments per thread and chunk (at least 4 waves)
  constexpr int TRS = 16 * CG + 16;                 // LDS row stride of a code tile, bytes
  constexpr int TB = 16 * TRS + 16 * CG * 2 + 16 * CG;  // codes, scales, zero bytes of one tile
  __shared__ __align__(16) uint16_t As[2][BM * RowH];
  __shared__ __align__(16) unsigned char Wt[kMaxW][NT][TB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int nthreads = blockDim.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int W = nthreads >> 6;
  const int r4 = lane >> 4, c = lane & 15;
  const int G = v.G, KP = 32 * G;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int64_t rowA = ((int64_t)blockIdx.x * W + wave) * (16 * NT);  // this wave's first row
  const int64_t left = v.N - rowA;
  const int rows = left <= 0 ? 0 : (left < 16 * NT ? (int)left : 16 * NT);
  const int64_t rows_m = (M - m0) < BM ? (M - m0) : BM;

  // descriptors on this wave's rows and this block's x rows
  const int64_t i0 = (rows > 0 ? rowA : 0) * G;
  const __amdgpu_buffer_rsrc_t rc = rsrc(v.codes + i0, (uint64_t)rows * G * 16);
  const __amdgpu_buffer_rsrc_t rs = rsrc(v.scales + i0, (uint64_t)rows * G * 2);
  const int64_t zb0 = i0 >> 1;
  const __amdgpu_buffer_rsrc_t rz = rsrc(v.zeros + zb0, (uint64_t)(((i0 + (int64_t)rows * G + 1) >> 1) - zb0));
  const __amdgpu_buffer_rsrc_t rx = rsrc(xw + m0 * KW, (uint64_t)rows_m * KW * 2);

  auto load_w = [&](WFrag<NT, CR>& f, int ch) {
#pragma unroll
    for (int k = 0; k < CR; ++k) {
      const int q = 64 * k + lane, row = q / CG, g = ch * CG + q % CG;
      const bool ok = g < G;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint32_t local = (uint32_t)((16 * t + row) * G + g);
        f.c[t][k] = __builtin_amdgcn_raw_buffer_load_b128(rc, ok ? local * 16u : kOob, 0, 0);
        f.s[t][k] = __builtin_amdgcn_raw_buffer_load_b16(rs, ok ? local * 2u : kOob, 0, 0);
        const uint32_t zoff = (uint32_t)(((i0 + local) >> 1) - zb0);
        f.z[t][k] = __builtin_amdgcn_raw_buffer_load_b8(rz, ok ? zoff : kOob, 0, 0);
      }
    }
  };
  // x chunk: BM rows x SEG segments of 8 halves
  auto load_x = [&](u32x4* xr, int ch) {
#pragma unroll
    for (int i = 0; i < XS; ++i) {
      const int seg = tid + nthreads * i;
      const int mrow = seg / SEG, col = ch * CK + 8 * (seg % SEG);
      xr[i] = __builtin_amdgcn_raw_buffer_load_b128(
          rx, (seg < BM * SEG && col < KP) ? (uint32_t)(mrow * KW + col) * 2u : kOob, 0, 0);
    }
  };
  auto store_x = [&](const u32x4* xr, uint16_t* buf) {
#pragma unroll
    for (int i = 0; i < XS; ++i) {
      const int seg = tid + nthreads * i;
      if (seg < BM * SEG) *reinterpret_cast<u32x4*>(buf + (seg / SEG) * RowH + 8 * (seg % SEG)) = xr[i];
    }
  };

  float4_t acc[NT][MT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int tm = 0; tm < MT; ++tm) acc[t][tm] = float4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const WFrag<NT, CR>& f, int ch, const uint16_t* buf) {
    // this wave's records to its LDS tiles, then back in MFMA order: lane
    // (r, c) takes dword r of row c's record for each group of the chunk
    uint32_t R[NT][CG];
    uint32_t sz[NT][CG];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      unsigned char* tile = Wt[wave][t];
#pragma unroll
      for (int k = 0; k < CR; ++k) {
        const int q = 64 * k + lane, row = q / CG, grp = q % CG;
        *reinterpret_cast<u32x4*>(tile + row * TRS + grp * 16) = f.c[t][k];
        reinterpret_cast<uint16_t*>(tile + 16 * TRS)[q] = (uint16_t)f.s[t][k];
        tile[16 * TRS + 32 * CG + q] = (unsigned char)f.z[t][k];
      }
#pragma unroll
      for (int j = 0; j < CG; ++j) {
        R[t][j] = *reinterpret_cast<const uint32_t*>(tile + c * TRS + j * 16 + 4 * r4);
        sz[t][j] = reinterpret_cast<const uint16_t*>(tile + 16 * TRS)[c * CG + j] |
                   ((uint32_t)tile[16 * TRS + 32 * CG + c * CG + j] << 16);
      }
    }
    half8 a[CG][MT];
#pragma unroll
    for (int j = 0; j < CG; ++j)
#pragma unroll
      for (int tm = 0; tm < MT; ++tm)
        a[j][tm] = *reinterpret_cast<const half8*>(buf + (16 * tm + c) * RowH + 32 * j + 8 * r4);
#pragma unroll
    for (int j = 0; j < CG; ++j) {
      const int g = ch * CG + j;
      if (g >= G) break;  // uniform: the last chunk may be partial
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint32_t par = (uint32_t)((i0 + (int64_t)(16 * t + c) * G + g) & 1);
        const uint32_t z = (sz[t][j] >> (16u + 4u * par)) & 0xFu;
        const half8 b = dequant_word(R[t][j], z);
        const float sc = h2f((uint16_t)sz[t][j]);
#pragma unroll
        for (int tm = 0; tm < MT; ++tm) {
          const float4_t p = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[j][tm], b, float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
          acc[t][tm] += sc * p;
        }
      }
    }
  };

  // x chunks run kXD steps ahead in registers (kXD register sets), then go
  // to one of two LDS buffers the step before they are used; weights run
  // 4 chunks ahead (f0 .. f3).  The loop is unrolled by 4 so every register
  // set is addressed at compile time.
  constexpr int kXD = XS >= 4 ? 2 : 4;
  const int nchunk = (G + CG - 1) / CG;
  u32x4 xr[kXD][XS];
  WFrag<NT, CR> f0, f1, f2, f3;
  // prologue in the steady state's issue order (weights, then x, per chunk)
  load_w(f0, 0);
  load_x(xr[0], 0);
  load_w(f1, 1);
  load_x(xr[1 % kXD], 1);
  load_w(f2, 2);
  if constexpr (kXD > 2) load_x(xr[2 % kXD], 2);
  load_w(f3, 3);
  if constexpr (kXD > 3) load_x(xr[3 % kXD], 3);
  store_x(xr[0], As[0]);
  __syncthreads();
  // One step: multiply chunk ch, refill its weight buffer with chunk ch + 4,
  // publish chunk ch + 1's x and request chunk ch + kXD's.
  auto step = [&](WFrag<NT, CR>& f, int ch, u32x4* x_next, u32x4* x_free) {
    compute(f, ch, As[ch & 1]);
    load_w(f, ch + 4);
    store_x(x_next, As[(ch + 1) & 1]);
    load_x(x_free, ch + kXD);
    __syncthreads();
  };
  // The step count is rounded up to a multiple of 4 (steps past the last
  // chunk multiply nothing) so the unrolled body has no early exits: the
  // compiler then keeps exact wait counts across the loop.
  for (int ch = 0; ch < nchunk; ch += 4) {
    step(f0, ch, xr[1 % kXD], xr[0]);
    step(f1, ch + 1, xr[2 % kXD], xr[1 % kXD]);
    step(f2, ch + 2, xr[3 % kXD], xr[2 % kXD]);
    step(f3, ch + 3, xr[0], xr[3 % kXD]);
  }

  // heavy-tailed columns: fp16 weights as they are, scale 1
  const int n_out = v.n_out;
  if (n_out > 0 && rows > 0) {
    const __amdgpu_buffer_rsrc_t ro = rsrc(v.outliers + rowA * n_out, (uint64_t)rows * n_out * 2);
    for (int o0 = 0; o0 < n_out; o0 += 32) {
      half8 a[MT];
#pragma unroll
      for (int tm = 0; tm < MT; ++tm) {
        const u32x4 t4 = __builtin_amdgcn_raw_buffer_load_b128(
            rx, (uint32_t)((16 * tm + c) * KW + KP + o0 + 8 * r4) * 2u, 0, 0);
        a[tm] = __builtin_bit_cast(half8, t4);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = o0 + 8 * r4 + e;
          h[e] = __builtin_amdgcn_raw_buffer_load_b16(
              ro, j < n_out ? (uint32_t)((16 * t + c) * n_out + j) * 2u : kOob, 0, 0);
        }
        const half8 b = __builtin_bit_cast(
            half8, u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)});
#pragma unroll
        for (int tm = 0; tm < MT; ++tm) acc[t][tm] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[tm], b, acc[t][tm], 0, 0, 0);
      }
    }
  }

  // D layout: lane (r, c) holds rows 4r + i of each m-subtile, output column c of each tile
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int64_t n = rowA + 16 * t + c;
    if (n >= v.N) continue;
#pragma unroll
    for (int tm = 0; tm < MT; ++tm) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + 16 * tm + 4 * r4 + i;
        if (m < M) y[m * v.N + n] = f2h(acc[t][tm][i]);
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

namespace {

template <int MT, int NT>
void launch_k(const DeviceView& v, const uint16_t* xw, int KW, int64_t M, uint16_t* y, int W,
              hipStream_t s) {
  constexpr int CG = (NT == 1 && MT <= 2) ? 8 : 4;  // one tile per wave: wider chunks keep more bytes in flight
  const int64_t tiles = (v.N + 15) / 16;
  const int64_t bx = (tiles + (int64_t)W * NT - 1) / ((int64_t)W * NT);
  const int64_t by = (M + 16 * MT - 1) / (16 * MT);
  hipLaunchKernelGGL((k_mfma<MT, NT, CG>), dim3((unsigned)bx, (unsigned)by), dim3(64 * W), 0, s, v, xw, KW, M, y);
}

// Waves per block W (4 .. 8) and 16-row tiles per wave NT so that one block
// row of the grid covers N with about one block per compute unit.
template <int MT>
void launch_mt(const DeviceView& v, const uint16_t* xw, int KW, int64_t M, uint16_t* y, hipStream_t s) {
  constexpr int kNTMax = MT >= 8 ? 1 : (MT >= 4 ? 2 : 4);  // accumulators: NT * MT * 4 registers
  const int64_t tiles = (v.N + 15) / 16;
  const int64_t cu = v.cu_count > 0 ? v.cu_count : 1;
  const int64_t tpc = (tiles + cu - 1) / cu;
  auto clampw = [](int64_t w) { return (int)(w < 4 ? 4 : (w > kMaxW ? kMaxW : w)); };
  if (tpc <= kMaxW || kNTMax == 1) {
    launch_k<MT, 1>(v, xw, KW, M, y, clampw(tpc), s);
  } else if (tpc <= 2 * kMaxW || kNTMax == 2) {
    if constexpr (kNTMax >= 2) launch_k<MT, 2>(v, xw, KW, M, y, clampw((tpc + 1) / 2), s);
  } else {
    if constexpr (kNTMax >= 4) launch_k<MT, 4>(v, xw, KW, M, y, clampw((tpc + 3) / 4), s);
  }
}

}  // namespace

hipError_t launch_mfma_ws(const DeviceView& v, const uint16_t* x, uint16_t* y, int64_t M,
                          void* workspace, hipStream_t s) {
  const int KW = 32 * v.G + ((v.n_out + 31) & ~31);
  uint16_t* xw = static_cast<uint16_t*>(workspace);
  const unsigned gy = (unsigned)(M < 65535 ? M : 65535);
  hipLaunchKernelGGL(k_xbulk, dim3((unsigned)((KW + kThreads - 1) / kThreads), gy),
                     dim3(kThreads), 0, s, v, x, M, xw, KW);
  if (M <= 16) launch_mt<1>(v, xw, KW, M, y, s);
  else if (M <= 32) launch_mt<2>(v, xw, KW, M, y, s);
  else if (M <= 64) launch_mt<4>(v, xw, KW, M, y, s);
  else launch_mt<8>(v, xw, KW, M, y, s);
  return hipGetLastError();
}

}  // namespace spectra
