// SPECTRA batched product for gfx950: y = x W_hat^T on the matrix cores
// (v_mfma_f32_16x16x32_f16): automatic from M = 3 on (the GEMV keeps M <= 2,
// and M <= 4 where the tiled kernel declines), and for shapes the GEMV declines.
//
// The SPECTRA page reports Tensor-Core prefill next to its decode kernels
// (highlight 4); this is the gfx950 counterpart for batched rows, written for
// 64-wide wavefronts and CDNA4 MFMA rather than from the page's kernels.
//
// Pass 1 (k_xbulk): x is permuted once per call into a workspace row per m:
// bulk order, zero padded to 32G, followed by the heavy-tailed x values
// zero padded to a multiple of 32.
//
// Pass 2 is k_mfma_ks (below) when 1 <= M <= 16 and the M rows of x fit in
// LDS, else k_mfma.
//
// k_mfma: a wave owns 16 * NT consecutive output rows for the whole
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


// ---------------------------------------------------------------------------
// k_mfma_ks: the batched product for 1 <= M <= 16 when M rows of x fit in
// LDS.  k_mfma gives each wave 16 rows for the whole K loop, so at any moment
// the chip reads a few records of every row of the matrix: a column-wise
// sweep that opens many DRAM pages for a few bytes each.  Here a block owns a
// tile of 16 consecutive rows at a time (one contiguous stretch of the code
// section) and its 8 waves split the tile's groups between them: wave w takes
// quads of groups w*Q .. w*Q + Q - 1 (a quad is 4 consecutive groups).  Blocks
// walk the tiles b, b + B, b + 2B, ..., so the chip streams one moving window
// of the matrix, as the GEMV does.
//
// Lane (r, c) (r = lane / 16, c = lane % 16) loads the whole record of row c,
// group 4q + r (16 bytes).  A 4 x 4 transpose across the lane quarters and the
// four words (v_permlane32_swap and v_permlane16_swap) leaves lane (r, c)
// holding word r of the records of row c for the four groups of the quad: the
// B operand of v_mfma_f32_16x16x32_f16 (members 8r .. 8r + 7 of row c) for
// each group.  Scales and zero bytes are loaded row-contiguously instead
// (consecutive lanes on consecutive groups of a row: a few cache lines per
// instruction, where one scale per record lane would touch 16 rows) and pass
// through a small wave-private LDS area, from which lane (r, c) reads the four
// scales and zero bytes of row c and the quad.  Each group's product goes into
// a zero accumulator and is added with its fp32 scale, as in k_mfma.  The A
// operand is x in bulk order, read from LDS; lanes of rows m >= M read row
// M - 1, and those output rows are never stored.
// Each wave then holds a partial 16 x 16 product; the waves add theirs through
// LDS (two alternating buffers, one barrier per tile) and M * 16 threads write
// the tile's outputs.  Heavy-tailed columns: wave w takes the 32-column blocks
// w and w + 8 of the fp16 outlier matrix.
constexpr int kKsWaves = 8;
constexpr int kKsThreads = 64 * kKsWaves;
constexpr int kKsXSeg = 24;    // 16-byte x segments per thread staged in one round trip
constexpr int kKsMaxQ = 10;    // quads per wave (G <= 320); more would spill registers
constexpr int kStreamNt = 2;   // cache-policy bit nt on code records (read once)

template <int Q, int OB>
struct KsFrag {
  u32x4 c[Q];
  uint32_t s[Q], z[Q];  // scale and zero byte of element 64 i + lane of the wave's 16 x 4Q groups
  // 8 fp16 heavy-tailed weights per outlier block, one per register until
  // the tile is computed: packing them at load time would wait for the loads
  uint32_t o[OB > 0 ? OB : 1][8];
};

// Lane (r, c) register j <- lane (j, c) register r, for r, j < 4.
__device__ __forceinline__ void transpose4(uint32_t& a0, uint32_t& a1, uint32_t& a2, uint32_t& a3) {
  auto p = __builtin_amdgcn_permlane32_swap(a0, a2, false, false);
  a0 = p[0];
  a2 = p[1];
  p = __builtin_amdgcn_permlane32_swap(a1, a3, false, false);
  a1 = p[0];
  a3 = p[1];
  p = __builtin_amdgcn_permlane16_swap(a0, a1, false, false);
  a0 = p[0];
  a1 = p[1];
  p = __builtin_amdgcn_permlane16_swap(a2, a3, false, false);
  a2 = p[0];
  a3 = p[1];
}

// Wave-private metadata rows: 4Q groups + 4 of padding (keeps the 8-byte
// reads aligned and spreads the 16 rows over the banks).
constexpr int ks_meta_stride(int Q) { return 4 * Q + 4; }
constexpr int ks_meta_bytes(int Q) { return 16 * ks_meta_stride(Q) * 3; }  // u16 scales, then u8 zeros

size_t ks_lds_bytes(int KW, int64_t M, int Q) {
  const size_t mr = (size_t)((M + 3) / 4);
  return (size_t)M * ((size_t)KW + 8) * 2 + 2 * kKsWaves * 16 * mr * 16 + (size_t)kKsWaves * ks_meta_bytes(Q);
}

template <int Q, int OB>
__global__ __launch_bounds__(kKsThreads) void k_mfma_ks(const DeviceView v, const uint16_t* __restrict__ xw,
                                                        int KW, int M, uint16_t* __restrict__ y) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r4 = lane >> 4, c = lane & 15;
  const int G = v.G, n_out = v.n_out;
  const int KP = 32 * G;
  const int nob = (n_out + 31) >> 5;
  const int RS = KW + 8;  // LDS row stride in halves: rows 16 bytes apart mod 128 (conflict-free reads)
  const int MR = (M + 3) >> 2;
  constexpr int MS = ks_meta_stride(Q);
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  float4_t* part = reinterpret_cast<float4_t*>(smem + (size_t)M * RS * 2);  // [2][waves][16 * MR]
  unsigned char* meta = reinterpret_cast<unsigned char*>(part + 2 * kKsWaves * 16 * MR) + w * ks_meta_bytes(Q);
  uint16_t* ms = reinterpret_cast<uint16_t*>(meta);  // [16][MS] scales
  unsigned char* mz = meta + 16 * MS * 2;            // [16][MS] zero bytes
  const int64_t ntiles = (v.N + 15) / 16;
  const int64_t B = gridDim.x;
  int64_t tile = blockIdx.x;

  auto load_tile = [&](KsFrag<Q, OB>& f, int64_t t) {
    const int64_t row0 = t * 16;
    const int64_t left = v.N - row0;
    const int rows = left <= 0 ? 0 : (left < 16 ? (int)left : 16);
    const int64_t i0 = (rows > 0 ? row0 : 0) * G;
    const __amdgpu_buffer_rsrc_t rc = rsrc(v.codes + i0, (uint64_t)rows * G * 16);
    const __amdgpu_buffer_rsrc_t rs = rsrc(v.scales + i0, (uint64_t)rows * G * 2);
    const int64_t zb0 = i0 >> 1;
    const uint32_t i0odd = (uint32_t)(i0 & 1);
    const __amdgpu_buffer_rsrc_t rz = rsrc(v.zeros + zb0, (uint64_t)(((i0 + (int64_t)rows * G + 1) >> 1) - zb0));
#pragma unroll
    for (int i = 0; i < Q; ++i) {
      const int g = 4 * (w * Q + i) + r4;
      const bool ok = g < G;  // a group past G would be the next row's
      const uint32_t local = (uint32_t)(c * G + g);
      f.c[i] = __builtin_amdgcn_raw_buffer_load_b128(rc, ok ? local * 16u : kOob, 0, kStreamNt);
    }
#pragma unroll
    for (int i = 0; i < Q; ++i) {
      const int e = 64 * i + lane, row = e / (4 * Q), g = 4 * w * Q + e % (4 * Q);
      const bool ok = g < G;
      const uint32_t local = (uint32_t)(row * G + g);
      f.s[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, ok ? local * 2u : kOob, 0, 0);
      f.z[i] = __builtin_amdgcn_raw_buffer_load_b8(rz, ok ? (local + i0odd) >> 1 : kOob, 0, 0);
    }
    if constexpr (OB > 0) {
      const __amdgpu_buffer_rsrc_t ro =
          rsrc(v.outliers + (rows > 0 ? row0 : 0) * n_out, (uint64_t)rows * n_out * 2);
#pragma unroll
      for (int k = 0; k < OB; ++k) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = 32 * (w + kKsWaves * k) + 8 * r4 + e;
          f.o[k][e] = __builtin_amdgcn_raw_buffer_load_b16(ro, j < n_out ? (uint32_t)(c * n_out + j) * 2u : kOob, 0, 0);
        }
      }
    }
  };

  // x rows in bulk order from the workspace: every thread's segments in one
  // round trip, the block's first tile requested right behind them.
  KsFrag<Q, OB> fa, fb;
  {
    const int segs_row = KW >> 3;
    const int nseg = M * segs_row;
    const __amdgpu_buffer_rsrc_t rx = rsrc(xw, (uint64_t)M * KW * 2);
    u32x4 xv[kKsXSeg];
#pragma unroll
    for (int i = 0; i < kKsXSeg; ++i) {
      if (i * kKsThreads >= nseg) break;  // block-uniform
      const int s = tid + kKsThreads * i;
      xv[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, s < nseg ? (uint32_t)s * 16u : kOob, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    load_tile(fa, tile);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kKsXSeg; ++i) {
      if (i * kKsThreads >= nseg) break;
      const int s = tid + kKsThreads * i;
      if (s < nseg) {
        const int m = s / segs_row, col = s - m * segs_row;
        *reinterpret_cast<u32x4*>(xs + m * RS + 8 * col) = xv[i];
      }
    }
  }
  __syncthreads();

  const uint16_t* xa = xs + (c < M ? c : M - 1) * RS + 8 * r4;  // this lane's A row (rows past M: not stored)
  // Straight-line compute (no exit past the last group: groups past G load
  // zero codes, zeros and scales and add exactly 0) lets the scheduler overlap
  // one quad's loads and products with the next quad's; it takes more
  // registers, so it is used where it still fits without spills.
  constexpr bool kFlat = OB == 0 ? Q <= 5 : (OB == 1 ? Q <= 8 : Q <= 6);
  auto compute = [&](const KsFrag<Q, OB>& f, int64_t t) {
    float4_t acc = float4_t{0.f, 0.f, 0.f, 0.f};
    const uint32_t rowpar = (uint32_t)(((t * 16 + c) * (int64_t)G) & 1);  // flat index parity at group 0
    // this tile's scales and zero bytes through the wave's LDS rows (the
    // previous tile's reads come first in this wave's LDS order)
#pragma unroll
    for (int i = 0; i < Q; ++i) {
      const int e = 64 * i + lane, row = e / (4 * Q), grp = e % (4 * Q);
      ms[row * MS + grp] = (uint16_t)f.s[i];
      mz[row * MS + grp] = (unsigned char)f.z[i];
    }
#pragma unroll
    for (int i = 0; i < Q; ++i) {
      const int gq = 4 * (w * Q + i);
      if constexpr (!kFlat)
        if (gq >= G) break;  // wave-uniform
      uint32_t R[4] = {f.c[i].x, f.c[i].y, f.c[i].z, f.c[i].w};
      transpose4(R[0], R[1], R[2], R[3]);
      const uint2 s4 = *reinterpret_cast<const uint2*>(ms + c * MS + 4 * i);
      const uint32_t z4 = *reinterpret_cast<const uint32_t*>(mz + c * MS + 4 * i);
      const uint32_t S[4] = {s4.x, s4.x >> 16, s4.y, s4.y >> 16};
      float4_t p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (!kFlat)
          if (gq + j >= G) break;
        // past G (straight-line form only) any x slot of the row will do
        const int ga = gq + j < G ? gq + j : (G > 0 ? G - 1 : 0);
        const uint32_t par = (rowpar ^ (uint32_t)(gq + j)) & 1u;
        const uint32_t z = (z4 >> (8u * j + 4u * par)) & 0xFu;
        const half8 b = dequant_word(R[j], z);
        const half8 a = *reinterpret_cast<const half8*>(xa + 32 * ga);
        p[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (!kFlat)
          if (gq + j >= G) break;
        acc += h2f((uint16_t)S[j]) * p[j];
      }
    }
    if constexpr (OB > 0) {
#pragma unroll
      for (int k = 0; k < OB; ++k) {
        const int ob = w + kKsWaves * k;
        if (ob < nob) {
          const half8 a = *reinterpret_cast<const half8*>(xa + KP + 32 * ob);
          const uint32_t* o = f.o[k];
          const half8 b = __builtin_bit_cast(
              half8, u32x4{o[0] | (o[1] << 16), o[2] | (o[3] << 16), o[4] | (o[5] << 16), o[6] | (o[7] << 16)});
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
        }
      }
    }
    return acc;
  };
  // Sum of the waves' partials for tile t: D lane (r, c) holds rows m = 4r + i
  // of output column c; lanes r < MR carry the rows m < M.
  auto reduce = [&](const float4_t acc, int64_t t, int buf) {
    float4_t* pb = part + buf * kKsWaves * 16 * MR;
    if (lane < 16 * MR) pb[w * 16 * MR + lane] = acc;
    __syncthreads();
    if (tid < 16 * M) {
      const int m = tid >> 4, n = tid & 15;
      const float* pf = reinterpret_cast<const float*>(pb) + ((m >> 2) * 16 + n) * 4 + (m & 3);
      float sum = 0.f;
#pragma unroll
      for (int ww = 0; ww < kKsWaves; ++ww) sum += pf[ww * 16 * MR * 4];
      const int64_t row = t * 16 + n;
      if (row < v.N) y[(int64_t)m * v.N + row] = f2h(sum);
    }
  };
  // Two register buffers: a buffer is refilled as soon as its tile has been
  // multiplied, before the barrier of the cross-wave sum, so two tiles stay in
  // flight while the waves wait for one another; no early exit sits between a
  // load and its use.
  load_tile(fb, tile + B);
  for (; tile < ntiles; tile += 2 * B) {
    __builtin_amdgcn_sched_barrier(0);
    float4_t acc = compute(fa, tile);
    __builtin_amdgcn_sched_barrier(0);
    load_tile(fa, tile + 2 * B);
    __builtin_amdgcn_sched_barrier(0);
    reduce(acc, tile, 0);
    // unconditional, so the wait counts are the same on every path (a tile
    // past the end multiplies zeros and is not stored)
    acc = compute(fb, tile + B);
    __builtin_amdgcn_sched_barrier(0);
    load_tile(fb, tile + 3 * B);
    __builtin_amdgcn_sched_barrier(0);
    if (tile + B < ntiles) reduce(acc, tile + B, 1);
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

struct KsShape {
  int Q, OB;  // quads of groups per wave, heavy-tailed blocks per wave
};
KsShape ks_shape(const DeviceView& v) {
  const int quads = (v.G + 3) / 4;
  const int q = (quads + kKsWaves - 1) / kKsWaves;
  const int nob = (v.n_out + 31) / 32;
  return KsShape{q < 1 ? 1 : q, (nob + kKsWaves - 1) / kKsWaves};
}

template <int Q, int OB>
hipError_t launch_ks_q(const DeviceView& v, const uint16_t* xw, int KW, int64_t M, uint16_t* y, hipStream_t s) {
  const size_t lds = ks_lds_bytes(KW, M, Q);
  if (lds > 64 * 1024) {  // dynamic LDS past 64 KiB must be allowed per kernel
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_mfma_ks<Q, OB>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int64_t tiles = (v.N + 15) / 16;
  const int64_t cu = v.cu_count > 0 ? v.cu_count : 1;
  const unsigned blocks = (unsigned)(tiles < cu ? tiles : cu);
  hipLaunchKernelGGL((k_mfma_ks<Q, OB>), dim3(blocks), dim3(kKsThreads), lds, s, v, xw, KW, (int)M, y);
  return hipGetLastError();
}

template <int OB>
hipError_t launch_ks_ob(int Q, const DeviceView& v, const uint16_t* xw, int KW, int64_t M, uint16_t* y,
                        hipStream_t s) {
  switch (Q) {
    case 1: return launch_ks_q<1, OB>(v, xw, KW, M, y, s);
    case 2: return launch_ks_q<2, OB>(v, xw, KW, M, y, s);
    case 3: return launch_ks_q<3, OB>(v, xw, KW, M, y, s);
    case 4: return launch_ks_q<4, OB>(v, xw, KW, M, y, s);
    case 5: return launch_ks_q<5, OB>(v, xw, KW, M, y, s);
    case 6: return launch_ks_q<6, OB>(v, xw, KW, M, y, s);
    case 7: return launch_ks_q<7, OB>(v, xw, KW, M, y, s);
    case 8: return launch_ks_q<8, OB>(v, xw, KW, M, y, s);
    case 9: return launch_ks_q<9, OB>(v, xw, KW, M, y, s);
    case 10: return launch_ks_q<10, OB>(v, xw, KW, M, y, s);
    default: return hipErrorNotSupported;
  }
}

size_t ks_lds_limit(const DeviceView& v) {
  const size_t dev = v.lds_per_block > 0 ? (size_t)v.lds_per_block : 64 * 1024;
  return dev < (size_t)160 * 1024 ? dev : (size_t)160 * 1024;
}

// The tiled kernel runs 1 <= M <= 16 when the M rows of x, the partial sums
// and the metadata rows fit in LDS and two tiles fit in registers without
// spills: Q + OB <= 10 (G <= 320 with no heavy-tailed columns; each further
// heavy-tailed block per wave takes the place of one quad).
bool ks_supports(const DeviceView& v, int KW, int64_t M) {
  if (M < 1 || M > 16) return false;
  const KsShape sh = ks_shape(v);
  if (sh.Q > kKsMaxQ || sh.OB > 2 || sh.Q + sh.OB > kKsMaxQ) return false;  // past these: register spills
  if ((int64_t)M * KW * 2 >= 0x7FFFFFFF || (int64_t)M * (KW / 8) > (int64_t)kKsXSeg * kKsThreads) return false;
  return ks_lds_bytes(KW, M, sh.Q) <= ks_lds_limit(v);
}

hipError_t launch_ks(const DeviceView& v, const uint16_t* xw, int KW, int64_t M, uint16_t* y, hipStream_t s) {
  const KsShape sh = ks_shape(v);
  switch (sh.OB) {
    case 0: return launch_ks_ob<0>(sh.Q, v, xw, KW, M, y, s);
    case 1: return launch_ks_ob<1>(sh.Q, v, xw, KW, M, y, s);
    default: return launch_ks_ob<2>(sh.Q, v, xw, KW, M, y, s);
  }
}

}  // namespace

bool mfma_tiled_supports(const DeviceView& v, int64_t M) {
  return ks_supports(v, 32 * v.G + ((v.n_out + 31) & ~31), M);
}

hipError_t launch_mfma_ws(const DeviceView& v, const uint16_t* x, uint16_t* y, int64_t M,
                          void* workspace, hipStream_t s) {
  const int KW = 32 * v.G + ((v.n_out + 31) & ~31);
  uint16_t* xw = static_cast<uint16_t*>(workspace);
  const unsigned gy = (unsigned)(M < 65535 ? M : 65535);
  hipLaunchKernelGGL(k_xbulk, dim3((unsigned)((KW + kThreads - 1) / kThreads), gy),
                     dim3(kThreads), 0, s, v, x, M, xw, KW);
  if (ks_supports(v, KW, M)) return launch_ks(v, xw, KW, M, y, s);
  if (M <= 16) launch_mt<1>(v, xw, KW, M, y, s);
  else if (M <= 32) launch_mt<2>(v, xw, KW, M, y, s);
  else if (M <= 64) launch_mt<4>(v, xw, KW, M, y, s);
  else launch_mt<8>(v, xw, KW, M, y, s);
  return hipGetLastError();
}

}  // namespace spectra
