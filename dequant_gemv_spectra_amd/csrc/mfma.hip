// SPECTRA batched product for gfx950: y = x W_hat^T on the matrix cores
// (v_mfma_f32_16x16x32_f16): automatic from M = 3 on (the GEMV keeps M <= 2,
// and M <= 4 where only the strip kernel would take the shape), and for
// shapes the GEMV declines.
//
// The SPECTRA page reports Tensor-Core prefill next to its decode kernels
// (highlight 4); this is the gfx950 counterpart for batched rows, written for
// 64-wide wavefronts and CDNA4 MFMA rather than from the page's kernels.
//
// Pass 1 (k_xbulk): x is permuted once per call into a workspace row per m:
// bulk order, zero padded to 32G, followed by the heavy-tailed x values
// zero padded to a multiple of 32.
//
// Pass 2 is one of three kernels: k_mfma_sk + k_sk_sum (split-K, below;
// the default for M <= 16 where it takes the shape), k_mfma_ks (16-row tiles
// with the M rows of x in LDS) or k_mfma (one 16-row strip per wave).
//
// k_mfma: a wave owns 16 * NT consecutive output rows for the whole
// K loop.  Per chunk of CG groups it loads its code records row-contiguously
// (consecutive lanes on consecutive records of a row: whole cache lines),
// stores them to a small wave-private LDS tile and reads them back in the
// B-operand order of v_mfma_f32_16x16x32_f16: lane (r, c) takes dword r of
// row c's record, members 8r .. 8r + 7 of the group.  The dword is
// dequantized in registers to exact fp16 (q - z): (w & 0x000F000F) | 0x6400
// 6400 holds 1024 + q of two members, (w & 0x00F000F0) | 0x5400 5400 holds
// 64 + q of the next two, and subtracting 1024 + z or 64 + z is exact.  The
// B operand is then fp16(s16 * (q - z)): each dequantized weight rounded once
// to fp16, the tensor-core form of the weights, and one MFMA per group and
// m-subtile accumulates straight into the fp32 sum, with no vector-ALU work
// between MFMAs.  The rounding adds at most 2^-11 |w_hat| per weight (2^-25
// absolute below fp16's normal range), inside the product's tolerance
// 1e-3 |W_hat| |x|.  A row whose scales reach 4096 (15 s16 could pass fp16's
// range) switches, from the first such group on, to operands scaled by
// 2^-12: its running sum is multiplied by 2^-12 once (exact) and its outputs
// by 2^12 at the store.  A block is 7 compute waves and one loader wave:
// the loader streams the A operand (x in bulk order, 16*MT rows x 32*CG
// positions per chunk) into a ring of 4 LDS buffers by LDS-DMA, three
// chunks ahead of the compute waves, and a barrier per chunk hands each
// buffer over; the compute waves keep their weights 4 chunks ahead in
// registers and issue no other loads in the loop.  The
// heavy-tailed columns follow as plain MFMA steps (fp16 weights, scale 1).
// Loads use buffer descriptors: rows past N or M and positions past the
// padded K read as zero.
#include "../../include/spectra.h"
#include "spectra_internal.h"

namespace spectra {
namespace {

constexpr int kThreads = 256;   // k_xbulk
constexpr int kRsrcWord3 = 0x00020000;
constexpr uint32_t kOob = 0x80000000u;
constexpr int kStreamNt = 2;   // cache-policy bit nt on code records (read once)

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

// Scales of 4096 and more: 15 s16 may pass 65504, fp16's largest finite value
// (scales are never negative, so their bits compare as integers).
constexpr uint32_t kBigScale = 0x6C00u;  // fp16 bits of 4096
constexpr float kDown = 1.0f / 4096.0f;

// The 8 members times the group's scale and the row's exponent factor (1 or
// 2^-12), rounded once to fp16 (the factor makes the scale's product exact
// when it is 1; in a row of huge scales, where it is 2^-12, the tolerance is
// as large as the weights).
__device__ __forceinline__ half8 scale8(half8 d, uint32_t s16, _Float16 em) {
  const _Float16 sh = __builtin_bit_cast(_Float16, (uint16_t)s16) * em;
  return d * sh;
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

// One LDS-DMA instruction: lane l's 16 bytes at buffer offset `off` land at
// LDS byte lds + 16 l (buffer_load_dwordx4 ... lds).  Inline assembly, so
// the compiler neither waits on it before LDS reads nor drains it at
// barriers; the issuing wave counts its own instructions.  M0 is saved and
// restored; the leading s_nop keeps SGPR operands written by a VALU
// instruction just before at the required distance.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t off) {
  uint32_t save;
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "s"(lds), "v"(off), "s"(r)
      : "memory");
}

// Waits until at most n of this wave's vector memory operations are
// outstanding (n is a compile-time count up to 63).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Block barrier for LDS hand-offs that leaves vector memory operations in
// flight (this wave's LDS accesses complete first).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

constexpr int kMfmaCW = 7;                  // compute waves of k_mfma
constexpr int kMfmaThreads = 64 * (kMfmaCW + 1);  // plus the loader wave
constexpr int kXRing = 4;                   // x chunk buffers: the loader runs 3 chunks ahead

// LDS-DMA instructions of the loader per x chunk: 16 MT rows of 32 CG
// positions (4 CG 16-byte segments) plus one pad slot per row.
template <int MT, int CG>
constexpr int mfma_nx() {
  return (16 * MT * (4 * CG + 1) + 63) / 64;
}
// Every instruction writes a whole 1 KB block, so a ring buffer is NX blocks.
template <int MT, int CG>
constexpr size_t mfma_lds_bytes() {
  return (size_t)kXRing * mfma_nx<MT, CG>() * 1024;
}

// CG groups per K chunk (CR = CG / 4 records per lane and tile).  Waves
// 0 .. 6 compute (16 NT rows each), wave 7 streams x.
template <int MT, int NT, int CG>
__global__ __launch_bounds__(kMfmaThreads) void k_mfma(const DeviceView v, const uint16_t* __restrict__ xw,
                                                       int KW, int64_t M, uint16_t* __restrict__ y) {
  constexpr int BM = 16 * MT;
  constexpr int CR = CG / 4;
  constexpr int CK = 32 * CG;       // bulk positions per chunk
  constexpr int RowH = CK + 8;      // LDS row stride in halves (16 bytes of pad: conflict-free reads)
  constexpr int SEG = CK / 8;       // 16-byte x segments per row and chunk
  constexpr int SLOTS = BM * (SEG + 1);   // LDS slots of one chunk (pad slot per row)
  constexpr int NX = mfma_nx<MT, CG>();   // loader DMA instructions per chunk
  constexpr int XB = NX * 512;            // halves per ring buffer (whole 1 KB blocks)
  static_assert(NX * 64 >= SLOTS, "slots");
  constexpr int XWAIT = 2 * NX < 63 ? 2 * NX : 63;  // the loader's wait: two later chunks may stay in flight
  constexpr int TRS = 16 * CG + 16;                 // LDS row stride of a code tile, bytes
  constexpr int TB = 16 * TRS + 16 * CG * 2 + 16 * CG;  // codes, scales, zero bytes of one tile
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* As = reinterpret_cast<uint16_t*>(smem);  // [kXRing][XB]: rows of RowH halves
  __shared__ __align__(16) unsigned char Wt[kMfmaCW][NT][TB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r4 = lane >> 4, c = lane & 15;
  const int G = v.G, KP = 32 * G;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int64_t rows_m = (M - m0) < BM ? (M - m0) : BM;
  const __amdgpu_buffer_rsrc_t rx = rsrc(xw + m0 * KW, (uint64_t)rows_m * KW * 2);
  const int nchunk = (G + CG - 1) / CG;
  const int nsteps = (nchunk + 15) & ~15;  // the compute loop is unrolled by 16

  if (wave == kMfmaCW) {
    // loader: chunk ch of x (rows m0 .. m0 + BM - 1, positions ch CK ..) into
    // ring buffer ch % 4, slot s = (row, segment) with one pad slot per row;
    // chunks past the last one (and positions past 32G) read zeros, so every
    // step issues the same NX instructions and the wait counts hold
    const uint32_t ring = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)(smem);
    auto issue = [&](int ch) {
      const uint32_t base = ring + (uint32_t)((ch & (kXRing - 1)) * XB * 2);
#pragma unroll
      for (int k = 0; k < NX; ++k) {
        const int s = 64 * k + lane, row = s / (SEG + 1), sg = s % (SEG + 1);
        const int col = ch * CK + 8 * sg;
        const bool ok = s < SLOTS && sg < SEG && col < KP;
        dma16(rx, base + 1024u * (uint32_t)k, ok ? (uint32_t)(row * KW + col) * 2u : kOob);
      }
    };
    issue(0);
    issue(1);
    issue(2);
    for (int ch = 0; ch < nsteps; ++ch) {
      vm_wait<XWAIT>();  // chunk ch has landed
      lds_barrier();     // step ch: chunk ch is visible; buffer (ch + 3) % 4 is free
      issue(ch + 3);
    }
    return;
  }

  const int64_t rowA = ((int64_t)blockIdx.x * kMfmaCW + wave) * (16 * NT);  // this wave's first row
  const int64_t left = v.N - rowA;
  const int rows = left <= 0 ? 0 : (left < 16 * NT ? (int)left : 16 * NT);
  // descriptors on this wave's rows
  const int64_t i0 = (rows > 0 ? rowA : 0) * G;
  const __amdgpu_buffer_rsrc_t rc = rsrc(v.codes + i0, (uint64_t)rows * G * 16);
  const __amdgpu_buffer_rsrc_t rs = rsrc(v.scales + i0, (uint64_t)rows * G * 2);
  const int64_t zb0 = i0 >> 1;
  const __amdgpu_buffer_rsrc_t rz = rsrc(v.zeros + zb0, (uint64_t)(((i0 + (int64_t)rows * G + 1) >> 1) - zb0));

  auto load_w = [&](WFrag<NT, CR>& f, int ch) {
#pragma unroll
    for (int k = 0; k < CR; ++k) {
      const int q = 64 * k + lane, row = q / CG, g = ch * CG + q % CG;
      const bool ok = g < G;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint32_t local = (uint32_t)((16 * t + row) * G + g);
        f.c[t][k] = __builtin_amdgcn_raw_buffer_load_b128(rc, ok ? local * 16u : kOob, 0, kStreamNt);
        f.s[t][k] = __builtin_amdgcn_raw_buffer_load_b16(rs, ok ? local * 2u : kOob, 0, 0);
        const uint32_t zoff = (uint32_t)(((i0 + local) >> 1) - zb0);
        f.z[t][k] = __builtin_amdgcn_raw_buffer_load_b8(rz, ok ? zoff : kOob, 0, 0);
      }
    }
  };

  float4_t acc[NT][MT];
  _Float16 em[NT];  // this lane's row of tile t: operand factor (1, or 2^-12 once a scale reached 4096)
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    em[t] = (_Float16)1.0f;
#pragma unroll
    for (int tm = 0; tm < MT; ++tm) acc[t][tm] = float4_t{0.f, 0.f, 0.f, 0.f};
  }

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
    // a row meeting its first huge scale: sum so far times 2^-12, operands from now on too
    bool hit[NT];
    bool any = false;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      hit[t] = false;
#pragma unroll
      for (int j = 0; j < CG; ++j) hit[t] |= (sz[t][j] & 0xFFFFu) >= kBigScale;
      hit[t] = hit[t] && em[t] == (_Float16)1.0f;
      any |= hit[t];
    }
    if (__builtin_expect(__ballot(any) != 0, 0)) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
        if (hit[t]) {
          em[t] = (_Float16)kDown;
#pragma unroll
          for (int tm = 0; tm < MT; ++tm) acc[t][tm] *= kDown;
        }
    }
#pragma unroll
    for (int j = 0; j < CG; ++j) {
      const int g = ch * CG + j;
      if (g >= G) break;  // uniform: the last chunk may be partial
      half8 a[MT];  // x of group j for each m-subtile
#pragma unroll
      for (int tm = 0; tm < MT; ++tm)
        a[tm] = *reinterpret_cast<const half8*>(buf + (16 * tm + c) * RowH + 32 * j + 8 * r4);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint32_t par = (uint32_t)((i0 + (int64_t)(16 * t + c) * G + g) & 1);
        const uint32_t z = (sz[t][j] >> (16u + 4u * par)) & 0xFu;
        const half8 b = scale8(dequant_word(R[t][j], z), sz[t][j] & 0xFFFFu, em[t]);
#pragma unroll
        for (int tm = 0; tm < MT; ++tm)
          acc[t][tm] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[tm], b, acc[t][tm], 0, 0, 0);
      }
    }
  };

  // Weights run 4 chunks ahead in registers (f0 .. f3); x chunk ch is in
  // ring buffer ch % 4 from step ch's barrier on.  The loop is unrolled by
  // 16 so every register set is addressed at compile time and the compiler
  // keeps exact wait counts for the weights inside an iteration (at the loop
  // header it waits for every load in flight: once per 16 chunks); steps
  // past the last chunk multiply nothing, and no step exits early.
  WFrag<NT, CR> f0, f1, f2, f3;
  load_w(f0, 0);
  load_w(f1, 1);
  load_w(f2, 2);
  load_w(f3, 3);
  auto step = [&](WFrag<NT, CR>& f, int ch) {
    lds_barrier();
    compute(f, ch, As + (ch & (kXRing - 1)) * XB);
    load_w(f, ch + 4);
  };
  for (int ch = 0; ch < nsteps; ch += 16) {
#pragma unroll
    for (int u = 0; u < 16; u += 4) {
      step(f0, ch + u);
      step(f1, ch + u + 1);
      step(f2, ch + u + 2);
      step(f3, ch + u + 3);
    }
  }

  // heavy-tailed columns: fp16 weights as they are (times the row's factor)
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
            half8, u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)}) * em[t];
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
        if (m < M) y[m * v.N + n] = f2h(em[t] == (_Float16)1.0f ? acc[t][tm][i] : acc[t][tm][i] * 4096.0f);
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
// a zero accumulator and is added with its fp32 scale: at these M the
// products are short and the scale FMAs overlap the next group's MFMA
// (fp16(s16 (q - z)) operands accumulated by the MFMAs, as k_mfma does,
// measured 51.5 -> 56.1 us at 28672 x 8192, M = 8).  The A
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

// ---------------------------------------------------------------------------
// k_mfma_sk: the batched product for 1 <= M <= 16 with K split into S ranges
// of KR = 16 WG <= 128 groups.  The other kernels stream a few records of
// many rows per load instruction (16 rows x 64 bytes, or 8 rows x 128
// bytes), and this chip's memory system serves those at 4.0 - 4.9 TB/s where
// one row's 1 KB per instruction streams at 6 TB/s.  Here each block takes
// one K-range and walks 16-row tiles t0, t0 + B / S, ...; the S blocks on
// the ranges of one tile are 8 apart (one XCD, see below), so the chip still
// streams one moving window of the code section.  Each of the 16 waves moves one row
// of a tile per step into an LDS ring by LDS-DMA: its records of the range in
// two 1 KB instructions, its scales and its zero bytes in one 16-byte-per-lane
// instruction each; the ring holds 3 tiles, 2 of them in flight while one is
// computed.  Wave w keeps x of its WG groups (all 16 rows) as MFMA A operands
// in registers for the whole launch, so x is read from memory once per block
// and never passes through LDS.  Per group: lane (r, c) reads word r of row
// c's record from the tile, dequantizes it to exact fp16 (q - z), one MFMA
// into a zero accumulator, and adds it with the group's fp32 scale (the exact
// form of k_mfma_ks).  The waves' 16 x 16 partials of a tile are summed
// through LDS in fixed order and stored as fp32 to the workspace, P[s][m][n];
// k_sk_sum adds the S ranges in order and the heavy-tailed columns.
constexpr int kSkWaves = 16;  // 4 per SIMD: the LDS -> MFMA -> FMA chains of one hide behind the others
constexpr int kSkThreads = 64 * kSkWaves;
constexpr int kSkRow = 2064;   // LDS bytes per code row of a tile: 2 x 1 KB of DMA + 16 of pad (rows 4 banks apart)
constexpr int kSkCodes = 16 * kSkRow;
constexpr int kSkSRow = 272;   // per scale row: 17 x 16 bytes holding its KR scales from the dword of its first (68 banks apart)
constexpr int kSkScales = 16 * kSkSRow;
constexpr int kSkZWave = 80;   // per wave: 5 x 16 bytes holding its row's zero bytes (rows 20 banks apart)
constexpr int kSkZeros = kSkWaves * kSkZWave;
constexpr int kSkSlot = kSkCodes + kSkScales + kSkZeros;
constexpr int kSkDma = 4;      // DMA instructions per wave and tile
template <int MT>
constexpr int sk_ring() {
  return 3;
}
template <int MT>
constexpr size_t sk_lds_bytes() {
  return (size_t)sk_ring<MT>() * kSkSlot + 2 * kSkWaves * MT * 1024;
}

// One 4-byte LDS-DMA instruction: active lane l's dword at `off` lands at
// lds + 4 l (inactive lanes write nothing).
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t off) {
  uint32_t save;
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "s"(lds), "v"(off), "s"(r)
      : "memory");
}

// dma16 with the non-temporal hint (code records are read once).
__device__ __forceinline__ void dma16_nt(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t off) {
  uint32_t save;
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen nt lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "s"(lds), "v"(off), "s"(r)
      : "memory");
}

__host__ __device__ constexpr uint64_t round4(uint64_t b) { return (b + 3) & ~(uint64_t)3; }

template <int MT>
struct SkAcc {
  float4_t a[MT];
};

template <int MT, int WG>
__global__ __launch_bounds__(kSkThreads) void k_mfma_sk(const DeviceView v, const uint16_t* __restrict__ xw,
                                                        int KW, int M, int S, float* __restrict__ P) {
  constexpr int KR = kSkWaves * WG;
  constexpr int R = sk_ring<MT>();
  constexpr int D = R - 1;  // tiles in flight while one is computed
  static_assert(WG >= 1 && WG <= 8 && MT == 1, "groups per wave, m-subtiles");
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r4 = lane >> 4, c = lane & 15;
  const int G = v.G;
  const int64_t N = v.N;
  // Blocks are dispatched to the 8 XCDs in turn (block b on XCD b % 8).  When
  // the grid is a multiple of 8 S, the S ranges of a tile go to blocks 8
  // apart, i.e. to one XCD, whose L2 then serves the cache lines two ranges
  // (and two rows) share; else to consecutive blocks.
  const unsigned bid = blockIdx.x;
  const bool xcd = gridDim.x % (8u * (unsigned)S) == 0;
  const unsigned lane8 = bid & 7u, j8 = bid >> 3;
  const int s = (int)(xcd ? j8 % (unsigned)S : bid % (unsigned)S);
  const int64_t Bs = gridDim.x / S;
  const int64_t ntiles = (N + 15) / 16;
  const int g0 = KR * s;
  const int gw = g0 + WG * w;  // this wave's first group
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)(smem);
  float4_t* part = reinterpret_cast<float4_t*>(smem + R * kSkSlot);  // [2][waves][MT][64]
  const uint64_t NG = (uint64_t)N * (uint64_t)G;
  const __amdgpu_buffer_rsrc_t rc = rsrc(v.codes, NG * 16);
  // 16-byte DMAs: a load straddling a descriptor's end would read as zeros
  // in full, so the ranges are rounded up (sections are 256-byte padded)
  const __amdgpu_buffer_rsrc_t rs = rsrc(v.scales, (NG * 2 + 15) & ~15ull);
  const __amdgpu_buffer_rsrc_t rz = rsrc(v.zeros, ((NG + 1) / 2 + 15) & ~15ull);

  // Tile t into ring slot `slot`: this wave's rows 2w and 2w + 1 (the row
  // index is wave-uniform, so the offsets are a scalar base plus the lane).
  // Every wave issues kSkDma instructions per tile, past the last tile too
  // (all lanes out of range), so the wait counts are the same on every path.
  // Offsets fit 31 bits (the launcher checks N G 16).
  auto issue = [&](int64_t t, int slot) {
    const uint32_t base = lds0 + (uint32_t)(slot * kSkSlot);
    const int64_t r0 = t * 16 + w;
    const bool ok0 = t < ntiles && r0 < N;
    const uint32_t f0 = (uint32_t)(r0 * G + g0);
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // the row's records of the range, 1 KB per instruction
      const int gl = 64 * h + lane;
      const bool lc = gl < KR && g0 + gl < G;
      dma16_nt(rc, base + (uint32_t)(w * kSkRow + 1024 * h), ok0 && lc ? (f0 + gl) * 16u : kOob);
    }
    // scales from the dword holding the row's first (a row starts mid-dword
    // when its flat index is odd), and the zero nibbles from the dword
    // holding its first
    if (lane < 17) dma16(rs, base + (uint32_t)(kSkCodes + w * kSkSRow), ok0 ? ((f0 >> 1) + 4 * lane) * 4u : kOob);
    if (lane < 5)
      dma16(rz, base + (uint32_t)(kSkCodes + kSkScales + w * kSkZWave), ok0 ? (((f0 >> 1) & ~3u) + 16u * lane) : kOob);
  };

  const int64_t t0 = xcd ? (int64_t)(j8 / (unsigned)S) * 8 + lane8 : (int64_t)(bid / (unsigned)S);
#pragma unroll
  for (int d = 0; d < D; ++d) issue(t0 + d * Bs, d);

  // x of this wave's groups: A operand lane (r, c) = row 16 tm + c, positions
  // 8r .. 8r + 7 of the group; rows past M and groups past G read zeros.
  half8 xa[WG][MT];
  {
    const __amdgpu_buffer_rsrc_t rx = rsrc(xw, (uint64_t)M * KW * 2);
#pragma unroll
    for (int j = 0; j < WG; ++j)
#pragma unroll
      for (int tm = 0; tm < MT; ++tm) {
        const int m = 16 * tm + c, g = gw + j;
        const bool ok = m < M && g < G;
        xa[j][tm] = __builtin_bit_cast(
            half8, __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? (uint32_t)(m * KW + 32 * g + 8 * r4) * 2u : kOob, 0, 0));
      }
    // consume x here, before the loop: the compiler waits for these loads
    // (and so for the first tiles) once, not inside the loop
#pragma unroll
    for (int j = 0; j < WG; ++j)
#pragma unroll
      for (int tm = 0; tm < MT; ++tm) asm volatile("" ::"v"(xa[j][tm]));
  }

  auto compute = [&](int slot, int64_t t) {
    SkAcc<MT> acc;
    const unsigned char* base = smem + slot * kSkSlot;
    const int64_t n0 = (t * 16 + c) * G + g0;  // flat index of the row's first group of the range
    const int ph = (int)(n0 & 1);
    const int zq = (int)(n0 & 7) + WG * w;  // this wave's first zero nibble from the row's first dword
    const int zb = zq >> 1;
    const unsigned char* zr = base + kSkCodes + kSkScales + c * kSkZWave;
    const uint32_t z0 = *reinterpret_cast<const uint32_t*>(zr + (zb & ~3));
    const uint32_t z1 = *reinterpret_cast<const uint32_t*>(zr + (zb & ~3) + 4);
    const uint32_t z2 = *reinterpret_cast<const uint32_t*>(zr + (zb & ~3) + 8);
    const uint64_t zz = ((uint64_t)__builtin_amdgcn_alignbyte(z2, z1, (uint32_t)(zb & 3)) << 32 |
                         __builtin_amdgcn_alignbyte(z1, z0, (uint32_t)(zb & 3))) >> (4 * (zq & 1));  // nibble j: group gw + j
    const uint16_t* sr = reinterpret_cast<const uint16_t*>(base + kSkCodes + c * kSkSRow) + ph + WG * w;
    const unsigned char* cr = base + c * kSkRow + WG * w * 16 + 4 * r4;
#pragma unroll
    for (int tm = 0; tm < MT; ++tm) acc.a[tm] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < WG; ++j) {
      if (gw + j >= G) break;  // wave-uniform: the last range may be partial
      const uint32_t wd = *reinterpret_cast<const uint32_t*>(cr + 16 * j);
      const half8 b = dequant_word(wd, (uint32_t)(zz >> (4 * j)) & 0xFu);
      const float sc = h2f(sr[j]);
#pragma unroll
      for (int tm = 0; tm < MT; ++tm) {
        const float4_t p = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[j][tm], b, float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        acc.a[tm] += sc * p;
      }
    }
    return acc;
  };

  // Tile t's sum over the waves (partials in part[buf]); D lane (r, c) held
  // rows 16 tm + 4r + i of output column c.
  auto store = [&](int64_t t, int buf) {
    const float4_t* pb = part + buf * kSkWaves * MT * 64;
    for (int e = tid; e < 16 * M; e += kSkThreads) {
      const int m = e >> 4, n = e & 15;
      const int tm = m >> 4, mr = m & 15;
      const float* pf = reinterpret_cast<const float*>(pb + tm * 64 + (mr >> 2) * 16 + n) + (mr & 3);
      float sum = 0.f;
#pragma unroll
      for (int ww = 0; ww < kSkWaves; ++ww) sum += pf[ww * MT * 64 * 4];
      const int64_t row = t * 16 + n;
      if (row < N) P[((int64_t)s * M + m) * N + row] = sum;
    }
  };

  // Iteration it: tile t lands (this wave's part, then every wave's at the
  // barrier, which also means every wave is done with tile t - 1), tile
  // t + D goes into t - 1's slot, the previous tile's sums are stored, and
  // tile t is multiplied into part[it & 1].
  int64_t t = t0, prev = -1;
  int it = 0;
  for (; t < ntiles; t += Bs, ++it) {
    vm_wait<kSkDma * (D - 1)>();  // this wave's part of tile t has landed
    lds_barrier();
    issue(t + D * Bs, (it + D) % R);
    if (prev >= 0) store(prev, (it - 1) & 1);
    const SkAcc<MT> acc = compute(it % R, t);
#pragma unroll
    for (int tm = 0; tm < MT; ++tm) part[((it & 1) * kSkWaves + w) * MT * 64 + tm * 64 + lane] = acc.a[tm];
    prev = t;
  }
  vm_wait<0>();
  lds_barrier();
  if (prev >= 0) store(prev, (it - 1) & 1);
}

// y = the sum of the S range partials (in range order) plus the heavy-tailed
// columns: a block of 256 threads takes 64 rows, stages their fp16 outlier
// weights (one contiguous stretch of the section, 16-byte loads issued
// together) and the M rows of heavy-tailed x in LDS, and thread (n, q) writes
// rows m = q, q + 4, ... of output column n.
constexpr int kSumRows = 64;
constexpr int kSumThreads = 256;
constexpr int kSkMaxOut = 256;  // heavy-tailed columns k_sk_sum stages (LDS)
constexpr int kSkMaxM = 16;
constexpr int kSumLoads = (kSumRows * kSkMaxOut * 2 + 16 + 16 * kSumThreads - 1) / (16 * kSumThreads);
constexpr int kSumXLoads = kSkMaxM * (kSkMaxOut / 8) / kSumThreads;

template <int MI>
__global__ __launch_bounds__(kSumThreads) void k_sk_sum(const DeviceView v, const uint16_t* __restrict__ xw, int KW,
                                                        int M, int S, const float* __restrict__ P,
                                                        uint16_t* __restrict__ y) {
  __shared__ __align__(16) unsigned char ob[kSumLoads * 16 * kSumThreads];
  __shared__ __align__(16) uint16_t xo[kSkMaxM * kSkMaxOut];
  const int tid = threadIdx.x;
  const int n_out = v.n_out, KP = 32 * v.G;
  const int XS = (n_out + 7) & ~7;  // LDS row stride of heavy-tailed x, halves
  const int64_t N = v.N;
  const int64_t n0 = (int64_t)blockIdx.x * kSumRows;
  const int rows = (int)((N - n0) < kSumRows ? (N - n0) : kSumRows);
  const int nl = tid & (kSumRows - 1), q = tid / kSumRows;
  const int64_t n = n0 + (nl < rows ? nl : 0);
  // rows m = q + 4 i of x, i < MI; rows past M compute on row 0 and are not stored
  int mrow[MI];
#pragma unroll
  for (int i = 0; i < MI; ++i) mrow[i] = q + 4 * i < M ? q + 4 * i : 0;
  // the ranges four at a time, every load of a round issued before its adds;
  // round 0 goes out before the staging below
  float pv[MI][4];
  auto load_round = [&](int k0) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int k = k0 + kk < S ? k0 + kk : k0;
        const float p = P[((int64_t)k * M + mrow[i]) * N + n];
        pv[i][kk] = k0 + kk < S ? p : 0.f;
      }
  };
  load_round(0);
  int oh = 0;  // halves from ob's start to row n0's first weight
  if (n_out > 0) {
    const uint64_t sec = 2ull * (uint64_t)N * (uint64_t)n_out;
    const __amdgpu_buffer_rsrc_t ro = rsrc(v.outliers, (sec + 15) & ~15ull);  // sections are 256-byte padded
    const uint64_t b0 = 2ull * (uint64_t)n0 * (uint64_t)n_out, e0 = b0 + 2ull * (uint64_t)rows * (uint64_t)n_out;
    const uint64_t a0 = b0 & ~15ull;
    oh = (int)((b0 - a0) >> 1);
    u32x4 t[kSumLoads];
#pragma unroll
    for (int i = 0; i < kSumLoads; ++i) {
      const uint64_t off = a0 + 16ull * (uint64_t)(tid + kSumThreads * i);
      t[i] = __builtin_amdgcn_raw_buffer_load_b128(ro, off < e0 ? (uint32_t)off : kOob, 0, 0);
    }
    const int nv = XS / 8;  // 16-byte vectors per row of heavy-tailed x
    const __amdgpu_buffer_rsrc_t rx = rsrc(xw, (uint64_t)M * KW * 2);
    u32x4 u[kSumXLoads];
#pragma unroll
    for (int i = 0; i < kSumXLoads; ++i) {
      const int e = tid + kSumThreads * i, m = e / nv, k = e - m * nv;
      u[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, m < M ? (uint32_t)((m * KW + KP) * 2 + 16 * k) : kOob, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kSumLoads; ++i) *reinterpret_cast<u32x4*>(ob + 16 * (tid + kSumThreads * i)) = t[i];
#pragma unroll
    for (int i = 0; i < kSumXLoads; ++i) {
      const int e = tid + kSumThreads * i, m = e / nv, k = e - m * nv;
      if (m < M) *reinterpret_cast<u32x4*>(xo + m * XS + 8 * k) = u[i];
    }
  }
  __syncthreads();
  if (nl >= rows) return;
  float acc[MI];
#pragma unroll
  for (int i = 0; i < MI; ++i) acc[i] = 0.f;
  for (int k0 = 0; k0 < S; k0 += 4) {
    if (k0 > 0) load_round(k0);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) acc[i] += pv[i][kk];
  }
  // heavy-tailed columns two at a time on v_dot2: the row's weights start at
  // any half (two 16-bit reads make a pair), x rows at 16-byte boundaries
  // (one 32-bit read); a last odd column pairs with a zero weight
  const uint16_t* orow = reinterpret_cast<const uint16_t*>(ob) + oh + nl * n_out;
  const int np = n_out >> 1;
  int j = 0;
  for (; j + 4 <= np; j += 4) {
    uint32_t o2[4], x2[MI][4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o2[e] = (uint32_t)orow[2 * (j + e)] | ((uint32_t)orow[2 * (j + e) + 1] << 16);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) x2[i][e] = reinterpret_cast<const uint32_t*>(xo + mrow[i] * XS)[j + e];
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int i = 0; i < MI; ++i)
        acc[i] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, o2[e]), __builtin_bit_cast(half2_t, x2[i][e]),
                                        acc[i], false);
  }
  for (; j < np; ++j) {
    const uint32_t o2 = (uint32_t)orow[2 * j] | ((uint32_t)orow[2 * j + 1] << 16);
#pragma unroll
    for (int i = 0; i < MI; ++i)
      acc[i] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, o2),
                                      __builtin_bit_cast(half2_t, reinterpret_cast<const uint32_t*>(xo + mrow[i] * XS)[j]),
                                      acc[i], false);
  }
  if (n_out & 1) {
    const uint32_t o2 = (uint32_t)orow[n_out - 1];
#pragma unroll
    for (int i = 0; i < MI; ++i)
      acc[i] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, o2),
                                      __builtin_bit_cast(half2_t, reinterpret_cast<const uint32_t*>(xo + mrow[i] * XS)[np]),
                                      acc[i], false);
  }
#pragma unroll
  for (int i = 0; i < MI; ++i)
    if (q + 4 * i < M) y[(int64_t)(q + 4 * i) * N + n] = f2h(acc[i]);
}

}  // namespace

namespace {

struct SkShape {
  int S, WG;  // K-ranges, groups per wave (a range is 16 WG groups, one per wave of 16)
};
SkShape sk_shape(const DeviceView& v) {
  const int S = (v.G + 127) / 128;
  const int per = (v.G + S - 1) / S;
  return SkShape{S, (per + 15) / 16};
}

size_t ks_lds_limit(const DeviceView& v);

template <int MT>
bool sk_fits(const DeviceView& v) {
  return sk_lds_bytes<MT>() <= ks_lds_limit(v);
}

size_t sk_x_bytes(const DeviceView& v, int64_t M) {
  const int64_t KW = 32 * (int64_t)v.G + ((v.n_out + 31) & ~31);
  return ((size_t)(M * KW * 2) + 255) & ~(size_t)255;
}

}  // namespace

// The split-K kernel: 1 <= M <= 16, at most 256 heavy-tailed columns
// (k_sk_sum stages them in LDS), code and outlier section offsets within 31
// bits.
bool mfma_splitk_supports(const DeviceView& v, int64_t M) {
  if (M < 1 || M > kSkMaxM || v.N < 1) return false;
  if (v.G < 1 || v.n_out > kSkMaxOut) return false;
  if ((uint64_t)v.N * (uint64_t)v.G * 16 >= 0x7FFFFFFFull) return false;
  if ((uint64_t)v.N * (uint64_t)v.n_out * 2 >= 0x7FFFFFF0ull) return false;
  const int64_t KW = 32 * (int64_t)v.G + ((v.n_out + 31) & ~31);
  if (M * KW * 2 >= 0x7FFFFFFF) return false;
  return sk_fits<1>(v);
}

size_t mfma_splitk_workspace_bytes(const DeviceView& v, int64_t M) {
  return sk_x_bytes(v, M) + (size_t)sk_shape(v).S * (size_t)M * (size_t)v.N * 4;
}

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
hipError_t launch_k(const DeviceView& v, const uint16_t* xw, int KW, int64_t M, uint16_t* y, hipStream_t s) {
  constexpr int CG = (NT == 1 && MT <= 2) ? 8 : 4;  // one tile per wave: wider chunks keep more bytes in flight
  constexpr size_t lds = mfma_lds_bytes<MT, CG>();
  const void* fn = reinterpret_cast<const void*>(&k_mfma<MT, NT, CG>);
  if (lds > 64 * 1024) {  // dynamic LDS past 64 KiB must be allowed per kernel
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int64_t tiles = (v.N + 15) / 16;
  const int64_t bx = (tiles + (int64_t)kMfmaCW * NT - 1) / ((int64_t)kMfmaCW * NT);
  const int64_t by = (M + 16 * MT - 1) / (16 * MT);
  hipLaunchKernelGGL((k_mfma<MT, NT, CG>), dim3((unsigned)bx, (unsigned)by), dim3(kMfmaThreads), lds, s, v, xw,
                     KW, M, y);
  return hipGetLastError();
}

// 16-row tiles per wave NT so that one block row of the grid covers N with
// about one block per compute unit.
template <int MT>
hipError_t launch_mt(const DeviceView& v, const uint16_t* xw, int KW, int64_t M, uint16_t* y, hipStream_t s) {
  constexpr int kNTMax = MT >= 8 ? 1 : (MT >= 4 ? 2 : 4);  // accumulators: NT * MT * 4 registers
  const int64_t tiles = (v.N + 15) / 16;
  const int64_t cu = v.cu_count > 0 ? v.cu_count : 1;
  const int64_t tpc = (tiles + cu - 1) / cu;
  if (tpc <= kMfmaCW || kNTMax == 1) return launch_k<MT, 1>(v, xw, KW, M, y, s);
  if (tpc <= 2 * kMfmaCW || kNTMax == 2) {
    if constexpr (kNTMax >= 2) return launch_k<MT, 2>(v, xw, KW, M, y, s);
  }
  if constexpr (kNTMax >= 4) return launch_k<MT, 4>(v, xw, KW, M, y, s);
  return hipErrorNotSupported;
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

template <int MT, int WG>
hipError_t launch_sk_wg(const DeviceView& v, const uint16_t* xw, int KW, int64_t M, float* P, hipStream_t s,
                        int S) {
  constexpr size_t lds = sk_lds_bytes<MT>();
  const void* fn = reinterpret_cast<const void*>(&k_mfma_sk<MT, WG>);
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int64_t cu = v.cu_count > 0 ? v.cu_count : 1;
  const int64_t tiles = (v.N + 15) / 16;
  int64_t bs = cu / S;  // blocks per K-range: one block per compute unit in all
  if (bs < 1) bs = 1;
  if (bs > tiles) bs = tiles;
  hipLaunchKernelGGL((k_mfma_sk<MT, WG>), dim3((unsigned)(bs * S)), dim3(kSkThreads), lds, s, v, xw, KW, (int)M, S, P);
  return hipGetLastError();
}

template <int MT>
hipError_t launch_sk_mt(const DeviceView& v, const uint16_t* xw, int KW, int64_t M, float* P, hipStream_t s) {
  const SkShape sh = sk_shape(v);
  switch (sh.WG) {
    case 1: return launch_sk_wg<MT, 1>(v, xw, KW, M, P, s, sh.S);
    case 2: return launch_sk_wg<MT, 2>(v, xw, KW, M, P, s, sh.S);
    case 3: return launch_sk_wg<MT, 3>(v, xw, KW, M, P, s, sh.S);
    case 4: return launch_sk_wg<MT, 4>(v, xw, KW, M, P, s, sh.S);
    case 5: return launch_sk_wg<MT, 5>(v, xw, KW, M, P, s, sh.S);
    case 6: return launch_sk_wg<MT, 6>(v, xw, KW, M, P, s, sh.S);
    case 7: return launch_sk_wg<MT, 7>(v, xw, KW, M, P, s, sh.S);
    case 8: return launch_sk_wg<MT, 8>(v, xw, KW, M, P, s, sh.S);
    default: return hipErrorNotSupported;
  }
}

hipError_t launch_sk(const DeviceView& v, const uint16_t* xw, int KW, int64_t M, uint16_t* y, void* workspace,
                     hipStream_t s) {
  float* P = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + sk_x_bytes(v, M));
  const hipError_t e = launch_sk_mt<1>(v, xw, KW, M, P, s);
  if (e != hipSuccess) return e;
  const unsigned blocks = (unsigned)((v.N + kSumRows - 1) / kSumRows);
  const int S = sk_shape(v).S;
  if (M <= 4)
    hipLaunchKernelGGL(k_sk_sum<1>, dim3(blocks), dim3(kSumThreads), 0, s, v, xw, KW, (int)M, S, P, y);
  else if (M <= 8)
    hipLaunchKernelGGL(k_sk_sum<2>, dim3(blocks), dim3(kSumThreads), 0, s, v, xw, KW, (int)M, S, P, y);
  else
    hipLaunchKernelGGL(k_sk_sum<4>, dim3(blocks), dim3(kSumThreads), 0, s, v, xw, KW, (int)M, S, P, y);
  return hipGetLastError();
}

}  // namespace

bool mfma_tiled_supports(const DeviceView& v, int64_t M) {
  return ks_supports(v, 32 * v.G + ((v.n_out + 31) & ~31), M);
}

hipError_t launch_mfma_ws(const DeviceView& v, const uint16_t* x, uint16_t* y, int64_t M,
                          void* workspace, hipStream_t s, int plan) {
  const int KW = 32 * v.G + ((v.n_out + 31) & ~31);
  uint16_t* xw = static_cast<uint16_t*>(workspace);
  const unsigned gy = (unsigned)(M < 65535 ? M : 65535);
  hipLaunchKernelGGL(k_xbulk, dim3((unsigned)((KW + kThreads - 1) / kThreads), gy),
                     dim3(kThreads), 0, s, v, x, M, xw, KW);
  if (plan == SPECTRA_PLAN_MFMA_SPLITK) return launch_sk(v, xw, KW, M, y, workspace, s);
  if (plan == SPECTRA_PLAN_MFMA_TILED) return launch_ks(v, xw, KW, M, y, s);
  if (M <= 16) return launch_mt<1>(v, xw, KW, M, y, s);
  if (M <= 32) return launch_mt<2>(v, xw, KW, M, y, s);
  if (M <= 64) return launch_mt<4>(v, xw, KW, M, y, s);
  return launch_mt<8>(v, xw, KW, M, y, s);
}

}  // namespace spectra
