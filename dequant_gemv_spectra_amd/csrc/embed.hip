// SPECTRA fused embedding gather for gfx950: out[i][:] = W_hat[ids[i]][:], fp16.
//
// The SPECTRA page (abstract; highlight 5 on the fused embedding) keeps a
// vocabulary table in the same Group-32 4-bit format as the linear layers and
// dequantizes only the rows a forward pass gathers.  Here the table is a
// container with N = vocabulary rows and K = embedding channels; a gathered
// row is that row of W_hat in channel order: bulk entries (q - z) * s16,
// heavy-tailed channels their stored fp16 bits.
//
// Mapping.  One wave per token; a wave walks tokens w, w + W, ... with the
// next token's row loads in flight while the current one is written.  Lane l dequantizes the groups g = l + 64p of
// the token's row: (w & 0x000F000F) | 0x6400_6400 holds 1024 + q of two
// members and (w & 0x00F000F0) | 0x5400_5400 holds 64 + q of the next two;
// subtracting 1024 + z or 64 + z leaves q - z exactly, and one packed fp16
// multiply by s16 rounds the exact product (q - z) * s16 once, to nearest
// even.  The 32 values go to the wave's row buffer in LDS in bulk order (80-
// byte group slots, as the GEMV stages x), the heavy-tailed values after the
// slots.  The wave then writes the row in channel order: lane l takes channels
// 8c .. 8c + 7 for c = l + 64j, looks up where each channel sits in the row
// buffer through an inverse permutation the block builds once in LDS, and
// stores the 8 halves with one non-temporal 16-byte store (12 % faster than
// plain stores: 100 MB of rows per 16384 ids go out once).  Ids outside [0, N) read zeros
// through the buffer-descriptor range checks and produce zero rows.
#include "spectra_internal.h"

namespace spectra {
namespace {

constexpr int kWaveSlot = 40;      // halves per group slot in a row buffer (32 used)
constexpr int kMaxWaves = 8;       // waves per block
constexpr int kRsrcWord3 = 0x00020000;
constexpr uint32_t kOob = 0x80000000u;
constexpr int kStream = 2;         // non-temporal: table rows are read once

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint64_t bytes) {
  const int n = bytes >= 0x7FFFFFFFull ? 0x7FFFFFFF : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kRsrcWord3);
}
__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t as_u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

// The 8 members of code word w (members 8d .. 8d + 7 of the record) as fp16
// (q - z) * s, in member order, packed two per dword.
__device__ __forceinline__ u32x4 dequant_word(uint32_t w, uint32_t z, half2_t s2) {
  const half2_t zl = as_h2((0x6400u + z) * 0x00010001u);         // 1024 + z
  const half2_t zh = as_h2((0x5400u + (z << 4)) * 0x00010001u);  // 64 + z
  const uint32_t w8 = w >> 8;
  const half2_t p0 = (as_h2((w & 0x000F000Fu) | 0x64006400u) - zl) * s2;   // members 0, 1
  const half2_t p1 = (as_h2((w & 0x00F000F0u) | 0x54005400u) - zh) * s2;   // members 2, 3
  const half2_t p2 = (as_h2((w8 & 0x000F000Fu) | 0x64006400u) - zl) * s2;  // members 4, 5
  const half2_t p3 = (as_h2((w8 & 0x00F000F0u) | 0x54005400u) - zh) * s2;  // members 6, 7
  return u32x4{as_u32(p0), as_u32(p1), as_u32(p2), as_u32(p3)};
}

// One token's row in registers: P records per lane (groups lane + 64p) with
// their scale bits and zero bytes, and OE heavy-tailed values per lane.
constexpr int OE = 4;  // heavy-tailed channels held in registers: 64 * OE
template <int P>
struct RowFrag {
  u32x4 c[P];
  uint32_t s[P], z[P];
  uint32_t o[OE];
};

template <int P>
__device__ __forceinline__ void load_row(RowFrag<P>& f, const DeviceView& v, int32_t t, int lane) {
  const int G = v.G, n_out = v.n_out;
  const bool ok = t >= 0 && (int64_t)t < v.N;
  const int64_t row = ok ? t : 0;
  const int64_t i0 = row * G;  // flat index of the row's first group
  const __amdgpu_buffer_rsrc_t rc = rsrc(v.codes + i0, ok ? (uint64_t)G * 16 : 0);
  const __amdgpu_buffer_rsrc_t rs = rsrc(v.scales + i0, ok ? (uint64_t)G * 2 : 0);
  const int64_t zb0 = i0 >> 1;
  const __amdgpu_buffer_rsrc_t rz = rsrc(v.zeros + zb0, ok ? (uint64_t)(((i0 + G + 1) >> 1) - zb0) : 0);
  const __amdgpu_buffer_rsrc_t ro = rsrc(v.outliers + row * n_out, ok ? (uint64_t)n_out * 2 : 0);
  const uint32_t i0odd = (uint32_t)(i0 & 1);
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int g = lane + 64 * p;
    const bool in = g < G;
    f.c[p] = __builtin_amdgcn_raw_buffer_load_b128(rc, in ? (uint32_t)g * 16u : kOob, 0, kStream);
    f.s[p] = __builtin_amdgcn_raw_buffer_load_b16(rs, in ? (uint32_t)g * 2u : kOob, 0, 0);
    f.z[p] = __builtin_amdgcn_raw_buffer_load_b8(rz, in ? ((uint32_t)g + i0odd) >> 1 : kOob, 0, 0);
  }
#pragma unroll
  for (int k = 0; k < OE; ++k) {
    const int j = lane + 64 * k;
    f.o[k] = __builtin_amdgcn_raw_buffer_load_b16(ro, j < n_out ? (uint32_t)j * 2u : kOob, 0, 0);
  }
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Dequantize row t (already in f) into the row buffer and write it out as
// output row i in channel order.
template <int P>
__device__ __forceinline__ void emit_row(const RowFrag<P>& f, const DeviceView& v, int32_t t,
                                         int64_t i, const uint16_t* inv, uint16_t* rb,
                                         uint16_t* __restrict__ out, int aligned, int lane) {
  const int K = v.K, G = v.G, n_out = v.n_out;
  const bool ok = t >= 0 && (int64_t)t < v.N;
  const uint32_t i0odd = ok ? (uint32_t)(((int64_t)t * G) & 1) : 0u;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int g = lane + 64 * p;
    if (g < G) {
      const uint32_t z = (f.z[p] >> (4u * (((uint32_t)g + i0odd) & 1u))) & 0xFu;
      const half2_t s2 = as_h2(f.s[p] * 0x00010001u);
      u32x4* dst = reinterpret_cast<u32x4*>(rb + g * kWaveSlot);
      dst[0] = dequant_word(f.c[p].x, z, s2);
      dst[1] = dequant_word(f.c[p].y, z, s2);
      dst[2] = dequant_word(f.c[p].z, z, s2);
      dst[3] = dequant_word(f.c[p].w, z, s2);
    }
  }
#pragma unroll
  for (int k = 0; k < OE; ++k) {
    const int j = lane + 64 * k;
    if (j < n_out) rb[kWaveSlot * G + j] = (uint16_t)f.o[k];
  }
  if (n_out > 64 * OE && ok) {  // heavy-tailed channels beyond the register slots
    const uint16_t* orow = v.outliers + (int64_t)t * n_out;
    for (int j = lane + 64 * OE; j < n_out; j += 64) rb[kWaveSlot * G + j] = orow[j];
  } else if (n_out > 64 * OE) {
    for (int j = lane + 64 * OE; j < n_out; j += 64) rb[kWaveSlot * G + j] = 0;
  }
  wave_sync();  // the row buffer is this wave's alone: its writes before its reads
  uint16_t* orow = out + i * (int64_t)K;
  const int nch = (K + 7) >> 3;
  for (int c = lane; c < nch; c += 64) {
    const uint4 ix = *reinterpret_cast<const uint4*>(inv + 8 * c);
    const uint32_t h0 = rb[ix.x & 0xFFFFu], h1 = rb[ix.x >> 16];
    const uint32_t h2 = rb[ix.y & 0xFFFFu], h3 = rb[ix.y >> 16];
    const uint32_t h4 = rb[ix.z & 0xFFFFu], h5 = rb[ix.z >> 16];
    const uint32_t h6 = rb[ix.w & 0xFFFFu], h7 = rb[ix.w >> 16];
    if (aligned) {
      // streamed out: the rows are not read again by this kernel
      __builtin_nontemporal_store(u32x4{h0 | (h1 << 16), h2 | (h3 << 16), h4 | (h5 << 16), h6 | (h7 << 16)},
                                  reinterpret_cast<u32x4*>(orow + 8 * c));
    } else {
      const uint32_t h[8] = {h0, h1, h2, h3, h4, h5, h6, h7};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (8 * c + e < K) orow[8 * c + e] = (uint16_t)h[e];
    }
  }
  wave_sync();  // the next row overwrites the buffer only after every lane read it
}

// LDS: inv[ceil(K/8)*8] (row-buffer index of each channel; padding channels
// point at a zero), then one row buffer per wave of `rowh` halves.  A wave
// walks its tokens with two register buffers: the next token's row is in
// flight while the current one is dequantized and written.
template <int P>
__global__ __launch_bounds__(64 * kMaxWaves) void k_embed(const DeviceView v,
                                                          const int32_t* __restrict__ ids,
                                                          int64_t T, uint16_t* __restrict__ out,
                                                          int rowh, int aligned) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int K = v.K, K_b = v.K_b, G = v.G, n_out = v.n_out;
  const int nch = (K + 7) >> 3;  // 8-channel chunks of a row
  uint16_t* inv = reinterpret_cast<uint16_t*>(smem);
  const int waves = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint16_t* rb = inv + 8 * nch + wave * rowh;
  const int zero_slot = kWaveSlot * G + n_out;  // stays zero in every row buffer

  for (int j = threadIdx.x; j < 8 * nch; j += blockDim.x) {
    if (j < K) {
      const int k = v.perm[j];
      inv[k] = (uint16_t)(j < K_b ? (j >> 5) * kWaveSlot + (j & 31) : kWaveSlot * G + (j - K_b));
    }
    if (j >= K) inv[j] = (uint16_t)zero_slot;
  }
  if (lane == 0) rb[zero_slot] = 0;
  __syncthreads();

  const int64_t step = (int64_t)gridDim.x * waves;
  int64_t i = (int64_t)blockIdx.x * waves + wave;
  if (i >= T) return;
  // ids run two tokens ahead of the rows, rows one token ahead of the
  // dequantization; an id of -1 (past T) loads nothing
  RowFrag<P> fa, fb;
  int32_t t0 = ids[i];
  int32_t t1 = i + step < T ? ids[i + step] : -1;
  load_row<P>(fa, v, t0, lane);
  for (;;) {
    load_row<P>(fb, v, t1, lane);  // token i + step
    const int32_t t2 = i + 2 * step < T ? ids[i + 2 * step] : -1;
    __builtin_amdgcn_sched_barrier(0);
    emit_row<P>(fa, v, t0, i, inv, rb, out, aligned, lane);
    if (i + step >= T) break;
    i += step;
    load_row<P>(fa, v, t2, lane);  // token i + step
    const int32_t t3 = i + 2 * step < T ? ids[i + 2 * step] : -1;
    __builtin_amdgcn_sched_barrier(0);
    emit_row<P>(fb, v, t1, i, inv, rb, out, aligned, lane);
    if (i + step >= T) break;
    i += step;
    t0 = t2;
    t1 = t3;
  }
}

size_t row_halves(const DeviceView& v) {
  return (((size_t)kWaveSlot * v.G + (size_t)v.n_out + 1) + 7) & ~(size_t)7;
}

size_t lds_cap(const DeviceView& v) {
  const size_t dev = v.lds_per_block > 0 ? (size_t)v.lds_per_block : 64 * 1024;
  return dev < (size_t)160 * 1024 ? dev : (size_t)160 * 1024;
}

// Waves per block the LDS allows (0: none fits).
int embed_waves(const DeviceView& v) {
  const size_t inv_bytes = 16 * (((size_t)v.K + 7) / 8);
  const size_t row_bytes = 2 * row_halves(v);
  const size_t cap = lds_cap(v);
  if (inv_bytes + row_bytes > cap) return 0;
  const size_t w = (cap - inv_bytes) / row_bytes;
  return (int)(w < (size_t)kMaxWaves ? w : (size_t)kMaxWaves);
}

}  // namespace

bool embed_supports(const DeviceView& v) {
  // row-buffer indices are 16-bit; at most 8 records per lane (G <= 512)
  if (row_halves(v) > 65535 || v.G > 512) return false;
  return embed_waves(v) > 0;
}

hipError_t launch_embed(const DeviceView& v, const int32_t* ids, int64_t T, uint16_t* out,
                        hipStream_t s) {
  if (!embed_supports(v)) return hipErrorNotSupported;
  if (T == 0) return hipSuccess;
  const int waves = embed_waves(v);
  const size_t lds = 16 * (((size_t)v.K + 7) / 8) + 2 * row_halves(v) * (size_t)waves;
  const int aligned = (v.K % 8 == 0) && ((reinterpret_cast<uintptr_t>(out) & 15) == 0);
  const int64_t per_cu = (int64_t)v.cu_count * 2;
  int64_t blocks = (T + waves - 1) / waves;
  if (blocks > per_cu) blocks = per_cu;
  const int P = (v.G + 63) / 64;
  const void* fns[8] = {reinterpret_cast<const void*>(&k_embed<1>), reinterpret_cast<const void*>(&k_embed<2>),
                        reinterpret_cast<const void*>(&k_embed<3>), reinterpret_cast<const void*>(&k_embed<4>),
                        reinterpret_cast<const void*>(&k_embed<5>), reinterpret_cast<const void*>(&k_embed<6>),
                        reinterpret_cast<const void*>(&k_embed<7>), reinterpret_cast<const void*>(&k_embed<8>)};
  const int pi = P < 1 ? 0 : P - 1;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(fns[pi], hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)blocks), block(64 * waves);
  const int rowh = (int)row_halves(v);
  switch (pi) {
    case 0: hipLaunchKernelGGL(k_embed<1>, grid, block, lds, s, v, ids, T, out, rowh, aligned); break;
    case 1: hipLaunchKernelGGL(k_embed<2>, grid, block, lds, s, v, ids, T, out, rowh, aligned); break;
    case 2: hipLaunchKernelGGL(k_embed<3>, grid, block, lds, s, v, ids, T, out, rowh, aligned); break;
    case 3: hipLaunchKernelGGL(k_embed<4>, grid, block, lds, s, v, ids, T, out, rowh, aligned); break;
    case 4: hipLaunchKernelGGL(k_embed<5>, grid, block, lds, s, v, ids, T, out, rowh, aligned); break;
    case 5: hipLaunchKernelGGL(k_embed<6>, grid, block, lds, s, v, ids, T, out, rowh, aligned); break;
    case 6: hipLaunchKernelGGL(k_embed<7>, grid, block, lds, s, v, ids, T, out, rowh, aligned); break;
    default: hipLaunchKernelGGL(k_embed<8>, grid, block, lds, s, v, ids, T, out, rowh, aligned); break;
  }
  return hipGetLastError();
}

}  // namespace spectra
