// Device helpers of the M = 1 dequant-GEMV, shared by the single-product
// kernel (gemv.hip) and the persistent decode-step kernel (step.hip): buffer
// descriptors, the fp16 magic dequantization of one 16-byte code record fused
// into v_dot2_f32_f16 dot products, and the cross-lane team reduction.
//
// Arithmetic (SPECTRA page, abstract: Group-32 4-bit codes with an fp16 scale
// per group and 4-bit zero points).  For a code word w, (w & 0x000F000F) |
// 0x6400_6400 holds the fp16 values 1024 + q of members (8d, 8d+1);
// (w & 0x00F000F0) | 0x5400_5400 holds 64 + q of members (8d+2, 8d+3); the
// same two masks on w >> 8 give members (8d+4, 8d+5) and (8d+6, 8d+7).
// Subtracting the fp16 pairs 1024 + z and 64 + z leaves q - z exactly, and
// v_dot2_f32_f16 multiplies them by the matching x pairs in fp32.
#pragma once

#include "spectra_internal.h"

namespace spectra {
namespace g32k {

constexpr int kXSlot = 40;  // halves per group slot of x in LDS (32 used, 80 bytes)
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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

// Buffer descriptors (gfx9 raw buffer, stride 0): the hardware range check
// returns 0 for any byte offset at or past num_records, so loads need no
// branches.
constexpr int kRsrcWord3 = 0x00020000;
constexpr uint32_t kOob = 0x80000000u;  // an offset past every descriptor built here
constexpr int kStream = 2;  // cache-policy bit nt: streamed data, read once
constexpr int kAgentScope = 16;  // cache-policy bit sc1: coherent at agent (device) scope

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint64_t bytes) {
  const int n = bytes >= 0x7FFFFFFFull ? 0x7FFFFFFF : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kRsrcWord3);
}

// Nibble masks and fp16 magics of a code word.  The masks sit in scalar
// registers and the magics in vector registers, each written once by an
// opaque move, so that each (w & mask) | magic compiles to one v_and_or_b32:
// a gfx9 VOP3 encoding takes no literal, and with immediates the compiler
// emits a separate AND and OR.
struct Nib {
  uint32_t lo, hi;    // 0x000F000F and 0x00F000F0
  uint32_t mlo, mhi;  // 0x64006400 (1024) and 0x54005400 (64)
};

__device__ __forceinline__ Nib make_nib() {
  uint32_t nlo, nhi, mlo, mhi;
  asm volatile("s_mov_b32 %0, 0x000F000F" : "=s"(nlo));
  asm volatile("s_mov_b32 %0, 0x00F000F0" : "=s"(nhi));
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(mlo));
  asm volatile("v_mov_b32 %0, 0x54005400" : "=v"(mhi));
  return Nib{nlo, nhi, mlo, mhi};
}

// The 32 halves of one x group slot, as 16 pairs.
__device__ __forceinline__ void read_x(const uint16_t* src16, half2_t* xr) {
  const uint4* src = reinterpret_cast<const uint4*>(src16);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 t = src[q];
    xr[4 * q + 0] = as_h2(t.x);
    xr[4 * q + 1] = as_h2(t.y);
    xr[4 * q + 2] = as_h2(t.z);
    xr[4 * q + 3] = as_h2(t.w);
  }
}

// sum_e (q_e - z) * x_e over one record with the dequantization fused into the
// dot products: one chain of 16 v_dot2 per record (the lane's other records
// interleave with it; four chains cost four zeroing moves and three adds per
// record, 1 - 4 % slower on every M = 1 shape measured).
__device__ __forceinline__ float group_dot(const uint4 c, const uint32_t z, const half2_t* xr,
                                           const Nib nb) {
  const half2_t zl = as_h2((0x6400u + z) * 0x00010001u);
  const half2_t zh = as_h2((0x5400u + (z << 4)) * 0x00010001u);
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  float a = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t w8 = w[d] >> 8;
    a = __builtin_amdgcn_fdot2(as_h2((w[d] & nb.lo) | nb.mlo) - zl, xr[4 * d + 0], a, false);
    a = __builtin_amdgcn_fdot2(as_h2((w[d] & nb.hi) | nb.mhi) - zh, xr[4 * d + 1], a, false);
    a = __builtin_amdgcn_fdot2(as_h2((w8 & nb.lo) | nb.mlo) - zl, xr[4 * d + 2], a, false);
    a = __builtin_amdgcn_fdot2(as_h2((w8 & nb.hi) | nb.mhi) - zh, xr[4 * d + 3], a, false);
  }
  return a;
}

// Position of bulk channel j in the LDS group slots.
__device__ __forceinline__ int xs_index(int j) { return (j >> 5) * kXSlot + (j & 31); }

}  // namespace g32k
}  // namespace spectra
