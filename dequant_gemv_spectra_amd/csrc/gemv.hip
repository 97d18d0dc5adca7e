// SPECTRA dequant-GEMV for gfx950 at M = 1 (decode): y = x W_hat^T.
//
// The SPECTRA page (abstract; highlight 4 on its fused kernels) describes
// dequantization fused into the product so that only the packed weights cross
// DRAM; the decode product is bound by weight bytes (the techfi24 summary,
// section on the hardware context: every token re-reads all weights).  This
// kernel is a gfx950 design of that idea, not a port: the page's kernels
// target a laptop Ampere GPU.
//
// Mapping.  A team of L lanes (L = 16, 32 or 64) owns one output row at a
// time; lane t of a team owns the groups g = t + L*p (p < P) of every row it
// visits, so a team's load for slot p covers 16*L contiguous bytes of codes
// (buffer_load_dwordx4 per lane).  A tile is T*U rows (T teams per block, U
// rows per team); a block walks the tiles b, b + B, b + 2B, ... of its
// container, so at any moment all blocks stream one moving window of HBM.
// Two register buffers hold consecutive tiles: the next tile's loads are in
// flight while the current one is computed.  Loads go through buffer
// descriptors rebased on each tile, so rows past N and idle lanes read zeros
// from the hardware range check with no branches.  One launch may carry up to
// eight containers that share x (q/k/v or gate/up of a decoder layer).
//
// Staging.  Each block copies x into LDS and gathers it into bulk order
// through perm: x and perm are fetched with 16-byte loads in one round trip,
// and the block's first tile of weights is requested right behind them, so
// the gather and its barriers run while that tile is on its way from HBM (a
// wave's loads complete in issue order: had the tile gone first, the gather
// would have waited for it).  In LDS each group's 32 halves occupy an 80-byte
// slot, which keeps the per-lane 16-byte reads free of bank conflicts.  Blocks
// of 512 lanes, one per compute unit (one staging copy per CU), or two on
// long launches when registers and LDS allow (one wave's dequantization then
// overlaps another's loads).
//
// Code records are read with the non-temporal hint: each is used once, and
// the hint keeps them from displacing x, perm and the metadata in the caches.
//
// Arithmetic: exact fp16 pairs q - z from the code words (gemv_common.h),
// v_dot2_f32_f16 products accumulated in fp32, each group sum scaled by s16
// in fp32; the heavy-tailed columns are a dense fp16 side product in the same
// pass; team partials are reduced with DPP inside 16-lane rows and lane
// swizzles across rows.
#include "gemv_common.h"

#ifndef SPECTRA_GEMV_BLOCKS_PER_CU
#define SPECTRA_GEMV_BLOCKS_PER_CU 1
#endif
#ifndef SPECTRA_GEMV_TWO_BLOCK_TILES
#define SPECTRA_GEMV_TWO_BLOCK_TILES 6
#endif
#ifndef SPECTRA_GEMV_U
#define SPECTRA_GEMV_U 1
#endif

namespace spectra {
namespace {

using namespace g32k;

#ifndef SPECTRA_GEMV_BLOCK
#define SPECTRA_GEMV_BLOCK 512
#endif
constexpr int kBlock = SPECTRA_GEMV_BLOCK;
constexpr int kMaxTasks = 8;

struct GemvTask {
  DeviceView v;
  const uint16_t* x;
  uint16_t* y;
  int32_t nblocks;         // blocks serving this task
  int32_t rows_per_block;  // contiguous rows per block (short launches), else 0
};

// Kernel arguments.  Task 0 (its container base, x, y, N, K, n_out and row
// split), the rows of x and the first blocks of tasks 1 .. 3 come as 14
// leading scalar arguments, which the build preloads into scalar registers
// (kernarg preloading, -amdgpu-kernarg-preload-count=14).  A block of task 0
// (every block of a one-container launch) computes its section addresses from
// the base and the shape and touches no argument memory; a block of tasks
// 1 .. 3 reads its task's fields below in one batch of scalar loads, a single
// round trip before its first vector load; tasks 4 .. 7 read `begin` first.
struct GemvTasks {
  int32_t begin[kMaxTasks];  // first block of each task; INT32_MAX past the last task
  int32_t count;
  GemvTask t[kMaxTasks];
};

// The 32 members of one 16-byte code record as exact fp16 pairs q - z.  Bits
// 0-3 of each half under exponent 2^10 read as 1024 + q; bits 4-7 under
// exponent 2^6 read as 64 + q.  Pair j holds members (2j, 2j + 1), the order
// of x in the group slot.
__device__ __forceinline__ void dequant_record(const uint4 c, const uint32_t z, const Nib nb,
                                               half2_t* wq) {
  const half2_t zl = as_h2((0x6400u + z) * 0x00010001u);         // 1024 + z
  const half2_t zh = as_h2((0x5400u + (z << 4)) * 0x00010001u);  // 64 + z
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t w8 = w[d] >> 8;
    wq[4 * d + 0] = as_h2((w[d] & nb.lo) | nb.mlo) - zl;
    wq[4 * d + 1] = as_h2((w[d] & nb.hi) | nb.mhi) - zh;
    wq[4 * d + 2] = as_h2((w8 & nb.lo) | nb.mlo) - zl;
    wq[4 * d + 3] = as_h2((w8 & nb.hi) | nb.mhi) - zh;
  }
}

// sum over the 16 pairs of wq * xr in fp32; four accumulators keep the dot2
// chains short.
__device__ __forceinline__ float dot_record(const half2_t* wq, const half2_t* xr) {
  float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    a0 = __builtin_amdgcn_fdot2(wq[4 * d + 0], xr[4 * d + 0], a0, false);
    b0 = __builtin_amdgcn_fdot2(wq[4 * d + 1], xr[4 * d + 1], b0, false);
    a1 = __builtin_amdgcn_fdot2(wq[4 * d + 2], xr[4 * d + 2], a1, false);
    b1 = __builtin_amdgcn_fdot2(wq[4 * d + 3], xr[4 * d + 3], b1, false);
  }
  return (a0 + a1) + (b0 + b1);
}

// Gather x into LDS: bulk positions [0, K_b) in their 80-byte group slots,
// zeros up to 32G, then the heavy-tailed values (fp16) right after the slots.
//   A. One round trip: each thread issues 16-byte loads of x (8 channels) and
//      of perm (4 bulk positions), plus the perm entry of one heavy-tailed
//      channel.
//   B. x is written to LDS as is (`xraw`, channel order); barrier.
//   C. Each thread reads its 4 positions' values from xraw through the perm
//      entries and stores them as one 8-byte write into the group slot.
// For a batch tile of MX rows of x, B and C run once per row (row m's slots
// at xs + m * xstride), reusing xraw.  `between` runs after the loads of A
// are issued and before B waits for them: the caller issues its first weight
// loads there.  Positions past K_b, and
// channels past K, read zero through the range check of the buffer
// descriptors.
constexpr int kQuads = 8;    // perm quads per thread: 8 * 4 * kBlock = 16384 positions
constexpr int kXChunks = 4;  // 8-channel x chunks per thread: 4 * 8 * kBlock = 16384 channels
template <int MX, class F>
__device__ __forceinline__ void stage_x(const DeviceView& v, const uint16_t* __restrict__ x, int M,
                                        uint16_t* xs, int xstride, uint16_t* xraw, int tid,
                                        F&& between) {
  const int K = v.K, K_b = v.K_b, n_out = v.n_out;
  const int xo_base = kXSlot * v.G;  // heavy-tailed x (fp16) follow the group slots
  const int nquad = 8 * v.G;         // 32G / 4
  const int nchunk = (K + 7) >> 3;
  const __amdgpu_buffer_rsrc_t rp = rsrc(v.perm, (uint64_t)K * 4);
  // A. loads (rows m >= M of a batch tile read zeros)
  const uint32_t oidx = __builtin_amdgcn_raw_buffer_load_b32(
      rp, tid < n_out ? (uint32_t)(K_b + tid) * 4u : kOob, 0, 0);
  u32x4 xv[MX][kXChunks];
#pragma unroll
  for (int m = 0; m < MX; ++m) {
    // whole chunks only; row m starts 16-byte aligned (K % 8 == 0 whenever MX > 1)
    const __amdgpu_buffer_rsrc_t rx = rsrc(x + (int64_t)m * K, m < M ? (uint64_t)(K >> 3) * 16 : 0);
#pragma unroll
    for (int i = 0; i < kXChunks; ++i) {
      if (kBlock * i >= nchunk) break;  // block-uniform bound
      xv[m][i] = __builtin_amdgcn_raw_buffer_load_b128(rx, (uint32_t)(tid + kBlock * i) * 16u, 0, 0);
    }
  }
  u32x4 pq[kQuads];
#pragma unroll
  for (int i = 0; i < kQuads; ++i) {
    if (kBlock * i >= nquad) break;
    pq[i] = __builtin_amdgcn_raw_buffer_load_b128(rp, (uint32_t)(tid + kBlock * i) * 16u, 0, 0);
  }
  between();
#pragma unroll
  for (int m = 0; m < MX; ++m) {
    if (m) __syncthreads();  // every thread is done gathering row m - 1 from xraw
    // B. raw x into LDS (a partial last chunk is read channel by channel)
#pragma unroll
    for (int i = 0; i < kXChunks; ++i) {
      if (kBlock * i >= nchunk) break;
      const int c = tid + kBlock * i;
      if (c < nchunk) {
        u32x4 t = xv[m][i];
        if (8 * c + 8 > K) {
          uint32_t h[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) h[e] = (m < M && 8 * c + e < K) ? x[(int64_t)m * K + 8 * c + e] : 0u;
          t = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
        }
        *reinterpret_cast<u32x4*>(xraw + 8 * c) = t;
      }
    }
    __syncthreads();
    // C. gather from xraw into row m's group slots
    uint16_t* xm = xs + m * xstride;
#pragma unroll
    for (int i = 0; i < kQuads; ++i) {
      if (kBlock * i >= nquad) break;
      const int c = tid + kBlock * i;
      const int j = 4 * c;
      const uint32_t a0 = j + 0 < K_b ? xraw[pq[i].x] : 0u;
      const uint32_t a1 = j + 1 < K_b ? xraw[pq[i].y] : 0u;
      const uint32_t a2 = j + 2 < K_b ? xraw[pq[i].z] : 0u;
      const uint32_t a3 = j + 3 < K_b ? xraw[pq[i].w] : 0u;
      if (c < nquad)
        *reinterpret_cast<uint2*>(xm + xs_index(j)) = make_uint2(a0 | (a1 << 16), a2 | (a3 << 16));
    }
    if (tid < n_out) xm[xo_base + tid] = xraw[oidx];
    for (int j = tid + kBlock; j < n_out; j += kBlock) xm[xo_base + j] = xraw[v.perm[K_b + j]];
    // No bulk group (every channel heavy-tailed): the lanes' one slot reads
    // the first 32 halves, which then hold the heavy-tailed x and zeros,
    // never stale LDS (times the zero codes they add exactly 0).
    if (v.G == 0)
      for (int j = n_out + tid; j < 32; j += kBlock) xm[j] = 0;
  }
}

// Registers holding one tile of weights for a lane: U rows x P groups of
// codes, scale bits and zero bytes, and OS heavy-tailed weights per row.
// Scale and zero stay in separate registers until the tile is computed:
// combining them at load time would make the compiler wait for those loads
// before it issues the next tile's, which leaves one tile in flight.
template <int P, int U, int OS>
struct Frag {
  uint4 c[U][P];
  uint32_t s[U][P], z[U][P];
  uint32_t o[U][OS];
};

// Loads the tile whose first row is row0 (rows >= row_end read as zero).  The
// descriptors are rebased on the tile so offsets stay small for any size.
template <int L, int P, int U, int OS>
__device__ __forceinline__ void load_frag(Frag<P, U, OS>& f, const DeviceView& v, int64_t row0,
                                          int64_t row_end, int lt, int team) {
  constexpr int T = kBlock / L;
  const int G = v.G, n_out = v.n_out;
  const int64_t left = row_end - row0;
  const int64_t rows = left < (int64_t)T * U ? (left > 0 ? left : 0) : (int64_t)T * U;
  const int64_t i0 = row0 * G;  // flat group index of the tile's first group
  const __amdgpu_buffer_rsrc_t rc = rsrc(v.codes + i0, (uint64_t)rows * G * 16);
  const __amdgpu_buffer_rsrc_t rs = rsrc(v.scales + i0, (uint64_t)rows * G * 2);
  const int64_t zb0 = i0 >> 1;
  const uint32_t i0odd = (uint32_t)(i0 & 1);
  const __amdgpu_buffer_rsrc_t rz = rsrc(v.zeros + zb0, (uint64_t)(((i0 + rows * G + 1) >> 1) - zb0));
  const __amdgpu_buffer_rsrc_t ro = rsrc(v.outliers + row0 * n_out, (uint64_t)rows * n_out * 2);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int row = team + u * T;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int g = lt + L * p;
      const uint32_t local = (uint32_t)(row * G + g);
      const bool ok = g < G;
      const u32x4 c = __builtin_amdgcn_raw_buffer_load_b128(rc, ok ? local * 16u : kOob, 0, kStream);
      f.c[u][p] = make_uint4(c.x, c.y, c.z, c.w);
      f.s[u][p] = __builtin_amdgcn_raw_buffer_load_b16(rs, ok ? local * 2u : kOob, 0, 0);
      const uint32_t zoff = (local + i0odd) >> 1;  // byte of group i0 + local, from byte zb0
      f.z[u][p] = __builtin_amdgcn_raw_buffer_load_b8(rz, ok ? zoff : kOob, 0, 0);
    }
#pragma unroll
    for (int s = 0; s < OS; ++s) {
      const int j = lt + L * s;
      const uint32_t off = (uint32_t)(row * n_out + j) * 2u;
      f.o[u][s] = __builtin_amdgcn_raw_buffer_load_b16(ro, j < n_out ? off : kOob, 0, 0);
    }
  }
}

// y rows m < M of the tile: MX rows of x share each dequantized record.
// XR: one row of x, held in registers for this lane's groups (xreg) instead
// of read from LDS per tile.
template <int L, int P, int U, int OS, int MX, bool XR>
__device__ __forceinline__ void compute_frag(const Frag<P, U, OS>& f, const DeviceView& v,
                                             int64_t row0, int64_t row_end, int lt, int team,
                                             const uint16_t* xs, int xstride,
                                             const float (&xor_)[MX][OS], int M,
                                             uint16_t* __restrict__ y, const Nib nb,
                                             const half2_t (&xreg)[P][16]) {
  constexpr int T = kBlock / L;
  const int G = v.G, n_out = v.n_out;
  // The x slots are the same for every tile.  With several rows of x the
  // compiler would keep all of them in registers across tiles (MX * P * 16,
  // which spills); an opaque zero in the address makes it read them per tile.
  int x0 = 0, slot_dep = 0;
  if constexpr (MX > 1) asm volatile("v_mov_b32 %0, 0" : "=v"(x0));
  float acc[MX][U];
#pragma unroll
  for (int m = 0; m < MX; ++m)
#pragma unroll
    for (int u = 0; u < U; ++u) acc[m][u] = 0.f;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int g = lt + L * p;
    const int slot = (g < G ? g : 0) * kXSlot + x0 + slot_dep;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // flat group index (row * G + g): its parity picks the zero nibble
      const uint32_t odd = (((uint32_t)(row0 + team + (int64_t)u * T) & (uint32_t)G) ^ (uint32_t)g) & 1u;
      const uint32_t z = (f.z[u][p] >> (4u * odd)) & 0xFu;
      const float sc = h2f((uint16_t)f.s[u][p]);
      if constexpr (MX == 1) {
        if constexpr (XR) {
          acc[0][u] = __builtin_fmaf(sc, group_dot(f.c[u][p], z, xreg[p], nb), acc[0][u]);
        } else {
          half2_t xr[16];
          read_x(xs + slot, xr);
          acc[0][u] = __builtin_fmaf(sc, group_dot(f.c[u][p], z, xr, nb), acc[0][u]);
        }
      } else {
        half2_t wq[16];
        dequant_record(f.c[u][p], z ^ slot_dep, nb, wq);
        int mdep = 0;  // four rows: the x reads of row m + 2 wait for row m's products
#pragma unroll
        for (int m = 0; m < MX; ++m) {
          half2_t xr[16];
          read_x(xs + m * xstride + slot + mdep, xr);
          acc[m][u] = __builtin_fmaf(sc, dot_record(wq, xr), acc[m][u]);
          if (MX > 2 && m % 2 == 1) asm volatile("" : "+v"(mdep) : "v"(acc[m][u]));
        }
        // The next group's x reads and dequantization take an opaque zero
        // produced after this group's products: one group in registers at a
        // time (16 pairs + MX * 16 x values), else the compiler front-loads
        // every group and spills.
        asm volatile("" : "+v"(slot_dep) : "v"(acc[MX - 1][u]));
      }
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t n = row0 + team + (int64_t)u * T;
#pragma unroll
    for (int m = 0; m < MX; ++m) {
      float a = acc[m][u];
#pragma unroll
      for (int s = 0; s < OS; ++s) a = __builtin_fmaf(xor_[m][s], h2f((uint16_t)f.o[u][s]), a);
      if (n < row_end && n_out > L * OS) {  // heavy-tailed columns beyond the register slots
        const uint16_t* orow = v.outliers + n * n_out;
        const uint16_t* xo = xs + m * xstride + kXSlot * G;
        for (int j = lt + L * OS; j < n_out; j += L) a = __builtin_fmaf(h2f(xo[j]), h2f(orow[j]), a);
      }
      const float s = team_sum<L>(a);
      if (lt == 0 && n < row_end && m < M) y[(int64_t)m * v.N + n] = f2h(s);
    }
  }
}

// NT == 0: the block walks the tiles b, b + B, b + 2B, ... of its container
// (long launches).  NT >= 1: the block owns rows_per_block consecutive rows,
// at most NT tiles (short launches: every block gets the same number of rows,
// where whole tiles would leave some blocks a tile more than others).
//
// MX rows of x (a batch tile, M <= MX) share every dequantized record.
template <int L, int P, int U, int NT, int MX>
__global__ __launch_bounds__(kBlock) void k_gemv_m1(const unsigned char* base0, const uint16_t* x0, uint16_t* y0,
                                                    const int32_t N0, const int32_t K0, const int32_t n_out0,
                                                    const int32_t spread0, const int32_t m_rows,
                                                    const int32_t begin1, const int32_t begin2,
                                                    const int32_t begin3, const GemvTasks tasks) {
  constexpr int OS = (L == 16) ? 4 : 2;  // heavy-tailed slots per lane held in registers
  constexpr int T = kBlock / L;          // teams per block
  constexpr int kTileRows = T * U;
  extern __shared__ __align__(16) unsigned char smem[];
  DeviceView v;
  const uint16_t* xp;
  uint16_t* yp;
  int32_t spread;  // NT >= 1: rows per block; NT == 0: blocks of the task
  int first = 0;   // the task's first block
  const int32_t bx = (int32_t)blockIdx.x;
  if (bx < begin1) {
    // task 0 from the preloaded arguments alone: section addresses from the
    // container base and the shape, no memory access
    const Layout lay = make_layout(K0, N0, n_out0);
    v.codes = reinterpret_cast<const uint4*>(base0 + lay.codes);
    v.scales = reinterpret_cast<const uint16_t*>(base0 + lay.scales);
    v.zeros = base0 + lay.zeros;
    v.outliers = reinterpret_cast<const uint16_t*>(base0 + lay.outliers);
    v.perm = reinterpret_cast<const int32_t*>(base0 + lay.perm);
    v.mask = reinterpret_cast<const uint32_t*>(base0 + lay.mask);
    v.N = N0;
    v.K = K0;
    v.n_out = n_out0;
    v.K_b = K0 - n_out0;
    v.G = (v.K_b + kGroup - 1) / kGroup;
    v.cu_count = 0;
    v.lds_per_block = 0;
    xp = x0;
    yp = y0;
    spread = spread0;
  } else {
    int ti = 1;
    first = begin1;
    if (bx >= begin3) {
      ti = 3;
      first = begin3;
#pragma unroll
      for (int i = 4; i < kMaxTasks; ++i)
        if (bx >= tasks.begin[i]) {
          ti = i;
          first = tasks.begin[i];
        }
    } else if (bx >= begin2) {
      ti = 2;
      first = begin2;
    }
    const GemvTask& task = tasks.t[ti];
    // Every field of the task in scalar registers at once: used one by one,
    // the compiler spreads their loads over several dependent round trips.
    asm volatile("" ::"s"(task.v.codes), "s"(task.v.scales), "s"(task.v.zeros), "s"(task.v.outliers),
                 "s"(task.v.perm), "s"(task.x), "s"(task.y), "s"(task.v.N), "s"(task.v.K), "s"(task.v.K_b),
                 "s"(task.v.G), "s"(task.v.n_out), "s"(task.nblocks), "s"(task.rows_per_block));
    v = task.v;
    xp = task.x;
    yp = task.y;
    spread = NT ? task.rows_per_block : task.nblocks;
  }
  // Nibble masks in scalar registers and fp16 magics in vector registers,
  // written so the compiler cannot fold them back into literals (see Nib).
  const Nib nb = make_nib();
  const int G = v.G, n_out = v.n_out;
  const int xstride = ((kXSlot * G + n_out) + 7) & ~7;  // halves per x row; 16-byte multiple
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  uint16_t* xraw = xs + MX * xstride;
  const int tid = threadIdx.x;
  const int lt = tid % L;
  const int team = tid / L;
  const int64_t lb = (int64_t)((int32_t)blockIdx.x - first);
  // NT >= 1: rows [row, end) in tiles of kTileRows; NT == 0: tiles `stride` apart
  const int64_t stride = NT ? (int64_t)kTileRows : (int64_t)spread * kTileRows;
  int64_t row = NT ? lb * spread : lb * kTileRows;
  const int64_t end = NT ? (row + spread < v.N ? row + spread : v.N) : v.N;

  // The first tile's weights are requested right behind the x and perm
  // loads, so their HBM latency overlaps the gather and the barriers.
  Frag<P, U, OS> fa, fb;
  half2_t xreg[P][16];  // used by the long loop with one row of x
  stage_x<MX>(v, xp, m_rows, xs, xstride, xraw, tid, [&] {
    __builtin_amdgcn_sched_barrier(0);
    load_frag<L, P, U, OS>(fa, v, row, end, lt, team);
    __builtin_amdgcn_sched_barrier(0);
  });
  __syncthreads();

  float xor_[MX][OS];
#pragma unroll
  for (int m = 0; m < MX; ++m)
#pragma unroll
    for (int s = 0; s < OS; ++s) {
      const int j = lt + L * s;
      xor_[m][s] = j < n_out ? h2f(xs[m * xstride + kXSlot * G + j]) : 0.f;
    }
  // Two register buffers: the next tile is in flight while this one is
  // computed.  Neither form has an early exit between a load and the compute
  // that uses it (a tile past `end` loads nothing and its compute is skipped
  // by a branch that holds no loads), and scheduling barriers keep work on
  // the current tile's values below the next tile's load instructions: both
  // let the compiler wait for exactly the current tile, so the next one
  // stays in flight.
  if constexpr (NT >= 1) {
    // several tiles: this lane's groups of x are read from LDS once
    constexpr bool XR = MX == 1 && P <= 5 && NT >= 2;
    if constexpr (XR) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int g = lt + L * p;
        read_x(xs + (g < G ? g : 0) * kXSlot, xreg[p]);
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      Frag<P, U, OS>& cur = (t & 1) ? fb : fa;
      Frag<P, U, OS>& nxt = (t & 1) ? fa : fb;
      if (t + 1 < NT) load_frag<L, P, U, OS>(nxt, v, row + (t + 1) * stride, end, lt, team);
      __builtin_amdgcn_sched_barrier(0);
      if (row + t * stride < end)
        compute_frag<L, P, U, OS, MX, XR>(cur, v, row + t * stride, end, lt, team, xs, xstride, xor_, m_rows, yp,
                                          nb, xreg);
    }
  } else {
    // One row of x: this lane's groups of x stay in registers across the
    // tiles (the long loop reads them from LDS once instead of per tile).
    constexpr bool XR = MX == 1 && P <= 5;  // 16 registers per slot: more would spill
    if constexpr (XR) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int g = lt + L * p;
        read_x(xs + (g < G ? g : 0) * kXSlot, xreg[p]);
      }
    }
    for (; row < v.N; row += 2 * stride) {
      load_frag<L, P, U, OS>(fb, v, row + stride, end, lt, team);
      __builtin_amdgcn_sched_barrier(0);
      compute_frag<L, P, U, OS, MX, XR>(fa, v, row, end, lt, team, xs, xstride, xor_, m_rows, yp, nb,
                                        xreg);
      load_frag<L, P, U, OS>(fa, v, row + 2 * stride, end, lt, team);
      __builtin_amdgcn_sched_barrier(0);
      if (row + stride < v.N)
        compute_frag<L, P, U, OS, MX, XR>(fb, v, row + stride, end, lt, team, xs, xstride, xor_, m_rows, yp,
                                          nb, xreg);
    }
  }
}

struct Variant {
  int L, P;
};

// Lanes-per-row L and slots-per-lane P = ceil(G/L) with the best lane use
// (ties: fewer slots, i.e. fewer registers).  P == 0: no variant fits.
// One exception, measured: with one row of x and 64 < G <= 96, 32-lane teams
// (3 slots; 83 % of the lanes busy at G = 80) beat fully used 16-lane teams
// (5 slots).  A short launch's block then walks twice as many tiles of half
// the rows, so one tile's transfer overlaps the previous one's arithmetic
// (the 4B-class decode step's q/k/v and gate/up launches at K = 2560: step
// 1.046 -> 1.008 ms, gate/up 9.7 -> 8.9 us); a long launch at G = 80 was
// unchanged, and at G = 48 (K = 1536) the 32-lane teams were slower.
Variant pick_variant(int G, int mx) {
  if (mx == 1 && G > 64 && G <= 96) return Variant{32, (G + 31) / 32};
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

// LDS of one block: MX rows of x in group slots, plus the raw x of one row.
size_t lds_bytes(const DeviceView& v, int mx) {
  const size_t xstride = (((size_t)kXSlot * v.G + (size_t)v.n_out) + 7) & ~(size_t)7;
  return 2 * (size_t)mx * xstride + 16 * (((size_t)v.K + 7) / 8);
}

size_t lds_limit(const DeviceView& v) {
  const size_t dev = v.lds_per_block > 0 ? (size_t)v.lds_per_block : 64 * 1024;
  return dev < (size_t)160 * 1024 ? dev : (size_t)160 * 1024;
}

// Rows of x one launch carries: M = 1, 2 or up to 4 (rows past M read zeros).
int batch_tile(int64_t M) { return M <= 1 ? 1 : (M == 2 ? 2 : 4); }

constexpr int kU = SPECTRA_GEMV_U;
constexpr int64_t kPipeTiles = 6;  // tiles per block from which the loop without early exits pays

// Split a budget of per_cu blocks per CU between the tasks in proportion to
// their rows, never past the budget (one block over it would run as a second
// round on some CU and cost the launch a whole extra block's time).
int64_t plan_blocks(GemvTasks& ts, int64_t per_cu) {
  int64_t total_rows = 0;
  for (int i = 0; i < ts.count; ++i) total_rows += ts.t[i].v.N;
  const int64_t budget = (int64_t)ts.t[0].v.cu_count * per_cu;
  int64_t nb[kMaxTasks], used = 0;
  for (int i = 0; i < ts.count; ++i) {
    // more blocks than whole tiles is fine: short launches then give every
    // block a partial tile (rows_per_block below the tile)
    int64_t b = budget * ts.t[i].v.N / total_rows;
    if (b > ts.t[i].v.N) b = ts.t[i].v.N;
    if (b < 1) b = 1;
    nb[i] = b;
    used += b;
  }
  for (bool grew = true; used < budget && grew;) {  // hand out what flooring left over
    grew = false;
    for (int i = 0; i < ts.count && used < budget; ++i)
      if (nb[i] < ts.t[i].v.N) {
        ++nb[i];
        ++used;
        grew = true;
      }
  }
  int64_t begin = 0;
  for (int i = 0; i < kMaxTasks; ++i) {
    ts.begin[i] = i < ts.count ? (int32_t)begin : INT32_MAX;
    if (i < ts.count) {
      ts.t[i].nblocks = (int32_t)nb[i];
      begin += nb[i];
    }
  }
  return begin;
}

template <int L, int P, int NT, int MX>
hipError_t launch_k(dim3 grid, size_t lds, hipStream_t s, const GemvTasks& ts, int32_t m_rows) {
  const void* fn = reinterpret_cast<const void*>(&k_gemv_m1<L, P, kU, NT, MX>);
  if (lds > 64 * 1024) {  // dynamic LDS past 64 KiB must be allowed per kernel
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const DeviceView& v0 = ts.t[0].v;
  const Layout lay = make_layout(v0.K, v0.N, v0.n_out);
  const unsigned char* base0 = reinterpret_cast<const unsigned char*>(v0.codes) - lay.codes;
  const int32_t spread0 = NT ? ts.t[0].rows_per_block : ts.t[0].nblocks;
  hipLaunchKernelGGL((k_gemv_m1<L, P, kU, NT, MX>), grid, dim3(kBlock), lds, s, base0, ts.t[0].x, ts.t[0].y,
                     (int32_t)v0.N, v0.K, v0.n_out, spread0, m_rows, ts.begin[1], ts.begin[2], ts.begin[3], ts);
  return hipGetLastError();
}

template <int L, int P, int MX>
hipError_t launch_lp(GemvTasks& ts, size_t lds, hipStream_t s, int32_t m_rows) {
  constexpr int64_t kTileRows = (int64_t)(kBlock / L) * kU;
  int64_t blocks = plan_blocks(ts, SPECTRA_GEMV_BLOCKS_PER_CU);
  int64_t most = 0, all_tiles = 0;  // most tiles any block walks when blocks take whole tiles in turn
  for (int i = 0; i < ts.count; ++i) {
    const int64_t tiles = (ts.t[i].v.N + kTileRows - 1) / kTileRows;
    const int64_t per = (tiles + ts.t[i].nblocks - 1) / ts.t[i].nblocks;
    most = per > most ? per : most;
    all_tiles += tiles;
  }
  if (MX > 1 || most >= kPipeTiles) {  // batch tiles always take the loop form
    // Long launches run a second block per CU (16 waves: one wave's dequant
    // work overlaps another's loads) when two fit, registers and LDS as the
    // occupancy calculator counts them, and every block still walks several
    // tiles.
    if (all_tiles >= (int64_t)ts.t[0].v.cu_count * 2 * SPECTRA_GEMV_TWO_BLOCK_TILES) {
      int fit = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
              &fit, reinterpret_cast<const void*>(&k_gemv_m1<L, P, kU, 0, MX>), kBlock, lds) == hipSuccess &&
          fit >= 2)
        blocks = plan_blocks(ts, 2);
    }
    for (int i = 0; i < ts.count; ++i) ts.t[i].rows_per_block = 0;
    return launch_k<L, P, 0, MX>(dim3((unsigned)blocks), lds, s, ts, m_rows);
  }
  const dim3 grid((unsigned)blocks);
  // Short launch: equal row ranges per block, at most nt tiles each.
  int64_t nt = 1;
  for (int i = 0; i < ts.count; ++i) {
    const int64_t r = (ts.t[i].v.N + ts.t[i].nblocks - 1) / ts.t[i].nblocks;
    ts.t[i].rows_per_block = (int32_t)r;
    const int64_t t = (r + kTileRows - 1) / kTileRows;
    nt = t > nt ? t : nt;
  }
  switch (nt) {
    case 1: return launch_k<L, P, 1, 1>(grid, lds, s, ts, m_rows);
    case 2: return launch_k<L, P, 2, 1>(grid, lds, s, ts, m_rows);
    case 3: return launch_k<L, P, 3, 1>(grid, lds, s, ts, m_rows);
    case 4: return launch_k<L, P, 4, 1>(grid, lds, s, ts, m_rows);
    default: return launch_k<L, P, 5, 1>(grid, lds, s, ts, m_rows);
  }
}

// Most slots per lane a batch tile of MX rows of x runs without spilling registers.
constexpr int max_slots(int mx) { return mx >= 4 ? 4 : 8; }

template <int L, int MX>
hipError_t launch_l(int P, GemvTasks& ts, size_t lds, hipStream_t s, int32_t m_rows) {
  if constexpr (max_slots(MX) < 8) {
    switch (P) {
      case 1: return launch_lp<L, 1, MX>(ts, lds, s, m_rows);
      case 2: return launch_lp<L, 2, MX>(ts, lds, s, m_rows);
      case 3: return launch_lp<L, 3, MX>(ts, lds, s, m_rows);
      case 4: return launch_lp<L, 4, MX>(ts, lds, s, m_rows);
      default: return hipErrorNotSupported;
    }
  } else {
    switch (P) {
      case 1: return launch_lp<L, 1, MX>(ts, lds, s, m_rows);
      case 2: return launch_lp<L, 2, MX>(ts, lds, s, m_rows);
      case 3: return launch_lp<L, 3, MX>(ts, lds, s, m_rows);
      case 4: return launch_lp<L, 4, MX>(ts, lds, s, m_rows);
      case 5: return launch_lp<L, 5, MX>(ts, lds, s, m_rows);
      case 6: return launch_lp<L, 6, MX>(ts, lds, s, m_rows);
      case 7: return launch_lp<L, 7, MX>(ts, lds, s, m_rows);
      case 8: return launch_lp<L, 8, MX>(ts, lds, s, m_rows);
      default: return hipErrorNotSupported;
    }
  }
}

template <int MX>
hipError_t launch_mx(int L, int P, GemvTasks& ts, size_t lds, hipStream_t s, int32_t m_rows) {
  switch (L) {
    case 16: return launch_l<16, MX>(P, ts, lds, s, m_rows);
    case 32: return launch_l<32, MX>(P, ts, lds, s, m_rows);
    default: return launch_l<64, MX>(P, ts, lds, s, m_rows);
  }
}

hipError_t launch_tasks(GemvTasks& ts, int64_t M, hipStream_t s) {
  const int mx = batch_tile(M);
  int gmax = 0;
  size_t lds = 0;
  for (int i = 0; i < ts.count; ++i) {
    if (ts.t[i].v.G > gmax) gmax = ts.t[i].v.G;
    const size_t b = lds_bytes(ts.t[i].v, mx);
    if (b > lds) lds = b;
  }
  const Variant vr = pick_variant(gmax, mx);
  if (vr.P == 0 || lds > lds_limit(ts.t[0].v)) return hipErrorNotSupported;
  switch (mx) {
    case 1: return launch_mx<1>(vr.L, vr.P, ts, lds, s, (int32_t)M);
    case 2: return launch_mx<2>(vr.L, vr.P, ts, lds, s, (int32_t)M);
    default: return launch_mx<4>(vr.L, vr.P, ts, lds, s, (int32_t)M);
  }
}

}  // namespace

bool gemv_variant(int G, int* L, int* P) {
  const Variant vr = pick_variant(G, 1);
  *L = vr.L;
  *P = vr.P;
  return vr.P > 0;
}

bool gemv_supports(const DeviceView& v, int64_t M) {
  if (M < 1 || M > 4) return false;
  if (v.N > INT32_MAX) return false;  // rows travel as a 32-bit kernel argument
  if (M > 1 && v.K % 8 != 0) return false;  // each row of x must start 16-byte aligned
  // a block stages at most kXChunks * 8 * kBlock channels and kQuads * 4 * kBlock bulk positions
  if (v.K > kXChunks * 8 * kBlock || (int64_t)kGroup * v.G > (int64_t)kQuads * 4 * kBlock) return false;
  const int P = pick_variant(v.G, batch_tile(M)).P;
  if (P == 0 || P > max_slots(batch_tile(M))) return false;
  return lds_bytes(v, batch_tile(M)) <= lds_limit(v);
}

hipError_t launch_gemv(const DeviceView& v, const uint16_t* x, uint16_t* y, int64_t M,
                       hipStream_t s) {
  if (!gemv_supports(v, M)) return hipErrorNotSupported;
  GemvTasks ts;
  ts.count = 1;
  ts.t[0].v = v;
  ts.t[0].x = x;
  ts.t[0].y = y;
  return launch_tasks(ts, M, s);
}

hipError_t launch_gemv_grouped(const DeviceView* vs, int count, const uint16_t* x,
                               uint16_t* const* ys, hipStream_t s) {
  for (int base = 0; base < count; base += kMaxTasks) {
    GemvTasks ts;
    ts.count = (count - base < kMaxTasks) ? count - base : kMaxTasks;
    for (int i = 0; i < ts.count; ++i) {
      if (!gemv_supports(vs[base + i], 1)) return hipErrorNotSupported;
      ts.t[i].v = vs[base + i];
      ts.t[i].x = x;
      ts.t[i].y = ys[base + i];
    }
    const hipError_t e = launch_tasks(ts, 1, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace spectra
