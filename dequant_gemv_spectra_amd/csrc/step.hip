// Persistent decode-step kernel for gfx950: a chain of dependent M = 1
// SPECTRA products (y = x W_hat^T per container) run by one launch.
//
// Why.  At decode every token streams every weight once (techfi24 summary,
// section on the hardware context) and the page runs its fused kernels
// under graph replay to cut launch overhead (SPECTRA page, abstract and
// highlight 3).  A layer's projections depend on each other (q/k/v -> o ->
// gate/up -> down), and with one launch per projection every launch pays its
// dispatch, argument loads, x staging and the first weights' HBM latency
// before any byte streams: about 3 us on launches whose weights take 1 - 5
// us to stream.  Here one grid of one block per compute unit runs the whole
// chain; a block requests the next projection's weights (which do not depend
// on x) before the projection it works on is finished, so HBM keeps
// streaming across the dependency.
//
// Dependencies.  A phase is a set of containers that share one input x (up
// to four: q/k/v, gate/up).  Its input is either an external fp16 vector or
// the output of task 0 of an earlier phase.  Producers write each output
// value a second time as a 32-bit word (launch tag << 16 | fp16 bits) with
// agent-scope stores; a consumer's control wave loads the whole input with
// agent-scope loads and accepts it once every word carries this launch's
// tag.  Data and the "ready" mark arrive in the same aligned word, so the
// wait costs one round trip after the last producer's store lands, and no
// counter, fence or cache flush is involved.  The tag of a launch is
// 1 + (launches completed so far mod 65535), read from device memory at the
// start; the last block to finish advances the count, so replays of one
// plan (also inside a captured graph) need no argument change.  Every wait
// is bounded: past the poll limit the block records the timeout in the
// plan's error word and carries on with what it has, so the kernel always
// drains; the host reads the word with spectra_step_status.
//
// Block layout.  512 threads: waves 0 - 6 compute (448 lanes), wave 7 is the
// control wave.  The control wave loads the next phase's perm into LDS while
// the others compute, then stages x (external or polled) into LDS in channel
// order; all 512 threads gather it into bulk order (80-byte group slots) and
// the compute lanes copy their groups of x into registers.  Compute mapping
// as in the single-product GEMV: teams of L lanes (16, 32 or 64) own one
// row; lane t owns groups t + L*p, p < P <= 5; a tile is 448 / L rows.
// Every phase of a block has an even number of tiles (an empty one pads an
// odd count), so the two register buffers alternate in a fixed order and
// every tile load issues the same 19 instructions: the compiler's count of
// loads in flight then stays exact across phases, and the last two tiles'
// loads of a phase are the next phase's first two tiles.
//
// The arithmetic and its order per output are those of the GEMV (same lane
// to group assignment, fp32 accumulation, team reduction), so each output
// equals the single-product GEMV's bit for bit.
#include <math.h>
#include <string.h>

#include <new>
#include <string>
#include <vector>

#include "../../include/spectra.h"
#include "gemv_common.h"

namespace spectra {
namespace {

using namespace g32k;

constexpr int kStepBlock = 512;
constexpr int kCompute = 448;       // lanes of the compute waves
constexpr int kCtlWave = 7;         // wave index of the control wave
constexpr int kSP = 5;              // most group slots per lane
constexpr int kSOS = 4;             // heavy-tailed slots per lane
constexpr uint32_t kPollLimit = 1u << 16;
#ifndef SPECTRA_STEP_PREFETCH
#define SPECTRA_STEP_PREFETCH 0
#endif
constexpr int kPrefetch = SPECTRA_STEP_PREFETCH;  // where the next phase's first tiles are requested

// One tile of weights for a lane.  Scales, zero bytes and heavy-tailed
// weights keep the loads' own widths, so no conversion sits between a load
// and the compute that reads it (a conversion next to the load would make the
// compiler wait for it there).
// Block barrier for LDS hand-offs; global loads and stores stay in flight.
__device__ __forceinline__ void bar() { __syncthreads(); }

struct Frag {
  uint4 c[kSP];
  unsigned short s[kSP];
  unsigned char z[kSP];
  unsigned short o[kSOS];
};

// The rows one block owns in one phase.
struct BT {
  const uint4* codes;
  const uint16_t* scales;
  const uint8_t* zeros;
  const uint16_t* outliers;
  const int32_t* perm;
  uint16_t* y;
  uint32_t* ytag;
  int32_t K, K_b, G, n_out;
  int32_t lg, P;
  int32_t row0, row_end, ntiles;
  float xscale;   // the phase's input scale
  int32_t tagged; // the input is an earlier phase's tagged output
};

__device__ __forceinline__ BT resolve(const StepPhaseDev* __restrict__ ph, int p, int nph, int b) {
  BT r;
  if (p >= nph) {  // past the last phase: empty tiles
    r.codes = nullptr;
    r.scales = nullptr;
    r.zeros = nullptr;
    r.outliers = nullptr;
    r.perm = nullptr;
    r.y = nullptr;
    r.ytag = nullptr;
    r.K = r.K_b = r.G = r.n_out = 0;
    r.lg = 6;
    r.P = 0;
    r.row0 = r.row_end = 0;
    r.ntiles = 2;
    r.xscale = 1.0f;
    r.tagged = 0;
    return r;
  }
  const StepPhaseDev& P = ph[__builtin_amdgcn_readfirstlane(p)];  // scalar loads of the descriptor
  int i = 0;
#pragma unroll
  for (int j = 1; j < kStepMaxTasks; ++j)
    if (j < P.ntasks && b >= P.t[j].first_block) i = j;
  const StepTaskDev& t = P.t[i];
  r.codes = t.codes;
  r.scales = t.scales;
  r.zeros = t.zeros;
  r.outliers = t.outliers;
  r.perm = t.perm;
  r.y = t.y;
  r.ytag = t.ytag;
  r.K = t.K;
  r.K_b = t.K_b;
  r.G = t.G;
  r.n_out = t.n_out;
  r.lg = P.lg;
  r.P = P.P;
  const int lb = b - t.first_block;
  const int64_t row0 = (int64_t)lb * t.rows_per_block;
  const int64_t end = row0 + t.rows_per_block < t.N ? row0 + t.rows_per_block : (int64_t)t.N;
  r.row0 = (int32_t)(row0 < t.N ? row0 : t.N);
  r.row_end = (int32_t)(end > r.row0 ? end : r.row0);
  r.ntiles = t.ntiles;
  r.xscale = P.x_scale;
  r.tagged = P.xtag != nullptr;
  return r;
}

// Loads tile t of the block's rows (rows past row_end, slots p >= P and
// groups past G read zeros through the range checks).  Always 19 loads.
__device__ __forceinline__ void load_tile(Frag& f, const BT& bt, int t, int tid) {
  const int lg = bt.lg, L = 1 << lg, T = kCompute >> lg;
  const int lt = tid & (L - 1), team = tid >> lg;
  const int G = bt.G, n_out = bt.n_out;
  const int32_t row_a = bt.row0 + t * T;  // rows fit in 31 bits; all of this is scalar
  const int32_t left = bt.row_end - row_a;
  const int32_t rows = left < T ? (left > 0 ? left : 0) : T;
  const int64_t i0 = (int64_t)row_a * G;
  const __amdgpu_buffer_rsrc_t rc = rsrc(bt.codes + i0, (uint64_t)rows * G * 16);
  const __amdgpu_buffer_rsrc_t rs = rsrc(bt.scales + i0, (uint64_t)rows * G * 2);
  const int64_t zb0 = i0 >> 1;
  const uint32_t i0odd = (uint32_t)(i0 & 1);
  const __amdgpu_buffer_rsrc_t rz =
      rsrc(bt.zeros + zb0, rows ? (uint64_t)(((i0 + rows * G + 1) >> 1) - zb0) : 0);
  const __amdgpu_buffer_rsrc_t ro = rsrc(bt.outliers + (int64_t)row_a * n_out, (uint64_t)rows * n_out * 2);
#pragma unroll
  for (int p = 0; p < kSP; ++p) {
    const int g = lt + L * p;
    const uint32_t local = (uint32_t)(team * G + g);
    const bool ok = p < bt.P && g < G;
    const u32x4 c = __builtin_amdgcn_raw_buffer_load_b128(rc, ok ? local * 16u : kOob, 0, kStream);
    f.c[p] = make_uint4(c.x, c.y, c.z, c.w);
    f.s[p] = __builtin_amdgcn_raw_buffer_load_b16(rs, ok ? local * 2u : kOob, 0, 0);
    f.z[p] = __builtin_amdgcn_raw_buffer_load_b8(rz, ok ? (local + i0odd) >> 1 : kOob, 0, 0);
  }
#pragma unroll
  for (int s = 0; s < kSOS; ++s) {
    const int j = lt + L * s;
    f.o[s] = __builtin_amdgcn_raw_buffer_load_b16(ro, j < n_out ? (uint32_t)(team * n_out + j) * 2u : kOob, 0, 0);
  }
}

// Team sum for a runtime team width 2^lg (16, 32 or 64): the GEMV's sequence.
__device__ __forceinline__ float team_sum_rt(float v, int lg) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x124>(v);
  v += dpp<0x128>(v);
  if (lg >= 5) v += __shfl_xor(v, 16);
  if (lg >= 6) v += __shfl_xor(v, 32);
  return v;
}

// Computes tile t and stores its outputs (plain fp16, plus the tagged word
// when a later phase reads this output).  No memory loads; the two stores
// are issued by every lane of every tile through range-checked descriptors
// (offsets past the range for lanes without an output, for empty tiles and
// for outputs no phase reads), so the count of memory operations in flight
// is the same on every path.
// sum over the first P slots of s16 * sum_e (q_e - z) * x_e, unrolled.
template <int P>
__device__ __forceinline__ float slots_dot(const Frag& f, int lt, int L, int G, int32_t n,
                                          const half2_t (&xreg)[kSP][16], const Nib nb) {
  float acc = 0.f;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int g = lt + L * p;
    const uint32_t odd = (((uint32_t)n & (uint32_t)G) ^ (uint32_t)g) & 1u;  // parity of the flat group index
    const uint32_t z = ((uint32_t)f.z[p] >> (4u * odd)) & 0xFu;
    acc = __builtin_fmaf(h2f(f.s[p]), group_dot(f.c[p], z, xreg[p], nb), acc);
  }
  return acc;
}

__device__ __forceinline__ void compute_tile(const Frag& f, const BT& bt, int t, int tid,
                                             const half2_t (&xreg)[kSP][16], const float (&xo)[kSOS],
                                             const Nib nb, uint32_t tag) {
  const int lg = bt.lg, L = 1 << lg, T = kCompute >> lg;
  const int lt = tid & (L - 1), team = tid >> lg;
  const int32_t row_a = bt.row0 + t * T;
  const int G = bt.G;
  const int32_t n = row_a + team;
  float sum = 0.f;
  if (row_a < bt.row_end) {  // an empty tile skips the arithmetic (block-uniform)
    // The phase's P slots (groups past G loaded zero codes, zero points and
    // scales, so they add exactly 0).  Only arithmetic sits inside the
    // branches: every load was issued before, the same way on every path.
    float acc;
    switch (bt.P) {
      case 1: acc = slots_dot<1>(f, lt, L, G, n, xreg, nb); break;
      case 2: acc = slots_dot<2>(f, lt, L, G, n, xreg, nb); break;
      case 3: acc = slots_dot<3>(f, lt, L, G, n, xreg, nb); break;
      case 4: acc = slots_dot<4>(f, lt, L, G, n, xreg, nb); break;
      default: acc = slots_dot<5>(f, lt, L, G, n, xreg, nb); break;
    }
#pragma unroll
    for (int s = 0; s < kSOS; ++s) acc = __builtin_fmaf(xo[s], h2f(f.o[s]), acc);
    sum = team_sum_rt(acc, lg);
  }
  const bool mine = lt == 0 && n < bt.row_end;
  const uint32_t h = f2h(sum);
  const __amdgpu_buffer_rsrc_t ry = rsrc(bt.y, (uint64_t)bt.row_end * 2);
  const __amdgpu_buffer_rsrc_t rt = rsrc(bt.ytag, bt.ytag ? (uint64_t)bt.row_end * 4 : 0);
  __builtin_amdgcn_raw_buffer_store_b16((unsigned short)h, ry, mine ? (uint32_t)n * 2u : kOob, 0, 0);
  __builtin_amdgcn_raw_buffer_store_b32((tag << 16) | h, rt, mine ? (uint32_t)n * 4u : kOob, 0, kAgentScope);
}

__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// One 16-byte chunk per lane into LDS without passing through registers
// (buffer_load ... lds): chunk c = i*64 + lane of the buffer lands at
// lds_base + c*16 bytes, for c < nck only (a lane past the end issues
// nothing, so the LDS area needs exactly nck chunks).  Chunks past the
// descriptor's range read zeros.
template <int AUX>
__device__ __forceinline__ void lds_chunk(__amdgpu_buffer_rsrc_t r, void* lds_base, int i, int lane, int nck) {
  if (i * 64 + lane < nck)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, static_cast<unsigned char*>(lds_base) + i * 1024, 16,
                                             (uint32_t)(i * 64 + lane) * 16u, 0, 0, AUX);
}

// Control wave: perm of the phase into LDS (the perm section is padded to
// 256 bytes, so whole chunks stay inside the container).  Completes at the
// control wave's next wait_vm().
__device__ __forceinline__ void ctl_load_perm(const BT& bt, int32_t* perm_lds, int lane) {
  const int nck = (bt.K + 3) >> 2;
  const __amdgpu_buffer_rsrc_t rp = rsrc(bt.perm, (uint64_t)nck * 16);
  for (int i = 0; i * 64 < nck; ++i) lds_chunk<0>(rp, perm_lds, i, lane, nck);
}

// Control wave: the input of phase p into LDS, all of it requested at once.
// External input: fp16 in channel order (xin), the partial last chunk element
// by element.  Tagged input: 32-bit words (tag << 16 | fp16) in channel order
// (also xin), requested again chunk by chunk until every word carries `tag`.
// Returns false when a wait gave up.
__device__ __forceinline__ bool ctl_stage_x(const StepPhaseDev* __restrict__ ph, int p, int K, void* xin, int lane,
                                            uint32_t tag, uint32_t limit, StepCtl* ctl, bool skip_wait) {
  const StepPhaseDev& P = ph[__builtin_amdgcn_readfirstlane(p)];
  const uint16_t* x = P.x;
  const uint32_t* xt = P.xtag;
  if (!xt) {
    const int full = K >> 3, nck = (K + 7) >> 3;
    const __amdgpu_buffer_rsrc_t rx = rsrc(x, (uint64_t)full * 16);
    for (int i = 0; i * 64 < nck; ++i) lds_chunk<0>(rx, xin, i, lane, nck);
    wait_vm();
    if ((K & 7) && lane == 0) {
      uint16_t* xr = static_cast<uint16_t*>(xin);
      for (int e = 8 * full; e < K; ++e) xr[e] = x[e];
    }
    return true;
  }
  const int nck = (K + 3) >> 2;  // 4 words per chunk; the buffer is padded to whole chunks
  const __amdgpu_buffer_rsrc_t rt = rsrc(xt, (uint64_t)nck * 16);
  const int per = (nck + 63) >> 6;  // chunks per lane, at most 64
  uint64_t pend = 0;
  for (int i = 0; i < per; ++i) {
    lds_chunk<kAgentScope>(rt, xin, i, lane, nck);
    if (i * 64 + lane < nck) pend |= 1ull << i;
  }
  const uint32_t* st = static_cast<const uint32_t*>(xin);
  bool ok = true;
  for (uint32_t polls = 0;; ++polls) {
    wait_vm();
    for (int i = 0; i < per; ++i) {
      if ((pend >> i) & 1) {
        const int w = 4 * (i * 64 + lane);
        const u32x4 t = *reinterpret_cast<const u32x4*>(st + w);
        const bool fresh = (t.x >> 16) == tag && (w + 1 >= K || (t.y >> 16) == tag) &&
                           (w + 2 >= K || (t.z >> 16) == tag) && (w + 3 >= K || (t.w >> 16) == tag);
        if (fresh || skip_wait) pend &= ~(1ull << i);
      }
    }
    if (__ballot(pend != 0) == 0) break;
    if (polls >= limit) {
      if (lane == 0) __hip_atomic_fetch_or(&ctl->err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      skip_wait = true;  // take what is there; the error word reports it
      ok = false;
      continue;
    }
    __builtin_amdgcn_s_sleep(2);
    for (int i = 0; i < per; ++i)
      if ((pend >> i) & 1) lds_chunk<kAgentScope>(rt, xin, i, lane, nck);
  }
  return ok;
}

// All 512 threads: x from channel order (xin: fp16, or tagged 32-bit words)
// into bulk-order group slots through perm, times the phase's scale; zeros up
// to 32G; then the heavy-tailed values.
template <bool TAGGED>
__device__ __forceinline__ void gather_t(const BT& bt, const void* xin, const int32_t* perm_lds, uint16_t* xs,
                                         int tid, float sc) {
  const int G = bt.G, K_b = bt.K_b, n_out = bt.n_out;
  const bool unit = sc == 1.0f;
  auto val = [&](int k) -> uint32_t {
    const uint32_t h = TAGGED ? (static_cast<const uint32_t*>(xin)[k] & 0xFFFFu) : static_cast<const uint16_t*>(xin)[k];
    return unit ? h : f2h(h2f((uint16_t)h) * sc);
  };
  const int nquad = 8 * G;
  for (int c = tid; c < nquad; c += kStepBlock) {
    const int j = 4 * c;
    const u32x4 pq = *reinterpret_cast<const u32x4*>(perm_lds + j);
    const uint32_t a0 = j + 0 < K_b ? val(pq.x) : 0u;
    const uint32_t a1 = j + 1 < K_b ? val(pq.y) : 0u;
    const uint32_t a2 = j + 2 < K_b ? val(pq.z) : 0u;
    const uint32_t a3 = j + 3 < K_b ? val(pq.w) : 0u;
    *reinterpret_cast<uint2*>(xs + xs_index(j)) = make_uint2(a0 | (a1 << 16), a2 | (a3 << 16));
  }
  const int xo_base = kXSlot * G;
  for (int j = tid; j < n_out; j += kStepBlock) xs[xo_base + j] = (uint16_t)val(perm_lds[K_b + j]);
  // No bulk group (every channel heavy-tailed): the lanes' one slot reads the
  // first 32 halves, which then hold the heavy-tailed x and zeros, never
  // stale LDS (times the zero codes they add exactly 0).
  if (G == 0)
    for (int j = n_out + tid; j < 32; j += kStepBlock) xs[j] = 0;
}

__device__ __forceinline__ void gather(const BT& bt, const void* xin, const int32_t* perm_lds, uint16_t* xs,
                                       int tid) {
  if (bt.tagged) gather_t<true>(bt, xin, perm_lds, xs, tid, bt.xscale);
  else gather_t<false>(bt, xin, perm_lds, xs, tid, bt.xscale);
}

// The block's tiles of one phase, two register buffers alternating.  On
// entry fa and fb hold (or have in flight) tiles 0 and 1.  Mode 0 (the
// build's choice): each tile is reloaded right after its compute, the last
// pair with the next phase's tiles 0 and 1.  Mode 1: the last pair computes
// (and stores) both tiles, signals the control wave (B0), then loads the
// next phase's first tiles, so this block's outputs leave ahead of that
// burst.  Mode 2: no load crosses a phase (the next phase loads its first
// tiles after its input is staged).  Measured on the 36-layer 4B-class step:
// 1.69, 1.78 and 1.83 ms.
__device__ __forceinline__ void run_phase(Frag& fa, Frag& fb, const BT& cur, const BT& nx, int tid,
                                          const uint16_t* xs, const Nib nb, uint32_t tag) {
  // this lane's P groups of x and its heavy-tailed x, into registers once
  const int L = 1 << cur.lg;
  const int lt = tid & (L - 1);
  half2_t xreg[kSP][16];
  float xo[kSOS];
#pragma unroll
  for (int q = 0; q < kSP; ++q) {
    const int g = lt + L * q;
    if (q < cur.P) read_x(xs + (g < cur.G ? g : 0) * kXSlot, xreg[q]);
  }
#pragma unroll
  for (int s = 0; s < kSOS; ++s) {
    const int j = lt + L * s;
    xo[s] = j < cur.n_out ? h2f(xs[kXSlot * cur.G + j]) : 0.f;
  }
  const int nt = cur.ntiles;
  int t = 0;
  for (; t + 2 < nt; t += 2) {
    compute_tile(fa, cur, t, tid, xreg, xo, nb, tag);
    load_tile(fa, cur, t + 2, tid);
    __builtin_amdgcn_sched_barrier(0);
    compute_tile(fb, cur, t + 1, tid, xreg, xo, nb, tag);
    load_tile(fb, cur, t + 3, tid);
    __builtin_amdgcn_sched_barrier(0);
  }
  compute_tile(fa, cur, t, tid, xreg, xo, nb, tag);
  if (kPrefetch == 0) load_tile(fa, nx, 0, tid);
  __builtin_amdgcn_sched_barrier(0);
  compute_tile(fb, cur, t + 1, tid, xreg, xo, nb, tag);
  if (kPrefetch == 0) {
    load_tile(fb, nx, 1, tid);
  } else {
    bar();  // B0: this block's outputs of the phase are stored
    if (kPrefetch == 1) {
      load_tile(fa, nx, 0, tid);
      load_tile(fb, nx, 1, tid);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

__global__ __launch_bounds__(kStepBlock) void k_step(const StepPhaseDev* __restrict__ ph, const int32_t nph,
                                                     StepCtl* ctl, const int32_t xin_bytes,
                                                     const int32_t perm_words) {
  extern __shared__ __align__(16) unsigned char smem[];
  void* xin = smem;  // staged input: fp16 or tagged words, channel order
  int32_t* perm_lds = reinterpret_cast<int32_t*>(smem + (size_t)xin_bytes);
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem + (size_t)xin_bytes + 4 * (size_t)perm_words);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.x;
  const uint32_t seq = __builtin_amdgcn_readfirstlane(
      __hip_atomic_load(&ctl->seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  const uint32_t tag = 1u + seq % 65535u;

  BT cur = resolve(ph, 0, nph, b);
  BT nx = resolve(ph, 1, nph, b);
  if (wave == kCtlWave) {
    const int lane = tid & 63;
    bool skip = __hip_atomic_load(&ctl->err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
    const uint32_t lim = ctl->poll_limit ? ctl->poll_limit : kPollLimit;
    const uint32_t want = (tag + ctl->tag_skew) & 0xFFFFu;  // the tag this block waits for
    ctl_load_perm(cur, perm_lds, lane);
    for (int p = 0; p < nph; ++p) {
      bar();  // B0: the compute waves are done with phase p - 1
      if (!ctl_stage_x(ph, p, cur.K, xin, lane, want, lim, ctl, skip)) skip = true;
      wait_vm();  // the perm chunks too
      bar();  // B1: x of phase p and its perm are in LDS
      gather(cur, xin, perm_lds, xs, tid);
      bar();  // B2: x is in bulk order
      if (p + 1 < nph) ctl_load_perm(nx, perm_lds, lane);
      cur = nx;
      nx = resolve(ph, p + 2, nph, b);
    }
  } else {
    const Nib nb = make_nib();
    Frag fa, fb;
    if (kPrefetch != 2) {
      load_tile(fa, cur, 0, tid);
      load_tile(fb, cur, 1, tid);
    }
    for (int p = 0; p < nph; ++p) {
      // B0 (modes 1, 2: the previous phase's last tile pair holds it, so here
      // only before the first phase)
      if (kPrefetch == 0 || p == 0) bar();
      bar();  // B1
      gather(cur, xin, perm_lds, xs, tid);
      bar();  // B2
      if (kPrefetch == 2) {
        load_tile(fa, cur, 0, tid);
        load_tile(fb, cur, 1, tid);
      }
      run_phase(fa, fb, cur, nx, tid, xs, nb, tag);
      cur = nx;
      nx = resolve(ph, p + 2, nph, b);
    }
  }
  bar();
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(&ctl->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1u == (seq + 1u) * (uint32_t)gridDim.x)
      __hip_atomic_store(&ctl->seq, seq + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace

const void* step_kernel() { return reinterpret_cast<const void*>(&k_step); }

hipError_t launch_step(const StepPhaseDev* table, int32_t nph, StepCtl* ctl, int32_t xin_bytes,
                       int32_t perm_words, size_t lds, int grid, hipStream_t s) {
  hipLaunchKernelGGL(k_step, dim3((unsigned)grid), dim3(kStepBlock), lds, s, table, nph, ctl, xin_bytes,
                     perm_words);
  return hipGetLastError();
}


// ---------------------------------------------------------------------------
// Host side: the plan.
// ---------------------------------------------------------------------------

struct StepPlan {
  int device;
  int nph;
  int grid;
  size_t lds;
  int32_t xin_bytes, perm_words;
  unsigned char* dev;  // one allocation: control words, phase table, tag buffers
  size_t dev_bytes;
  StepCtl* ctl;
  StepPhaseDev* table;
  uint32_t* tags;
  size_t tag_bytes;
};

namespace {

uint64_t up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

bool pow2_scale(float s) {
  if (!(s > 0.f) || s != s) return false;
  int e = 0;
  const float m = frexpf(s, &e);
  return m == 0.5f && e >= -23 && e <= 25;  // 2^-24 .. 2^24
}

}  // namespace

int step_plan_create(const StepPhaseSpec* ph, int nph, int device, StepPlan** out) {
  *out = nullptr;
  if (nph < 1 || nph > 4096) return fail(SPECTRA_E_INVAL, "phase count out of range [1, 4096]");
  const DeviceProps& props = device_props(device);
  const int grid = props.cu_count;
  std::vector<StepPhaseDev> table(nph);
  std::vector<int64_t> tag_off(nph, -1);  // word offset of each phase's tagged output
  uint64_t tag_words = 0;
  for (int p = 0; p < nph; ++p)
    if (ph[p].input >= 0) {
      const int q = ph[p].input;
      if (q >= p) return fail(SPECTRA_E_INVAL, "a phase's input must be an earlier phase");
      if (tag_off[q] < 0) {
        tag_off[q] = (int64_t)tag_words;
        tag_words += up((uint64_t)ph[q].t[0].v.N, 4);
      }
    }
  int64_t xin_bytes = 16, perm_words = 4, xs_halves = 8;
  for (int p = 0; p < nph; ++p) {
    const StepPhaseSpec& s = ph[p];
    if (s.ntasks < 1 || s.ntasks > kStepMaxTasks)
      return fail(SPECTRA_E_INVAL, "tasks per phase out of range [1, 4]");
    const int64_t K = s.t[0].v.K;
    int gmax = 0;
    int64_t total_rows = 0;
    for (int i = 0; i < s.ntasks; ++i) {
      const DeviceView& v = s.t[i].v;
      if (v.K != K) return fail(SPECTRA_E_INVAL, "the containers of a phase must share K");
      if (!s.t[i].y || (reinterpret_cast<uintptr_t>(s.t[i].y) & 1))
        return fail(SPECTRA_E_INVAL, "null or misaligned y");
      gmax = v.G > gmax ? v.G : gmax;
      total_rows += v.N;
    }
    if (K > 16384) return fail(SPECTRA_E_UNSUPPORTED, "decode step: K above 16384");
    if (s.input < 0) {
      if (!s.x || (reinterpret_cast<uintptr_t>(s.x) & 3)) return fail(SPECTRA_E_INVAL, "null or misaligned x");
    } else if (ph[s.input].t[0].v.N != K) {
      return fail(SPECTRA_E_INVAL, "a phase's K differs from the length of the output it reads");
    }
    if (!pow2_scale(s.x_scale)) return fail(SPECTRA_E_INVAL, "x_scale must be a power of two in [2^-24, 2^24]");
    int L = 0, P = 0;
    if (!gemv_variant(gmax, &L, &P) || P > 5)
      return fail(SPECTRA_E_UNSUPPORTED, "decode step: more than 5 groups per lane (G above 320)");
    const int lg = L == 64 ? 6 : (L == 32 ? 5 : 4);
    const int T = 448 / L;
    StepPhaseDev& d = table[p];
    memset(&d, 0, sizeof(d));
    d.x = s.input < 0 ? s.x : nullptr;
    d.x_scale = s.x_scale;
    d.ntasks = s.ntasks;
    d.lg = lg;
    d.P = P;
    // blocks in proportion to rows, at least one per task, never more than its rows
    int64_t nb[kStepMaxTasks], used = 0;
    for (int i = 0; i < s.ntasks; ++i) {
      int64_t b = (int64_t)grid * s.t[i].v.N / total_rows;
      if (b > s.t[i].v.N) b = s.t[i].v.N;
      if (b < 1) b = 1;
      nb[i] = b;
      used += b;
    }
    if (used > grid) return fail(SPECTRA_E_UNSUPPORTED, "decode step: more tasks in a phase than compute units");
    for (bool grew = true; used < grid && grew;) {
      grew = false;
      for (int i = 0; i < s.ntasks && used < grid; ++i)
        if (nb[i] < s.t[i].v.N) {
          ++nb[i];
          ++used;
          grew = true;
        }
    }
    int64_t first = 0;
    for (int i = 0; i < s.ntasks; ++i) {
      const DeviceView& v = s.t[i].v;
      if (v.n_out > 4 * L) return fail(SPECTRA_E_UNSUPPORTED, "decode step: more than 4 heavy-tailed channels per lane");
      StepTaskDev& t = d.t[i];
      t.codes = v.codes;
      t.scales = v.scales;
      t.zeros = v.zeros;
      t.outliers = v.outliers;
      t.perm = v.perm;
      t.y = s.t[i].y;
      t.ytag = nullptr;  // set once the tag buffers are allocated
      t.N = (int32_t)v.N;
      t.K = v.K;
      t.K_b = v.K_b;
      t.G = v.G;
      t.n_out = v.n_out;
      t.first_block = (int32_t)first;
      const int64_t rpb = (v.N + nb[i] - 1) / nb[i];
      t.rows_per_block = (int32_t)rpb;
      int64_t nt = (rpb + T - 1) / T;
      nt = nt < 2 ? 2 : (nt + 1) / 2 * 2;
      t.ntiles = (int32_t)nt;
      first += nb[i];
      const int64_t pw = 32 * (int64_t)v.G > 4 * ((K + 3) / 4) ? 32 * (int64_t)v.G : 4 * ((K + 3) / 4);
      perm_words = pw > perm_words ? pw : perm_words;
      const int64_t xh = up((uint64_t)(40 * v.G + v.n_out), 8);
      xs_halves = xh > xs_halves ? xh : xs_halves;
    }
    // staged input: fp16 in whole 16-byte chunks, or tagged words in whole chunks
    const int64_t xb = 2 * (int64_t)up((uint64_t)K, 8) > 4 * (int64_t)up((uint64_t)K, 4)
                           ? 2 * (int64_t)up((uint64_t)K, 8) : 4 * (int64_t)up((uint64_t)K, 4);
    xin_bytes = xb > xin_bytes ? xb : xin_bytes;
  }
  perm_words = (int64_t)up((uint64_t)perm_words, 4);
  const size_t lds = (size_t)xin_bytes + 4 * (size_t)perm_words + 2 * (size_t)xs_halves;
  const size_t lim = props.lds_per_block < (size_t)160 * 1024 ? props.lds_per_block : (size_t)160 * 1024;
  if (lds > lim) return fail(SPECTRA_E_UNSUPPORTED, "decode step: staging does not fit in LDS");
  hipError_t e;
  const void* fn = step_kernel();
  if (lds > 64 * 1024 &&
      (e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess)
    return fail(SPECTRA_E_HIP, std::string("decode step LDS attribute: ") + hipGetErrorString(e));
  int fit = 0;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&fit, fn, 512, lds)) != hipSuccess)
    return fail(SPECTRA_E_HIP, std::string("decode step occupancy: ") + hipGetErrorString(e));
  if (fit < 1) return fail(SPECTRA_E_UNSUPPORTED, "decode step: one block does not fit on a compute unit");

  StepPlan* pl = new (std::nothrow) StepPlan();
  if (!pl) return fail(SPECTRA_E_NOMEM, "host allocation of the step plan failed");
  pl->device = device;
  pl->nph = nph;
  pl->grid = grid;
  pl->lds = lds;
  pl->xin_bytes = (int32_t)xin_bytes;
  pl->perm_words = (int32_t)perm_words;
  const size_t ctl_bytes = up(sizeof(StepCtl), 256);
  const size_t table_bytes = up(sizeof(StepPhaseDev) * (size_t)nph, 256);
  pl->tag_bytes = up(4 * tag_words, 256);
  pl->dev_bytes = ctl_bytes + table_bytes + pl->tag_bytes;
  void* mem = nullptr;
  if ((e = dev_malloc(&mem, pl->dev_bytes)) != hipSuccess) {
    delete pl;
    return fail(SPECTRA_E_NOMEM, std::string("hipMalloc (step plan): ") + hipGetErrorString(e));
  }
  pl->dev = static_cast<unsigned char*>(mem);
  pl->ctl = reinterpret_cast<StepCtl*>(pl->dev);
  pl->table = reinterpret_cast<StepPhaseDev*>(pl->dev + ctl_bytes);
  pl->tags = reinterpret_cast<uint32_t*>(pl->dev + ctl_bytes + table_bytes);
  for (int p = 0; p < nph; ++p) {  // tag offsets become device addresses
    if (tag_off[p] >= 0) table[p].t[0].ytag = pl->tags + tag_off[p];
    if (ph[p].input >= 0) table[p].xtag = pl->tags + tag_off[ph[p].input];
  }
  if ((e = hipMemset(pl->dev, 0, pl->dev_bytes)) != hipSuccess ||
      (e = hipMemcpy(pl->table, table.data(), sizeof(StepPhaseDev) * (size_t)nph, hipMemcpyHostToDevice)) !=
          hipSuccess) {
    (void)hipFree(pl->dev);
    delete pl;
    return fail(SPECTRA_E_HIP, std::string("step plan upload: ") + hipGetErrorString(e));
  }
  *out = pl;
  return SPECTRA_OK;
}

hipError_t step_plan_run(StepPlan* p, hipStream_t s) {
  return launch_step(p->table, p->nph, p->ctl, p->xin_bytes, p->perm_words, p->lds, p->grid, s);
}

int step_plan_check(StepPlan* p, hipStream_t s) {
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(SPECTRA_E_HIP, std::string("decode step: ") + hipGetErrorString(e));
  uint32_t err = 0;
  if ((e = hipMemcpy(&err, &p->ctl->err, 4, hipMemcpyDeviceToHost)) != hipSuccess)
    return fail(SPECTRA_E_HIP, std::string("decode step status: ") + hipGetErrorString(e));
  if (!err) return 0;
  // start clean: launch count, tags and the error word back to zero
  const size_t ctl_bytes = up(sizeof(StepCtl), 256);
  if ((e = hipMemset(p->ctl, 0, ctl_bytes)) != hipSuccess ||
      (p->tag_bytes && (e = hipMemset(p->tags, 0, p->tag_bytes)) != hipSuccess) ||
      (e = hipDeviceSynchronize()) != hipSuccess)
    return fail(SPECTRA_E_HIP, std::string("decode step reset: ") + hipGetErrorString(e));
  return 1;
}

int step_plan_test_hooks(StepPlan* p, uint32_t poll_limit, uint32_t tag_skew) {
  const uint32_t w[2] = {poll_limit, tag_skew};
  const hipError_t e = hipMemcpy(&p->ctl->poll_limit, w, sizeof(w), hipMemcpyHostToDevice);
  if (e != hipSuccess) return fail(SPECTRA_E_HIP, std::string("decode step hooks: ") + hipGetErrorString(e));
  return SPECTRA_OK;
}

int step_plan_device(const StepPlan* p) { return p->device; }

void step_plan_free(StepPlan* p) {
  if (!p) return;
  (void)hipFree(p->dev);
  delete p;
}

}  // namespace spectra
