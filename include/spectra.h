/*
 * spectra.h -- C ABI of the SPECTRA sparse-precision dequant-GEMV library for
 * AMD Instinct MI355X (gfx950).
 *
 * What the library computes.  The SPECTRA page ("SPECTRA: Sparse-Precision
 * Exact Channel Tensor Reconstruction Architecture", abstract) describes a
 * weight codec: per input channel, a fourth-moment (kurtosis) test on the
 * weight column scaled by the upstream normalization gain sends heavy-tailed
 * channels to exact floating-point storage, and the Gaussian bulk to Group-32
 * 4-bit codes with per-group scales and bit-packed zero points; fused GPU
 * kernels then dequantize inside the matrix-vector product at decode batch
 * sizes (same page, highlight 4 on its fused kernels).
 * The page fixes neither formulas nor a memory layout.  Every choice below that
 * it leaves open is stated where it is made, as this library's reading.
 *
 * Shapes: W is [N][K] (an nn.Linear weight: N outputs, K inputs, K contiguous),
 * gamma is [K], x is [M][K], y is [M][N], all fp16 (IEEE binary16 bit patterns).
 * y = x W^T with W replaced by its SPECTRA reconstruction.
 *
 * ---------------------------------------------------------------------------
 * Quantization (what spectra_pack computes; all arithmetic in IEEE binary64
 * unless stated; rint = round half to even; fp16() = round to nearest even)
 * ---------------------------------------------------------------------------
 *  1. Saliency and split.  For each input channel k: s[n] = W[n][k]*gamma[k]
 *     (exact in binary64).  mean = sum_n s[n] / N; m2 = sum_n (s[n]-mean)^2 / N;
 *     m4 = sum_n ((s[n]-mean)^2)^2 / N.  Channel k is heavy-tailed iff m2 > 0
 *     and m4/(m2*m2) - 3 > 3.0 (excess kurtosis with population moments; the
 *     page names only a fourth-moment test with threshold 3.0 -- this library
 *     reads it as excess kurtosis, under which Gaussian columns are
 *     essentially never flagged).
 *     A constant column (N = 1, gamma[k] = 0, ...) has m2 = 0 and is bulk.
 *     The device evaluates the sums in a fixed tree order, so a channel whose
 *     kurtosis lies within a few ulp of the threshold may be classified
 *     differently from a sequential evaluation.
 *  2. Order.  perm[0..K_b) lists the bulk channels ascending, perm[K_b..K) the
 *     heavy-tailed channels ascending; n_out = K - K_b; G = ceil(K_b / 32).
 *     Bulk position j of row n holds W[n][perm[j]]; group g = positions
 *     [32g, 32g+32); positions >= K_b are padding.
 *  3. Per group (n, g), over its real members w (padding excluded):
 *       lo = min(0, min w), hi = max(0, max w), s = (hi - lo) / 15,
 *       s16 = fp16(s).
 *     If s16 == 0: z = 0 and every code is 0.  Otherwise
 *       z = min(15, rint(-lo / s16)),  q = min(15, max(0, rint(w / s16) + z)).
 *     Padding members get q = z.
 *  4. Reconstruction: w_hat = (q - z) * s16 (exact in binary32 and binary64).
 *     Heavy-tailed channels are not quantized: O[n][j] = W[n][perm[K_b+j]]
 *     bit for bit (no gain applied, no rounding).
 *  5. Product (spectra_gemm): y[m][n] = sum_{j<K_b} x[m][perm[j]] * w_hat[n][j]
 *     + sum_{j<n_out} x[m][perm[K_b+j]] * O[n][j], accumulated in binary32 and
 *     rounded to fp16.  The accuracy contract is, per element,
 *     |y - y_exact| <= 1e-3 * sum_k |W_hat[n][k]| * |x[m][k]| + 1e-6.
 *
 * ---------------------------------------------------------------------------
 * Container image (little-endian).  This is both the device-resident layout
 * and the byte stream spectra_export returns.
 * ---------------------------------------------------------------------------
 *  Header, 128 bytes:
 *    [0,4)    magic   u32 = 0x31435053 (bytes 'S' 'P' 'C' '1')
 *    [4,8)    version u32 = 1
 *    [8,16)   K       i64     [16,24)  N     i64     [24,32)  K_b   i64
 *    [32,40)  G       i64     [40,48)  n_out i64
 *    [48,56)  off_mask     u64    [56,64)  off_perm     u64
 *    [64,72)  off_codes    u64    [72,80)  off_scales   u64
 *    [80,88)  off_zeros    u64    [88,96)  off_outliers u64
 *    [96,104) total_bytes  u64    [104,128) zero
 *  Sections follow in the order below.  Each starts at the smallest multiple
 *  of 256 that is not below the end of the previous one (the header ends at
 *  128); total_bytes is the end of the last section rounded up to a multiple
 *  of 256.  Every padding byte is zero.  An empty section has size 0.
 *    mask     ceil(K/32) x u32.  Bit (k mod 32) of word floor(k/32) is 1 iff
 *             channel k is heavy-tailed.
 *    perm     K x i32, as in step 2.
 *    codes    N*G records of 16 bytes; the record of group (n, g) starts at
 *             byte 16*(n*G + g) and is four u32 words.  Member e (0..31) of the
 *             group is the 4-bit field of word floor(e/8) starting at bit
 *             16*(e mod 2) + 4*floor((e mod 8)/2).  (So (word >> 4i) & 0x000F000F
 *             holds members 8d+2i and 8d+2i+1 in its two 16-bit halves.)
 *    scales   N*G x fp16: s16 of group (n, g) at index n*G + g.
 *    zeros    ceil(N*G/2) bytes: z of flat group index i = n*G + g is in byte
 *             floor(i/2), bits [4*(i mod 2), 4*(i mod 2) + 4).
 *    outliers N x n_out fp16, row-major: O[n][j] at index n*n_out + j.
 *  Payload bytes (codes + scales + zeros + outliers, unpadded) are
 *  16*N*G + 2*N*G + ceil(N*G/2) + 2*N*n_out: 4 + 16/32 + 4/32 bits per bulk
 *  weight (K_b rounded up to 32G) plus 16 bits per heavy-tailed weight.
 *
 * ---------------------------------------------------------------------------
 * Conventions
 * ---------------------------------------------------------------------------
 *  - Functions returning int return SPECTRA_OK or a negative spectra_status.
 *    No exception or abort crosses the ABI.  spectra_last_error() returns a
 *    thread-local message describing the latest failure on the calling thread.
 *  - Handles (spectra_container*, spectra_kv*, spectra_step*) are opaque
 *    identifiers, never reissued: a freed handle stays invalid for the life of
 *    the process, and every call checks its handle before using it.
 *  - A container owns one device allocation on the device that was current
 *    when it was packed; it is immutable after packing and may be used by
 *    concurrent spectra_gemm* calls on any streams of that device.
 *  - x and y are caller-owned device buffers; the library never retains them.
 *  - gemm calls are asynchronous: launch errors are returned, device faults
 *    surface at the caller's next synchronization.
 */
#ifndef SPECTRA_H
#define SPECTRA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct spectra_container spectra_container;

typedef enum {
  SPECTRA_OK = 0,
  SPECTRA_E_INVAL = -1,        /* bad argument: null pointer, size out of range, misalignment, freed container */
  SPECTRA_E_NONFINITE = -2,    /* W or gamma holds an infinity or a NaN */
  SPECTRA_E_NOMEM = -3,        /* a device or host allocation failed */
  SPECTRA_E_HIP = -4,          /* a HIP runtime call failed (message has the HIP error string) */
  SPECTRA_E_UNSUPPORTED = -5,  /* the forced kernel cannot run this shape */
  SPECTRA_E_IO = -6,           /* a file could not be opened, read or written */
  SPECTRA_E_TIMEOUT = -7       /* a bounded wait inside a decode step gave up (its outputs are invalid) */
} spectra_status;

/* Kernel selection for spectra_gemm_ex. */
typedef enum {
  SPECTRA_KERNEL_AUTO = 0,        /* GEMV for M <= 2 (M <= 4 where no MFMA kernel but the strip
                                     kernel takes the shape) if it supports the shape, else as
                                     SPECTRA_KERNEL_MFMA */
  SPECTRA_KERNEL_GEMV = 1,        /* VALU dequant-GEMV, x in LDS, fp32 accumulate; M <= 4, and
                                     K % 8 == 0 when M > 1 (else SPECTRA_E_UNSUPPORTED) */
  SPECTRA_KERNEL_MFMA = 2,        /* the split-K kernel below where it takes the shape, else the
                                     tiled kernel where it does, else the strip kernel */
  SPECTRA_KERNEL_MFMA_TILED = 3,  /* 16-row tiles with K split over 8 waves: M <= 16, the M rows of
                                     x in LDS */
  SPECTRA_KERNEL_MFMA_STRIP = 4,  /* one 16-row strip per wave for the whole K loop: any shape the
                                     MFMA path takes */
  SPECTRA_KERNEL_MFMA_SPLITK = 5  /* K split in ranges over blocks, x of a range held in registers,
                                     fp32 partial sums in the workspace: M <= 16, at most 256
                                     heavy-tailed columns */
} spectra_kernel;

typedef struct {
  int64_t K, N, K_b, G, n_out;
  uint64_t bytes_codes;        /* 16*N*G */
  uint64_t bytes_scales;       /* 2*N*G */
  uint64_t bytes_zeros;        /* ceil(N*G/2) */
  uint64_t bytes_outliers;     /* 2*N*n_out */
  uint64_t bytes_payload;      /* sum of the four above */
  uint64_t bytes_meta;         /* 128 + 4*ceil(K/32) + 4*K (header, mask, perm; unpadded) */
  uint64_t bytes_total;        /* whole image including alignment padding (= total_bytes) */
} spectra_info_t;

/* Limits on the shapes spectra_pack accepts. */
#define SPECTRA_MAX_K ((int64_t)1 << 24)
#define SPECTRA_MAX_N ((int64_t)1 << 31)
#define SPECTRA_MAX_M ((int64_t)1 << 20)
#define SPECTRA_MAX_T ((int64_t)1 << 31)

/* Pack W (HOST memory, [N][K] fp16 bits, row-major) with gain gamma (HOST
 * memory, [K] fp16 bits) into a new device-resident container on the current
 * device.  The inputs are borrowed for the duration of the call only.
 * Synchronous: the container is complete when the call returns.
 * Requires 1 <= K <= SPECTRA_MAX_K and 1 <= N <= SPECTRA_MAX_N.
 * Returns NULL on error (E_INVAL, E_NONFINITE, E_NOMEM, E_HIP; see
 * spectra_last_error).  The split, quantization and layout are the steps and
 * the image described at the top of this file. */
spectra_container* spectra_pack(const uint16_t* W, const uint16_t* gamma, int64_t K, int64_t N);

/* As spectra_pack, but W and gamma are DEVICE pointers (current device) and the
 * packing kernels run on `stream` (a hipStream_t; NULL = null stream).  The
 * call still returns only once the container is complete. */
spectra_container* spectra_pack_device(const void* W, const void* gamma, int64_t K, int64_t N,
                                       void* stream);

/* y = x W_hat^T.  x: DEVICE fp16 [M][K] contiguous, y: DEVICE fp16 [M][N]
 * contiguous, overwritten; both 4-byte aligned, on the container's device.
 * 1 <= M <= SPECTRA_MAX_M.  Enqueued on the null stream; returns at once. */
int spectra_gemm(const spectra_container* c, const void* x, void* y, int64_t M);

/* As spectra_gemm, enqueued on `stream` (a hipStream_t; NULL = null stream),
 * with the kernel chosen by `kernel` (a spectra_kernel).  A forced kernel that
 * cannot run the shape returns SPECTRA_E_UNSUPPORTED and enqueues nothing. */
int spectra_gemm_ex(const spectra_container* c, const void* x, void* y, int64_t M,
                    void* stream, int kernel);

/* spectra_gemm_ex for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same product and kernels, bit for bit, but the MFMA path's workspace
 * (x permuted to bulk order, M * (32 G + n_out rounded up to 32) * 2 bytes,
 * plus for the split-K kernel 4 * M * N bytes of partial sums per K-range)
 * is a static 8 MiB device array of the library instead of the per-stream
 * workspace, and the call makes no device allocation at all.  Where the
 * split-K kernel's workspace exceeds 8 MiB and that kernel was not forced,
 * the MFMA kernel it replaces runs instead (same bound, not bit-equal to
 * spectra_gemm_ex).  The container's device must be the current device
 * (E_INVAL otherwise); a product whose workspace still exceeds 8 MiB
 * returns SPECTRA_E_UNSUPPORTED and enqueues nothing.  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (other streams,
 * other threads) race and must be serialized by the caller. */
int spectra_gemm_noalloc(const spectra_container* c, const void* x, void* y, int64_t M,
                         void* stream, int kernel);

/* Which kernel spectra_gemm_ex would run for M rows of x and the selector
 * `kernel` (a spectra_kernel), without any device work: the product is the
 * fused dequantize-and-multiply of spectra_gemm (SPECTRA page, abstract and
 * highlight 4); this only reports how it would be launched.  Returns
 * SPECTRA_PLAN_GEMV, SPECTRA_PLAN_MFMA_TILED, SPECTRA_PLAN_MFMA or
 * SPECTRA_PLAN_MFMA_SPLITK; or, as
 * spectra_gemm_ex would, SPECTRA_E_INVAL (invalid container, M out of range,
 * unknown selector) or SPECTRA_E_UNSUPPORTED (a forced kernel that cannot run
 * the shape). */
enum {
  SPECTRA_PLAN_GEMV = 1,        /* k_gemv_m1: VALU dequant-GEMV */
  SPECTRA_PLAN_MFMA_TILED = 2,  /* k_xbulk + k_mfma_ks: 16-row tiles, K split over 8 waves */
  SPECTRA_PLAN_MFMA = 3,        /* k_xbulk + k_mfma: one 16-row strip per wave */
  SPECTRA_PLAN_MFMA_SPLITK = 4  /* k_xbulk + k_mfma_sk + k_sk_sum: K split in ranges, fp32 partials */
};
int spectra_gemm_plan(const spectra_container* c, int64_t M, int kernel);

/* Several containers that share K and the same input x (e.g. the q/k/v or the
 * gate/up projections of one decoder layer) in one launch: ys[i] = x W_i^T.
 * cs and ys are HOST arrays of `count` entries (1 <= count <= 64); every ys[i]
 * is a DEVICE fp16 [M][N_i] buffer.  Runs on `stream`; returns at once.  Same
 * result, element for element, as `count` spectra_gemm_ex calls with the
 * GEMV kernel; M must be 1. */
int spectra_gemm_grouped(const spectra_container* const* cs, int count, const void* x,
                         void* const* ys, int64_t M, void* stream);

/* Fused embedding gather (SPECTRA page, abstract and highlight 5: a
 * vocabulary table kept in the Group-32 4-bit format, its rows dequantized
 * as a forward pass gathers them).  The container holds the table E [V][D]
 * packed as W with N = V rows and K = D channels.  For i < T:
 *   out[i][k] = fp16(W_hat[ids[i]][k])  in channel order k < K,
 * where W_hat's bulk entries are (q - z) * s16 (exact in fp32, rounded once
 * to nearest even) and its heavy-tailed channels the stored fp16 bits; the
 * result is bit-identical to dequantizing the row and rounding it to fp16.
 * ids: DEVICE int32 [T]; out: DEVICE fp16 [T][K] contiguous, overwritten;
 * both 4-byte aligned, on the container's device (16-byte aligned out with
 * K % 8 == 0 takes whole-chunk stores).  An id outside [0, N) yields a row
 * of zeros; nothing is read or written out of bounds.  0 <= T <= SPECTRA_MAX_T
 * (T = 0 enqueues nothing).  Enqueued on `stream` (NULL = null stream);
 * returns at once.  E_INVAL on bad arguments, E_UNSUPPORTED when one row
 * does not fit the kernel's LDS row buffer (K above about 50000). */
int spectra_embed(const spectra_container* c, const void* ids, int64_t T, void* out, void* stream);

/* ---------------------------------------------------------------------------
 * Decode step: a chain of dependent M = 1 products in one launch.
 *
 * At decode every token streams all weights once and the projections of a
 * layer depend on one another (SPECTRA page, abstract: its fused kernels run
 * under graph replay to cut per-launch overhead; techfi24 summary, section on
 * the hardware context: decode is bound by weight bytes).  A step is a list
 * of phases; phase p computes y_i = x_p W_hat_i^T (as spectra_gemm with
 * M = 1, bit for bit the GEMV's result) for its 1 .. 4 containers, which share
 * K.  Its input x_p is either an external DEVICE fp16 [K] vector or the output
 * of task 0 of an earlier phase q (then K must equal that container's N), and
 * it is staged as fp16(x * x_scale) with x_scale a power of two in
 * [2^-24, 2^24] (exact; 1 leaves x unchanged).  One launch runs every phase
 * in order with one persistent block per compute unit: a phase starts its
 * arithmetic once the output it reads is complete, while the blocks already
 * stream its weights.
 *
 * Ownership: the plan borrows the containers and the x and y buffers, which
 * must stay valid until spectra_step_free; it owns a small device allocation
 * (control words, phase table and a 4-byte tagged copy of each output that a
 * later phase reads).  Runs of one plan must not overlap (one stream, or
 * ordered streams); plans are independent of one another.  Each wait inside
 * the kernel is bounded: a wait that gives up marks the plan and the kernel
 * still completes; spectra_step_status reports it.
 * Limits: K <= 16384, at most 320 groups per row (G), at most 4 heavy-tailed
 * channels per lane of the GEMV mapping (n_out <= 64 for G <= 80, 128 for
 * G <= 160, 256 otherwise), and the staging of the largest phase within the
 * LDS of one block (E_UNSUPPORTED otherwise).
 * ------------------------------------------------------------------------- */
typedef struct spectra_step spectra_step;

#define SPECTRA_STEP_MAX_TASKS 4

typedef struct {
  int32_t ntasks;                                   /* 1 .. SPECTRA_STEP_MAX_TASKS */
  const spectra_container* c[SPECTRA_STEP_MAX_TASKS];
  void* y[SPECTRA_STEP_MAX_TASKS];                  /* DEVICE fp16 [N_i] outputs, 2-byte aligned */
  int32_t input;                                    /* -1: x below; else an earlier phase index */
  const void* x;                                    /* DEVICE fp16 [K], 4-byte aligned, when input == -1 */
  float x_scale;                                    /* power of two applied to the staged input */
} spectra_step_phase;

/* Validates the phases and builds the plan on the containers' device.  NULL
 * on error (E_INVAL, E_UNSUPPORTED, E_NOMEM, E_HIP; see spectra_last_error). */
spectra_step* spectra_step_create(const spectra_step_phase* phases, int32_t nphases);

/* Enqueues one run of every phase on `stream` (NULL = null stream); returns
 * at once.  May be captured into a HIP graph and replayed. */
int spectra_step_run(spectra_step* st, void* stream);

/* Waits for `stream`, then reports whether a wait of an earlier run gave up:
 * SPECTRA_OK, or SPECTRA_E_TIMEOUT (the plan's control state is then reset,
 * so the next run starts clean). */
int spectra_step_status(spectra_step* st, void* stream);

/* Testing the bounded waits: poll_limit (0 = built-in) caps each wait's
 * polls, and tag_skew != 0 makes every wait expect a mark no producer
 * writes, so each wait gives up after poll_limit polls.  Synchronous. */
int spectra_step_test_hooks(spectra_step* st, uint32_t poll_limit, uint32_t tag_skew);

/* Releases the plan's device memory.  NULL-safe; unknown handles are ignored. */
void spectra_step_free(spectra_step* st);

/* ---------------------------------------------------------------------------
 * Testing the error paths: of the device and pinned-host allocations the
 * library makes from now on (containers, staging, workspaces, KV caches,
 * step plans, file staging), the next `skip` succeed and the `count` after
 * them fail as out of memory, so the calling entry point returns
 * SPECTRA_E_NOMEM (NULL for handle returns) and releases what it had
 * allocated.  For callers' tests of their error handling; (0, 0) turns it
 * off.  Process-wide, thread-safe.  E_INVAL for negative arguments.
 * ------------------------------------------------------------------------- */
int spectra_test_fail_allocations(int64_t skip, int64_t count);

/* ---------------------------------------------------------------------------
 * Group-32 4-bit KV cache (SPECTRA page, abstract: the key-value cache is kept
 * in microscaled Group-32 4-bit form).  One cache holds the keys and values of
 * one attention layer for up to `capacity` tokens, `heads` cache heads of
 * `head_dim` channels (64, 128 or 256).  Each head vector is quantized on
 * append exactly as a bulk weight group per 32 consecutive channels (range
 * [min(0, min), max(0, max)], s16 = fp16(range / 15), z = rint(-lo / s16),
 * q = clamp(rint(w / s16) + z, 0, 15), in binary64), with no heavy-tailed
 * split.  The handle is opaque, owns its device memory (on the device current
 * at creation) and tracks its length on the host.
 * ------------------------------------------------------------------------- */
typedef struct spectra_kv spectra_kv;

/* NULL on error (E_INVAL for shapes, E_NOMEM). */
spectra_kv* spectra_kv_create(int64_t capacity, int32_t heads, int32_t head_dim);

/* Quantize T new tokens and store them at positions [length, length + T).
 * k, v: DEVICE fp16 [T][heads][head_dim], 16-byte aligned, finite values (a
 * non-finite value leaves its group unspecified, never out of bounds).
 * E_INVAL if length + T would exceed the capacity.  Enqueued on `stream`;
 * the length grows at once on the host. */
int spectra_kv_append(spectra_kv* kv, const void* k, const void* v, int64_t T, void* stream);

/* Decode-step attention over the `length` cached tokens:
 *   out[h] = softmax(q[h] K_hat^T / sqrt(head_dim)) V_hat,  h < q_heads,
 * query head h reading cache head h / (q_heads / heads); K_hat, V_hat are the
 * dequantized cache ((q - z) * s16).  q: DEVICE fp16 [q_heads][head_dim];
 * out: DEVICE fp16 [q_heads][head_dim]; both 4-byte aligned.  q_heads must be
 * a multiple of heads with 1 .. 16 query heads per cache head (any ratio);
 * length >= 1 (E_INVAL otherwise) and at most 524288 (E_UNSUPPORTED).
 * Per element, |out - ref| <= 1e-3 * (sum_t p_t |V_hat[t]|) + 1e-6 with ref
 * and p in binary64.  Uses the per-stream workspace (4 * q_heads *
 * (head_dim + 2) * ceil(length / 128) bytes); enqueued on `stream`. */
int spectra_kv_attend(const spectra_kv* kv, const void* q, int32_t q_heads, void* out, void* stream);

/* Tokens currently cached (-1 for an invalid handle). */
int64_t spectra_kv_length(const spectra_kv* kv);

/* Forget every cached token (length 0); the memory is kept. */
int spectra_kv_reset(spectra_kv* kv);

/* Copy the first `length` tokens' quantized data to HOST memory, for
 * bit-exact checks: K records, K scales, K zero bytes, then the same for V,
 * each section [length][heads][G] in the device order (zeros [length][heads]
 * [G/2]); 2 * length * heads * G * (16 + 2 + 1/2) bytes.  Synchronous. */
int spectra_kv_export(const spectra_kv* kv, void* host_dst, uint64_t cap);

/* Release the cache.  NULL-safe; unknown or freed handles are ignored. */
void spectra_kv_free(spectra_kv* kv);

/* Release the container and its device memory.  NULL-safe; freeing a handle
 * twice, or one this library did not return, does nothing.  Any later call
 * with a freed handle returns SPECTRA_E_INVAL (handles are never reissued). */
void spectra_free(spectra_container* c);

/* Shape and byte counts of a container. */
int spectra_info(const spectra_container* c, spectra_info_t* out);

/* Copy the container image (header + sections, total_bytes) to HOST memory
 * host_dst of capacity cap bytes.  E_INVAL if cap < total_bytes.  Synchronous. */
int spectra_export(const spectra_container* c, void* host_dst, uint64_t cap);

/* ---------------------------------------------------------------------------
 * Container files.  The SPECTRA page (abstract) serializes every weight,
 * scale and offset into one self-contained binary container that is streamed
 * straight into GPU memory so that initialization has a bounded memory spike.
 * Here the file is the container image itself (layout above, total_bytes
 * long), and loading streams it through a fixed-size staging buffer: peak
 * host memory is 2 * chunk_bytes of pinned staging plus the mask and perm
 * sections (about 4.1 * K bytes), whatever the payload's size.
 * chunk_bytes = 0 selects 8 MiB; other values are rounded up to a multiple
 * of 256 and to at least 4096.
 * ------------------------------------------------------------------------- */

/* Check a container image held in HOST memory without touching any device:
 * magic and version, K, N, K_b = K - n_out, G = ceil(K_b / 32), section
 * offsets equal to the layout above, bytes == total_bytes, mask bits past K
 * zero and n_out of them set, perm = the bulk channels ascending then the
 * heavy-tailed ones ascending, every scale a finite fp16 >= 0, every
 * heavy-tailed weight finite, the unused zero nibble 0.  SPECTRA_OK or
 * SPECTRA_E_INVAL with the first violation in spectra_last_error(). */
int spectra_validate_image(const void* image, uint64_t bytes);

/* A new container on the current device from a HOST image (validated as
 * above, then copied).  Synchronous; NULL on error (spectra_last_error). */
spectra_container* spectra_import(const void* image, uint64_t bytes);

/* Write the container's image to `path` (created or truncated), copying it
 * out through the staging buffer chunk by chunk.  Synchronous.  E_IO on any
 * file error (a partial file is removed), E_HIP on a copy error. */
int spectra_save(const spectra_container* c, const char* path, uint64_t chunk_bytes);

/* Read a container file into a new container on the current device: the
 * header is checked first, then the file is streamed in chunks (the next
 * chunk is read from the file while the previous one is copied to the
 * device) and each chunk is validated as it passes; the mask and perm are
 * checked once complete.  Synchronous; NULL on error (E_IO, E_INVAL for a
 * malformed image, E_NOMEM, E_HIP; see spectra_last_error). */
spectra_container* spectra_load(const char* path, uint64_t chunk_bytes);

/* Device workspaces.  The MFMA path and KV attention use a device workspace
 * per (device, stream), allocated on first use and grown (to at least twice
 * its size) when a call needs more.  A grown-out buffer is kept, not freed: a
 * HIP graph captured earlier on that stream may still hold its address.  The
 * first call at a new largest size allocates, so make it before a capture.
 * spectra_release_workspaces synchronizes each device that holds one and
 * frees every grown-out buffer; call it only when no graph captured before a
 * growth will be replayed again.  SPECTRA_OK or SPECTRA_E_HIP. */
int spectra_release_workspaces(void);

/* Thread-local description of the latest error on the calling thread ("" if none). */
const char* spectra_last_error(void);

/* Status code (a negative spectra_status) of that latest error, SPECTRA_OK if
 * none: how a caller classifies the failure of an entry point that returns a
 * NULL handle (spectra_pack, spectra_import, spectra_load, ...). */
int spectra_last_status(void);

/* ABI version (1). */
int spectra_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPECTRA_H */
