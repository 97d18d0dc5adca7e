// Internal declarations shared by the host ABI and the gfx950 kernels of
// libspectra.  Not part of the public interface (include/spectra.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

namespace spectra {

constexpr uint32_t kMagic = 0x31435053u;          // 'S' 'P' 'C' '1'
constexpr uint32_t kVersion = 1;
constexpr uint64_t kHeaderBytes = 128;
constexpr uint64_t kAlign = 256;
constexpr int kGroup = 32;
constexpr uint64_t kLiveTag = 0x5350454354524131ull;  // host handle tag while alive
constexpr uint64_t kDeadTag = 0xDEADDEADDEADDEADull;  // written by spectra_free

// Offsets of the six sections inside the container image.
struct Layout {
  uint64_t mask, perm, codes, scales, zeros, outliers, total;
};

__host__ __device__ inline uint64_t align_up(uint64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

__host__ __device__ inline Layout make_layout(int64_t K, int64_t N, int64_t n_out) {
  const int64_t K_b = K - n_out;
  const int64_t G = (K_b + kGroup - 1) / kGroup;
  const uint64_t NG = (uint64_t)N * (uint64_t)G;
  Layout L;
  uint64_t pos = kHeaderBytes;
  pos = align_up(pos); L.mask = pos; pos += 4ull * (uint64_t)((K + 31) / 32);
  pos = align_up(pos); L.perm = pos; pos += 4ull * (uint64_t)K;
  pos = align_up(pos); L.codes = pos; pos += 16ull * NG;
  pos = align_up(pos); L.scales = pos; pos += 2ull * NG;
  pos = align_up(pos); L.zeros = pos; pos += (NG + 1) / 2;
  pos = align_up(pos); L.outliers = pos; pos += 2ull * (uint64_t)N * (uint64_t)n_out;
  L.total = align_up(pos);
  return L;
}

// Device-side view of one container, passed by value to kernels.
struct DeviceView {
  const uint4* codes;        // [N*G] 16-byte records
  const uint16_t* scales;    // [N*G] fp16 bits
  const uint8_t* zeros;      // [ceil(N*G/2)] nibbles
  const uint16_t* outliers;  // [N][n_out] fp16 bits
  const int32_t* perm;       // [K]
  const uint32_t* mask;      // [ceil(K/32)] heavy-tailed channel bits
  int64_t N;
  int32_t K, K_b, G, n_out;
  int32_t cu_count;          // compute units of the container's device (launch sizing)
  int32_t lds_per_block;     // LDS bytes one block may use on that device
};

// Per-device properties the launchers need.
struct DeviceProps {
  int cu_count;
  size_t lds_per_block;
};
const DeviceProps& device_props(int device);

}  // namespace spectra

struct spectra_container {
  uint64_t tag;
  int device;
  int64_t K, N, K_b, G, n_out;
  spectra::Layout lay;
  unsigned char* dev;  // one device allocation holding the whole image
  spectra::DeviceView view() const {
    spectra::DeviceView v;
    v.codes = reinterpret_cast<const uint4*>(dev + lay.codes);
    v.scales = reinterpret_cast<const uint16_t*>(dev + lay.scales);
    v.zeros = reinterpret_cast<const uint8_t*>(dev + lay.zeros);
    v.outliers = reinterpret_cast<const uint16_t*>(dev + lay.outliers);
    v.perm = reinterpret_cast<const int32_t*>(dev + lay.perm);
    v.mask = reinterpret_cast<const uint32_t*>(dev + lay.mask);
    v.N = N;
    v.K = (int32_t)K;
    v.K_b = (int32_t)K_b;
    v.G = (int32_t)G;
    v.n_out = (int32_t)n_out;
    v.cu_count = spectra::device_props(device).cu_count;
    v.lds_per_block = (int32_t)spectra::device_props(device).lds_per_block;
    return v;
  }
};

namespace spectra {

// Records the latest failure of the calling thread (status SPECTRA_OK for "").
void set_error(const std::string& msg, int status);
int fail(int status, const std::string& msg);

// ---- container images on the host (image.cpp) ----
// Shape limits of a container (status; message set on failure).
int check_shape(int64_t K, int64_t N);
struct ImageFields {
  int64_t K, N, K_b, G, n_out;
  Layout lay;
};
// Header checks: fields, shape limits, offsets equal to the layout, total.
int parse_header(const unsigned char* h, uint64_t bytes, ImageFields& f);
// Checks on the bytes [pos, pos + len) of the image (any split into ranges at
// even positions): scales finite and >= 0, heavy-tailed weights finite, the
// zero nibble past N*G zero.
int check_range(const ImageFields& f, uint64_t pos, const unsigned char* p, uint64_t len);
// mask: n_out bits set, none past K; perm: the canonical channel order.
int check_meta(const ImageFields& f, const uint32_t* mask, const int32_t* perm);
// All of the above on a whole host image.
int validate_host_image(const unsigned char* img, uint64_t bytes, ImageFields& f);

// ---- packer (pack.hip) ----
// Scratch needed by the kurtosis passes for a K x N matrix, in bytes.
uint64_t kurtosis_scratch_bytes(int64_t K, int64_t N);
// Runs the split passes; writes ceil(K/32) mask words and one status word
// (bit 0: non-finite input seen) into `status_out` (device, (1 + ceil(K/32)) u32).
hipError_t launch_kurtosis(const uint16_t* W, const uint16_t* gamma, int64_t K, int64_t N,
                           void* scratch, uint32_t* status_out, hipStream_t s);
// Fills perm, codes, scales, zeros and outliers of a container whose header and
// mask are already in place.
hipError_t launch_quantize(const uint16_t* W, const spectra_container* c, hipStream_t s);

// ---- product kernels (gemv.hip, mfma.hip) ----
// Return hipErrorNotSupported (without launching) when the kernel cannot run the shape.
bool gemv_supports(const DeviceView& v, int64_t M);
hipError_t launch_gemv(const DeviceView& v, const uint16_t* x, uint16_t* y, int64_t M, hipStream_t s);
hipError_t launch_gemv_grouped(const DeviceView* vs, int count, const uint16_t* x,
                               uint16_t* const* ys, hipStream_t s);
bool mfma_supports(const DeviceView& v, int64_t M);
// The MFMA path runs the shape on its 16-row tiled kernel (k_mfma_ks).
bool mfma_tiled_supports(const DeviceView& v, int64_t M);
// The MFMA path runs the shape on its split-K kernel (k_mfma_sk + k_sk_sum).
bool mfma_splitk_supports(const DeviceView& v, int64_t M);
// Device workspace the MFMA path needs for M input rows: x permuted to bulk
// order, and for the split-K kernel the fp32 partial sums of every K-range.
size_t mfma_workspace_bytes(const DeviceView& v, int64_t M);
size_t mfma_splitk_workspace_bytes(const DeviceView& v, int64_t M);
// plan: SPECTRA_PLAN_MFMA_SPLITK (the workspace holds
// mfma_splitk_workspace_bytes), SPECTRA_PLAN_MFMA_TILED or SPECTRA_PLAN_MFMA,
// each on a shape its supports test accepts.
hipError_t launch_mfma_ws(const DeviceView& v, const uint16_t* x, uint16_t* y, int64_t M,
                          void* workspace, hipStream_t s, int plan);

// ---- row gather (embed.hip) ----
bool embed_supports(const DeviceView& v);
hipError_t launch_embed(const DeviceView& v, const int32_t* ids, int64_t T, uint16_t* out,
                        hipStream_t s);

// ---- Group-32 4-bit KV cache (kv.hip) ----
struct KvPlane {
  uint4* codes;     // [cap][H][G] 16-byte records
  uint16_t* scales; // [cap][H][G] fp16 bits
  uint8_t* zeros;   // [cap][H][G/2] nibbles
};
struct KvView {
  KvPlane k, v;
  int64_t cap;
  int32_t H, D, G;
};
bool kv_shape_supported(int64_t heads, int64_t head_dim);
int kv_max_rep();
int64_t kv_max_attend_length();  // cached tokens one attention call handles
size_t kv_attend_workspace_bytes(const KvView& c, int rep, int64_t L);
hipError_t launch_kv_append(const KvView& c, const uint16_t* k, const uint16_t* v, int64_t T, int64_t pos0,
                            hipStream_t s);
hipError_t launch_kv_attend(const KvView& c, const uint16_t* q, int rep, int64_t L, uint16_t* out, void* ws,
                            hipStream_t s);

// ---- persistent decode step (step.hip) ----
constexpr int kStepMaxTasks = 4;
// One container of a phase, as the kernel reads it (device table).
struct StepTaskDev {
  const uint4* codes;
  const uint16_t* scales;
  const uint8_t* zeros;
  const uint16_t* outliers;
  const int32_t* perm;
  uint16_t* y;        // plain fp16 output [N]
  uint32_t* ytag;     // tagged copy (tag << 16 | fp16) when a later phase reads it, else null
  int32_t N, K, K_b, G, n_out;
  int32_t first_block, rows_per_block, ntiles;
};
struct StepPhaseDev {
  const uint16_t* x;     // external input [K], or null
  const uint32_t* xtag;  // tagged input (an earlier phase's output), or null
  float x_scale;         // power of two applied to x as it is staged
  int32_t ntasks;
  int32_t lg, P;         // log2 of lanes per row, group slots per lane
  int32_t pad[2];
  StepTaskDev t[kStepMaxTasks];
};
// Control words of one plan (device memory, zeroed at creation and after an error).
struct StepCtl {
  uint32_t seq;          // launches completed (the tag of a launch is 1 + seq % 65535)
  uint32_t pad0[63];
  uint32_t done;         // blocks finished, cumulative over launches
  uint32_t pad1[63];
  uint32_t err;          // bit 0: a wait gave up
  uint32_t poll_limit;   // 0: the built-in limit; testing hook
  uint32_t tag_skew;     // added to the tag consumers expect; testing hook (0 in use)
  uint32_t pad2[61];
};
struct StepTaskSpec {
  DeviceView v;
  uint16_t* y;
};
struct StepPhaseSpec {
  int ntasks;
  StepTaskSpec t[kStepMaxTasks];
  int input;             // -1: external x; else an earlier phase whose task 0 output is the input
  const uint16_t* x;
  float x_scale;
};
struct StepPlan;
// Builds the plan (device table, control words, tag buffers); status < 0 with
// the error set on failure.
int step_plan_create(const StepPhaseSpec* ph, int nph, int device, StepPlan** out);
hipError_t step_plan_run(StepPlan* p, hipStream_t s);
// Waits for s, reads the error word; on an error clears the plan's control
// words and tags and returns 1.  < 0: a HIP call failed.
int step_plan_check(StepPlan* p, hipStream_t s);
int step_plan_test_hooks(StepPlan* p, uint32_t poll_limit, uint32_t tag_skew);
int step_plan_device(const StepPlan* p);
void step_plan_free(StepPlan* p);
// Lanes per row and group slots per lane of the M = 1 GEMV for G groups per
// row (false: no variant runs G).
bool gemv_variant(int G, int* L, int* P);

// ---- allocation (abi.hip): every device and pinned-host allocation of the
// library goes through these, so a test hook can make them fail ----
hipError_t dev_malloc(void** p, size_t bytes);
hipError_t pinned_malloc(void** p, size_t bytes);

// ---- per-stream workspace (abi.hip) ----
// A device buffer of at least `bytes` reserved for work enqueued on stream s
// of `device`; grown on demand (growth waits for s and reallocates).
hipError_t stream_workspace(int device, hipStream_t s, size_t bytes, void** out);

}  // namespace spectra
