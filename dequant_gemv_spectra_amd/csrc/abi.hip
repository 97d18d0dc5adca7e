// Host side of libspectra: the extern "C" entry points declared in
// include/spectra.h -- argument checks, the container's device allocation and
// header, packing orchestration and kernel dispatch.  Every computation on
// the data runs in the device kernels of pack.hip, gemv.hip and mfma.hip.
#include <stdio.h>
#include <string.h>
#include <sys/stat.h>
#include <unistd.h>

#include <map>
#include <mutex>
#include <new>
#include <unordered_map>
#include <utility>
#include <vector>

#include "../../include/spectra.h"
#include "spectra_internal.h"

namespace spectra {

namespace {
thread_local std::string g_last_error;
thread_local int g_last_status = SPECTRA_OK;

struct PropsCache {
  std::mutex mu;
  std::vector<DeviceProps> props;
  std::vector<bool> have;
};
PropsCache& props_cache() {
  static PropsCache pc;
  return pc;
}
}  // namespace

void set_error(const std::string& msg, int status) {
  g_last_error = msg;
  g_last_status = msg.empty() ? SPECTRA_OK : status;
}

int fail(int status, const std::string& msg) {
  set_error(msg, status);
  return status;
}

const DeviceProps& device_props(int device) {
  PropsCache& pc = props_cache();
  std::lock_guard<std::mutex> lk(pc.mu);
  if ((int)pc.props.size() <= device) {
    pc.props.resize(device + 1);
    pc.have.resize(device + 1, false);
  }
  if (!pc.have[device]) {
    hipDeviceProp_t p;
    DeviceProps d{256, 64 * 1024};
    if (hipGetDeviceProperties(&p, device) == hipSuccess) {
      d.cu_count = p.multiProcessorCount > 0 ? p.multiProcessorCount : 256;
      d.lds_per_block = p.sharedMemPerBlock;
    }
    pc.props[device] = d;
    pc.have[device] = true;
  }
  return pc.props[device];
}

namespace {
// Per (device, stream) workspaces.  A buffer that is outgrown is retired, not
// freed: a HIP graph captured earlier on that stream may still hold its
// address and be replayed later.  Retired buffers are freed only by
// spectra_release_workspaces, which the caller invokes once no such graph
// will run again (the total retired is below the live size, since each
// growth at least doubles it).
struct WorkspaceCache {
  std::mutex mu;
  std::map<std::pair<int, void*>, std::pair<void*, size_t>> bufs;
  std::vector<std::pair<int, void*>> retired;  // (device, buffer)
};
WorkspaceCache& workspace_cache() {
  static WorkspaceCache wc;
  return wc;
}
}  // namespace

// ---- device and pinned-host allocation, with a test hook ----
// spectra_test_fail_allocations(skip, count): the next `skip` allocations
// succeed, the `count` after them fail as out of memory.
namespace {
std::mutex g_alloc_mu;
int64_t g_alloc_skip = 0, g_alloc_fail = 0;

bool injected_failure() {
  std::lock_guard<std::mutex> lk(g_alloc_mu);
  if (g_alloc_fail <= 0) return false;
  if (g_alloc_skip > 0) {
    --g_alloc_skip;
    return false;
  }
  --g_alloc_fail;
  return true;
}
}  // namespace

hipError_t dev_malloc(void** p, size_t bytes) {
  if (injected_failure()) {
    *p = nullptr;
    return hipErrorOutOfMemory;
  }
  return hipMalloc(p, bytes);
}

hipError_t pinned_malloc(void** p, size_t bytes) {
  if (injected_failure()) {
    *p = nullptr;
    return hipErrorOutOfMemory;
  }
  return hipHostMalloc(p, bytes, hipHostMallocDefault);
}

hipError_t stream_workspace(int device, hipStream_t s, size_t bytes, void** out) {
  WorkspaceCache& wc = workspace_cache();
  std::lock_guard<std::mutex> lk(wc.mu);
  auto& e = wc.bufs[std::make_pair(device, static_cast<void*>(s))];
  if (e.first && e.second >= bytes) {
    *out = e.first;
    return hipSuccess;
  }
  size_t nb = bytes < 2 * e.second ? 2 * e.second : bytes;
  if (nb < (1u << 20)) nb = 1u << 20;
  void* p = nullptr;
  const hipError_t err = dev_malloc(&p, nb);
  if (err != hipSuccess) return err;
  if (e.first) wc.retired.emplace_back(device, e.first);  // work or graphs on s may still use it
  e = std::make_pair(p, nb);
  *out = p;
  return hipSuccess;
}

int release_workspaces() {
  WorkspaceCache& wc = workspace_cache();
  std::lock_guard<std::mutex> lk(wc.mu);
  int cur = -1;
  (void)hipGetDevice(&cur);
  int st = SPECTRA_OK;
  for (const auto& r : wc.retired) {
    if (hipSetDevice(r.first) != hipSuccess || hipDeviceSynchronize() != hipSuccess || hipFree(r.second) != hipSuccess)
      st = SPECTRA_E_HIP;
  }
  wc.retired.clear();
  if (cur >= 0) (void)hipSetDevice(cur);
  return st;
}

namespace {

std::string hip_msg(const char* what, hipError_t e) {
  return std::string(what) + ": " + hipGetErrorString(e);
}

// Handles.  The pointers the ABI hands out are identifiers, not addresses:
// each is drawn once from a counter and never reissued, so a freed handle
// stays invalid even when a later object lands at the same address, and a
// handle is checked by lookup without ever being dereferenced.
template <class T>
struct HandleTable {
  std::mutex mu;
  std::unordered_map<uintptr_t, T*> objs;
  uintptr_t next = 0x10000;
  T* publish(T* o) {
    std::lock_guard<std::mutex> lk(mu);
    const uintptr_t h = next;
    next += 16;
    objs.emplace(h, o);
    return reinterpret_cast<T*>(h);
  }
  T* get(const void* h) {
    std::lock_guard<std::mutex> lk(mu);
    const auto it = objs.find(reinterpret_cast<uintptr_t>(h));
    return it == objs.end() ? nullptr : it->second;
  }
  T* retire(const void* h) {
    std::lock_guard<std::mutex> lk(mu);
    const auto it = objs.find(reinterpret_cast<uintptr_t>(h));
    if (it == objs.end()) return nullptr;
    T* o = it->second;
    objs.erase(it);
    return o;
  }
};
HandleTable<spectra_container>& containers() {
  static HandleTable<spectra_container> t;
  return t;
}
spectra_container* cont(const spectra_container* h) { return containers().get(h); }

// Frees device buffers on scope exit unless released.
struct DevBuf {
  void* p = nullptr;
  ~DevBuf() {
    if (p) (void)hipFree(p);
  }
  void* release() {
    void* q = p;
    p = nullptr;
    return q;
  }
};


spectra_container* pack_impl(const uint16_t* W_dev, const uint16_t* g_dev, int64_t K, int64_t N,
                             hipStream_t s) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_error(hip_msg("hipGetDevice", e), SPECTRA_E_HIP);
    return nullptr;
  }
  const uint64_t mask_words = (uint64_t)((K + 31) / 32);
  DevBuf scratch, status;
  e = dev_malloc(&scratch.p, kurtosis_scratch_bytes(K, N));
  if (e != hipSuccess) {
    set_error(hip_msg("hipMalloc (kurtosis scratch)", e), SPECTRA_E_NOMEM);
    return nullptr;
  }
  e = dev_malloc(&status.p, 4 * (1 + mask_words));
  if (e != hipSuccess) {
    set_error(hip_msg("hipMalloc (status)", e), SPECTRA_E_NOMEM);
    return nullptr;
  }
  uint32_t* st = static_cast<uint32_t*>(status.p);
  if ((e = hipMemsetAsync(st, 0, 4 * (1 + mask_words), s)) != hipSuccess ||
      (e = launch_kurtosis(W_dev, g_dev, K, N, scratch.p, st, s)) != hipSuccess) {
    set_error(hip_msg("kurtosis launch", e), SPECTRA_E_HIP);
    return nullptr;
  }
  std::vector<uint32_t> host_status(1 + mask_words);
  if ((e = hipMemcpyAsync(host_status.data(), st, 4 * (1 + mask_words), hipMemcpyDeviceToHost,
                          s)) != hipSuccess ||
      (e = hipStreamSynchronize(s)) != hipSuccess) {
    set_error(hip_msg("kurtosis readback", e), SPECTRA_E_HIP);
    return nullptr;
  }
  if (host_status[0] & 1u) {
    set_error("W or gamma holds a non-finite value", SPECTRA_E_NONFINITE);
    return nullptr;
  }
  int64_t n_out = 0;
  for (uint64_t w = 0; w < mask_words; ++w) n_out += __builtin_popcount(host_status[1 + w]);

  spectra_container* c = new (std::nothrow) spectra_container();
  if (!c) {
    set_error("host allocation of the container handle failed", SPECTRA_E_NOMEM);
    return nullptr;
  }
  c->tag = kLiveTag;
  c->device = dev;
  c->K = K;
  c->N = N;
  c->n_out = n_out;
  c->K_b = K - n_out;
  c->G = (c->K_b + kGroup - 1) / kGroup;
  c->lay = make_layout(K, N, n_out);
  DevBuf img;
  e = dev_malloc(&img.p, c->lay.total);
  if (e != hipSuccess) {
    delete c;
    set_error(hip_msg("hipMalloc (container)", e), SPECTRA_E_NOMEM);
    return nullptr;
  }
  c->dev = static_cast<unsigned char*>(img.p);

  uint64_t hdr[kHeaderBytes / 8];
  memset(hdr, 0, sizeof(hdr));
  hdr[0] = (uint64_t)kMagic | ((uint64_t)kVersion << 32);
  hdr[1] = (uint64_t)K;
  hdr[2] = (uint64_t)N;
  hdr[3] = (uint64_t)c->K_b;
  hdr[4] = (uint64_t)c->G;
  hdr[5] = (uint64_t)n_out;
  hdr[6] = c->lay.mask;
  hdr[7] = c->lay.perm;
  hdr[8] = c->lay.codes;
  hdr[9] = c->lay.scales;
  hdr[10] = c->lay.zeros;
  hdr[11] = c->lay.outliers;
  hdr[12] = c->lay.total;
  if ((e = hipMemsetAsync(c->dev, 0, c->lay.total, s)) != hipSuccess ||
      (e = hipMemcpyAsync(c->dev, hdr, sizeof(hdr), hipMemcpyHostToDevice, s)) != hipSuccess ||
      (e = hipMemcpyAsync(c->dev + c->lay.mask, st + 1, 4 * mask_words, hipMemcpyDeviceToDevice,
                          s)) != hipSuccess ||
      (e = launch_quantize(W_dev, c, s)) != hipSuccess ||
      (e = hipStreamSynchronize(s)) != hipSuccess) {
    delete c;
    set_error(hip_msg("packing", e), SPECTRA_E_HIP);
    return nullptr;
  }
  img.release();
  return containers().publish(c);
}

// A registered container for fields f with a fresh device image (contents
// to be filled by the caller); nullptr with the error set on failure.
spectra_container* new_container(const ImageFields& f) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_error(hip_msg("hipGetDevice", e), SPECTRA_E_HIP);
    return nullptr;
  }
  spectra_container* c = new (std::nothrow) spectra_container();
  if (!c) {
    set_error("host allocation of the container handle failed", SPECTRA_E_NOMEM);
    return nullptr;
  }
  c->tag = kLiveTag;
  c->device = dev;
  c->K = f.K;
  c->N = f.N;
  c->K_b = f.K_b;
  c->G = f.G;
  c->n_out = f.n_out;
  c->lay = f.lay;
  void* p = nullptr;
  e = dev_malloc(&p, f.lay.total);
  if (e != hipSuccess) {
    delete c;
    set_error(hip_msg("hipMalloc (container)", e), SPECTRA_E_NOMEM);
    return nullptr;
  }
  c->dev = static_cast<unsigned char*>(p);
  return c;
}

void drop_container(spectra_container* c) {
  if (!c) return;
  if (c->dev) (void)hipFree(c->dev);
  delete c;
}

uint64_t chunk_size(uint64_t want) {
  uint64_t c = want == 0 ? (8ull << 20) : want;
  if (c < 4096) c = 4096;
  return (c + 255) / 256 * 256;
}

// Pinned host staging buffers, freed on scope exit.
struct Pinned {
  void* p = nullptr;
  ~Pinned() {
    if (p) (void)hipHostFree(p);
  }
};

struct File {
  FILE* fp = nullptr;
  ~File() {
    if (fp) fclose(fp);
  }
};

// ---- KV caches ----

}  // namespace
}  // namespace spectra

struct spectra_kv {
  int device;
  int64_t length;
  spectra::KvView view;
  unsigned char* dev;  // one allocation: K records, scales, zeros, then V's
  uint64_t plane_bytes[3];  // per plane: records, scales, zeros (capacity-sized)
};

struct spectra_step {
  spectra::StepPlan* plan;
};

namespace spectra {
namespace {
HandleTable<spectra_kv>& kvs() {
  static HandleTable<spectra_kv> t;
  return t;
}
HandleTable<spectra_step>& steps() {
  static HandleTable<spectra_step> t;
  return t;
}
}  // namespace
}  // namespace spectra

// ---- the no-allocation product's scratch ----
// A fixed device array that the MFMA path of spectra_gemm_noalloc uses as its
// workspace (x permuted to bulk order), so that call allocates nothing.  Each
// GPU the library runs on holds its own copy for the life of the process.
// In host code the array's name is only a host-side stand-in: its device
// address comes from hipGetSymbolAddress, once per device, and only that
// address is ever handed to a kernel.
constexpr size_t kScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace spectra {
namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];  // device address of `scratch` per device, once looked up

// The scratch address on `device`, which must be the current device.
hipError_t scratch_on(int device, void** out) {
  if (device < 0 || device >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = p;
  }
  *out = g_scratch_ptr[device];
  return hipSuccess;
}
}  // namespace
}  // namespace spectra

using namespace spectra;

extern "C" {

int spectra_version(void) { return 1; }

const char* spectra_last_error(void) { return g_last_error.c_str(); }

int spectra_last_status(void) { return g_last_status; }

int spectra_test_fail_allocations(int64_t skip, int64_t count) {
  if (skip < 0 || count < 0) return fail(SPECTRA_E_INVAL, "skip and count must be >= 0");
  {
    std::lock_guard<std::mutex> lk(g_alloc_mu);
    g_alloc_skip = skip;
    g_alloc_fail = count;
  }
  set_error("", SPECTRA_OK);
  return SPECTRA_OK;
}

int spectra_release_workspaces(void) {
  const int st = release_workspaces();
  if (st != SPECTRA_OK) return fail(st, "freeing a retired workspace failed");
  return SPECTRA_OK;
}

spectra_container* spectra_pack_device(const void* W, const void* gamma, int64_t K, int64_t N,
                                       void* stream) {
  set_error("", SPECTRA_E_INVAL);
  if (!W || !gamma) {
    set_error("null W or gamma", SPECTRA_E_INVAL);
    return nullptr;
  }
  if (check_shape(K, N) != SPECTRA_OK) return nullptr;
  return pack_impl(static_cast<const uint16_t*>(W), static_cast<const uint16_t*>(gamma), K, N,
                   static_cast<hipStream_t>(stream));
}

spectra_container* spectra_pack(const uint16_t* W, const uint16_t* gamma, int64_t K, int64_t N) {
  set_error("", SPECTRA_E_INVAL);
  if (!W || !gamma) {
    set_error("null W or gamma", SPECTRA_E_INVAL);
    return nullptr;
  }
  if (check_shape(K, N) != SPECTRA_OK) return nullptr;
  DevBuf wd, gd;
  hipError_t e;
  const size_t wbytes = 2ull * (uint64_t)N * (uint64_t)K;
  if ((e = dev_malloc(&wd.p, wbytes)) != hipSuccess || (e = dev_malloc(&gd.p, 2ull * K)) != hipSuccess) {
    set_error(hip_msg("hipMalloc (staging W/gamma)", e), SPECTRA_E_NOMEM);
    return nullptr;
  }
  if ((e = hipMemcpy(wd.p, W, wbytes, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(gd.p, gamma, 2ull * K, hipMemcpyHostToDevice)) != hipSuccess) {
    set_error(hip_msg("upload W/gamma", e), SPECTRA_E_HIP);
    return nullptr;
  }
  return pack_impl(static_cast<const uint16_t*>(wd.p), static_cast<const uint16_t*>(gd.p), K, N,
                   nullptr);
}

void spectra_free(spectra_container* h) {
  spectra_container* c = containers().retire(h);
  if (!c) return;
  c->tag = kDeadTag;
  int cur = -1;
  (void)hipGetDevice(&cur);
  if (cur != c->device) (void)hipSetDevice(c->device);
  (void)hipFree(c->dev);
  if (cur >= 0 && cur != c->device) (void)hipSetDevice(cur);
  c->dev = nullptr;
  delete c;
}

int spectra_info(const spectra_container* h, spectra_info_t* out) {
  const spectra_container* c = cont(h);
  if (!c) return fail(SPECTRA_E_INVAL, "invalid or freed container");
  if (!out) return fail(SPECTRA_E_INVAL, "null info pointer");
  const uint64_t NG = (uint64_t)c->N * (uint64_t)c->G;
  out->K = c->K;
  out->N = c->N;
  out->K_b = c->K_b;
  out->G = c->G;
  out->n_out = c->n_out;
  out->bytes_codes = 16 * NG;
  out->bytes_scales = 2 * NG;
  out->bytes_zeros = (NG + 1) / 2;
  out->bytes_outliers = 2ull * (uint64_t)c->N * (uint64_t)c->n_out;
  out->bytes_payload = out->bytes_codes + out->bytes_scales + out->bytes_zeros + out->bytes_outliers;
  out->bytes_meta = kHeaderBytes + 4ull * (uint64_t)((c->K + 31) / 32) + 4ull * (uint64_t)c->K;
  out->bytes_total = c->lay.total;
  return SPECTRA_OK;
}

int spectra_export(const spectra_container* h, void* host_dst, uint64_t cap) {
  const spectra_container* c = cont(h);
  if (!c) return fail(SPECTRA_E_INVAL, "invalid or freed container");
  if (!host_dst) return fail(SPECTRA_E_INVAL, "null destination");
  if (cap < c->lay.total) return fail(SPECTRA_E_INVAL, "destination smaller than total_bytes");
  hipError_t e = hipMemcpy(host_dst, c->dev, c->lay.total, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(SPECTRA_E_HIP, hip_msg("export copy", e));
  return SPECTRA_OK;
}

namespace {

// The kernel a product of M rows runs with the selector, or a status < 0
// (message set).  The container must be live and M and kernel in range.
int plan_of(const DeviceView& v, int64_t M, int kernel) {
  // auto: the GEMV for M <= 2; from M = 3 the split-K MFMA kernel where it
  // takes the shape (M <= 16; measured faster than the tiled kernel at every
  // shape both take), else the tiled kernel, else the strip kernel; the GEMV
  // again at M = 3, 4 where only the strip kernel would take the shape
  const bool splitk = mfma_splitk_supports(v, M), tiled = mfma_tiled_supports(v, M);
  const bool auto_gemv = gemv_supports(v, M) && (M <= 2 || (!splitk && !tiled));
  if (kernel == SPECTRA_KERNEL_GEMV || (kernel == SPECTRA_KERNEL_AUTO && auto_gemv)) {
    if (!gemv_supports(v, M)) return fail(SPECTRA_E_UNSUPPORTED, "GEMV kernel cannot run this shape");
    return SPECTRA_PLAN_GEMV;
  }
  if (!mfma_supports(v, M)) return fail(SPECTRA_E_UNSUPPORTED, "MFMA kernel cannot run this shape");
  switch (kernel) {
    case SPECTRA_KERNEL_MFMA_SPLITK:
      if (!splitk) return fail(SPECTRA_E_UNSUPPORTED, "split-K MFMA kernel cannot run this shape");
      return SPECTRA_PLAN_MFMA_SPLITK;
    case SPECTRA_KERNEL_MFMA_TILED:
      if (!tiled) return fail(SPECTRA_E_UNSUPPORTED, "tiled MFMA kernel cannot run this shape");
      return SPECTRA_PLAN_MFMA_TILED;
    case SPECTRA_KERNEL_MFMA_STRIP:
      return SPECTRA_PLAN_MFMA;
    default:
      return splitk ? SPECTRA_PLAN_MFMA_SPLITK : (tiled ? SPECTRA_PLAN_MFMA_TILED : SPECTRA_PLAN_MFMA);
  }
}

size_t workspace_of(const DeviceView& v, int64_t M, int plan) {
  return plan == SPECTRA_PLAN_MFMA_SPLITK ? mfma_splitk_workspace_bytes(v, M) : mfma_workspace_bytes(v, M);
}

int check_gemm_args(const spectra_container* c, int64_t M, int kernel) {
  if (!c) return fail(SPECTRA_E_INVAL, "invalid or freed container");
  if (M < 1 || M > SPECTRA_MAX_M) return fail(SPECTRA_E_INVAL, "M out of range [1, 2^20]");
  if (kernel < SPECTRA_KERNEL_AUTO || kernel > SPECTRA_KERNEL_MFMA_SPLITK)
    return fail(SPECTRA_E_INVAL, "unknown kernel selector");
  return SPECTRA_OK;
}

}  // namespace

int spectra_gemm_plan(const spectra_container* h, int64_t M, int kernel) {
  const spectra_container* c = cont(h);
  const int st = check_gemm_args(c, M, kernel);
  if (st != SPECTRA_OK) return st;
  return plan_of(c->view(), M, kernel);
}

int spectra_gemm_ex(const spectra_container* h, const void* x, void* y, int64_t M, void* stream,
                    int kernel) {
  const spectra_container* c = cont(h);
  if (!c) return fail(SPECTRA_E_INVAL, "invalid or freed container");
  if (!x || !y) return fail(SPECTRA_E_INVAL, "null x or y");
  if ((reinterpret_cast<uintptr_t>(x) & 3) || (reinterpret_cast<uintptr_t>(y) & 3))
    return fail(SPECTRA_E_INVAL, "x and y must be 4-byte aligned");
  const int st = check_gemm_args(c, M, kernel);
  if (st != SPECTRA_OK) return st;
  const DeviceView v = c->view();
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  uint16_t* yp = static_cast<uint16_t*>(y);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  const int plan = plan_of(v, M, kernel);
  if (plan < 0) return plan;
  if (plan == SPECTRA_PLAN_GEMV) {
    e = launch_gemv(v, xp, yp, M, s);
  } else {
    void* ws = nullptr;
    e = stream_workspace(c->device, s, workspace_of(v, M, plan), &ws);
    if (e != hipSuccess) return fail(SPECTRA_E_NOMEM, hip_msg("MFMA workspace", e));
    e = launch_mfma_ws(v, xp, yp, M, ws, s, plan);
  }
  if (e != hipSuccess) return fail(SPECTRA_E_HIP, hip_msg("kernel launch", e));
  return SPECTRA_OK;
}

int spectra_gemm_noalloc(const spectra_container* h, const void* x, void* y, int64_t M, void* stream, int kernel) {
  const spectra_container* c = cont(h);
  if (!c) return fail(SPECTRA_E_INVAL, "invalid or freed container");
  if (!x || !y) return fail(SPECTRA_E_INVAL, "null x or y");
  if ((reinterpret_cast<uintptr_t>(x) & 3) || (reinterpret_cast<uintptr_t>(y) & 3))
    return fail(SPECTRA_E_INVAL, "x and y must be 4-byte aligned");
  const int st = check_gemm_args(c, M, kernel);
  if (st != SPECTRA_OK) return st;
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return fail(SPECTRA_E_HIP, hip_msg("hipGetDevice", e));
  if (cur != c->device) return fail(SPECTRA_E_INVAL, "the container's device must be the current device");
  const DeviceView v = c->view();
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  uint16_t* yp = static_cast<uint16_t*>(y);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int plan = plan_of(v, M, kernel);
  if (plan < 0) return plan;
  if (plan == SPECTRA_PLAN_GEMV) {
    e = launch_gemv(v, xp, yp, M, s);  // no workspace
  } else {
    // the split-K kernel's partial sums may not fit the scratch: then, unless
    // it was forced, the kernel it replaces, whose workspace is x alone
    int run = plan;
    if (run == SPECTRA_PLAN_MFMA_SPLITK && kernel != SPECTRA_KERNEL_MFMA_SPLITK &&
        mfma_splitk_workspace_bytes(v, M) > kScratchBytes)
      run = mfma_tiled_supports(v, M) ? SPECTRA_PLAN_MFMA_TILED : SPECTRA_PLAN_MFMA;
    const size_t need = workspace_of(v, M, run);
    if (need > kScratchBytes)
      return fail(SPECTRA_E_UNSUPPORTED, "the product needs " + std::to_string(need) +
                                             " bytes of workspace, more than the 8 MiB static scratch");
    void* ws = nullptr;
    if ((e = scratch_on(c->device, &ws)) != hipSuccess) return fail(SPECTRA_E_HIP, hip_msg("static scratch address", e));
    e = launch_mfma_ws(v, xp, yp, M, ws, s, run);
  }
  if (e != hipSuccess) return fail(SPECTRA_E_HIP, hip_msg("kernel launch", e));
  return SPECTRA_OK;
}

int spectra_gemm(const spectra_container* c, const void* x, void* y, int64_t M) {
  return spectra_gemm_ex(c, x, y, M, nullptr, SPECTRA_KERNEL_AUTO);
}

int spectra_gemm_grouped(const spectra_container* const* cs, int count, const void* x,
                         void* const* ys, int64_t M, void* stream) {
  if (!cs || !ys || !x) return fail(SPECTRA_E_INVAL, "null argument");
  if (count < 1 || count > 64) return fail(SPECTRA_E_INVAL, "count out of range [1, 64]");
  if (M != 1) return fail(SPECTRA_E_UNSUPPORTED, "grouped launch supports M = 1");
  DeviceView vs[64];
  const spectra_container* objs[64];
  for (int i = 0; i < count; ++i) {
    objs[i] = cont(cs[i]);
    if (!objs[i]) return fail(SPECTRA_E_INVAL, "invalid or freed container in group");
    if (!ys[i] || (reinterpret_cast<uintptr_t>(ys[i]) & 3))
      return fail(SPECTRA_E_INVAL, "null or misaligned y in group");
    if (objs[i]->K != objs[0]->K || objs[i]->device != objs[0]->device)
      return fail(SPECTRA_E_INVAL, "grouped containers must share K and device");
    vs[i] = objs[i]->view();
    if (!gemv_supports(vs[i], 1))
      return fail(SPECTRA_E_UNSUPPORTED, "GEMV kernel cannot run a container of the group");
  }
  if (reinterpret_cast<uintptr_t>(x) & 3) return fail(SPECTRA_E_INVAL, "x must be 4-byte aligned");
  hipError_t e = launch_gemv_grouped(vs, count, static_cast<const uint16_t*>(x),
                                     reinterpret_cast<uint16_t* const*>(ys),
                                     static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return fail(SPECTRA_E_UNSUPPORTED, "grouped launch not available");
  if (e != hipSuccess) return fail(SPECTRA_E_HIP, hip_msg("grouped launch", e));
  return SPECTRA_OK;
}

int spectra_embed(const spectra_container* h, const void* ids, int64_t T, void* out, void* stream) {
  const spectra_container* c = cont(h);
  if (!c) return fail(SPECTRA_E_INVAL, "invalid or freed container");
  if (T < 0 || T > SPECTRA_MAX_T) return fail(SPECTRA_E_INVAL, "T out of range [0, 2^31]");
  if (T == 0) return SPECTRA_OK;
  if (!ids || !out) return fail(SPECTRA_E_INVAL, "null ids or out");
  if ((reinterpret_cast<uintptr_t>(ids) & 3) || (reinterpret_cast<uintptr_t>(out) & 3))
    return fail(SPECTRA_E_INVAL, "ids and out must be 4-byte aligned");
  const DeviceView v = c->view();
  if (!embed_supports(v)) return fail(SPECTRA_E_UNSUPPORTED, "row gather: a row does not fit the LDS row buffer");
  const hipError_t e = launch_embed(v, static_cast<const int32_t*>(ids), T, static_cast<uint16_t*>(out),
                                    static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SPECTRA_E_HIP, hip_msg("row gather launch", e));
  return SPECTRA_OK;
}

int spectra_validate_image(const void* image, uint64_t bytes) {
  if (!image) return fail(SPECTRA_E_INVAL, "null image");
  ImageFields f;
  return validate_host_image(static_cast<const unsigned char*>(image), bytes, f);
}

spectra_container* spectra_import(const void* image, uint64_t bytes) {
  if (!image) {
    set_error("null image", SPECTRA_E_INVAL);
    return nullptr;
  }
  ImageFields f;
  if (validate_host_image(static_cast<const unsigned char*>(image), bytes, f) != SPECTRA_OK) return nullptr;
  spectra_container* c = new_container(f);
  if (!c) return nullptr;
  const hipError_t e = hipMemcpy(c->dev, image, bytes, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    drop_container(c);
    set_error(hip_msg("upload of the image", e), SPECTRA_E_HIP);
    return nullptr;
  }
  return containers().publish(c);
}

int spectra_save(const spectra_container* h, const char* path, uint64_t chunk_bytes) {
  const spectra_container* c = cont(h);
  if (!c) return fail(SPECTRA_E_INVAL, "invalid or freed container");
  if (!path) return fail(SPECTRA_E_INVAL, "null path");
  const uint64_t chunk = chunk_size(chunk_bytes);
  Pinned stage;
  hipError_t e = pinned_malloc(&stage.p, chunk);
  if (e != hipSuccess) return fail(SPECTRA_E_NOMEM, hip_msg("pinned staging buffer", e));
  int st = SPECTRA_OK;
  {
    File out;
    out.fp = fopen(path, "wb");
    if (!out.fp) return fail(SPECTRA_E_IO, std::string("cannot create ") + path);
    for (uint64_t pos = 0; pos < c->lay.total && st == SPECTRA_OK; pos += chunk) {
      const uint64_t n = c->lay.total - pos < chunk ? c->lay.total - pos : chunk;
      e = hipMemcpy(stage.p, c->dev + pos, n, hipMemcpyDeviceToHost);
      if (e != hipSuccess) st = fail(SPECTRA_E_HIP, hip_msg("copy of the image", e));
      else if (fwrite(stage.p, 1, n, out.fp) != n) st = fail(SPECTRA_E_IO, std::string("write to ") + path + " failed");
    }
    if (st == SPECTRA_OK && fflush(out.fp) != 0) st = fail(SPECTRA_E_IO, std::string("write to ") + path + " failed");
    if (fclose(out.fp) != 0 && st == SPECTRA_OK) st = fail(SPECTRA_E_IO, std::string("close of ") + path + " failed");
    out.fp = nullptr;
  }
  if (st != SPECTRA_OK) (void)unlink(path);
  return st;
}

spectra_container* spectra_load(const char* path, uint64_t chunk_bytes) {
  if (!path) {
    set_error("null path", SPECTRA_E_INVAL);
    return nullptr;
  }
  File in;
  in.fp = fopen(path, "rb");
  if (!in.fp) {
    set_error(std::string("cannot open ") + path, SPECTRA_E_IO);
    return nullptr;
  }
  struct stat sb;
  if (fstat(fileno(in.fp), &sb) != 0 || sb.st_size < 0) {
    set_error(std::string("cannot stat ") + path, SPECTRA_E_IO);
    return nullptr;
  }
  const uint64_t bytes = (uint64_t)sb.st_size;
  unsigned char hdr[kHeaderBytes];
  if (bytes < kHeaderBytes || fread(hdr, 1, kHeaderBytes, in.fp) != kHeaderBytes) {
    set_error(std::string(path) + ": shorter than a container header", SPECTRA_E_INVAL);
    return nullptr;
  }
  ImageFields f;
  if (parse_header(hdr, bytes, f) != SPECTRA_OK) return nullptr;
  if (fseek(in.fp, 0, SEEK_SET) != 0) {
    set_error(std::string("cannot rewind ") + path, SPECTRA_E_IO);
    return nullptr;
  }
  // the container first, then the host staging and the stream: a failure
  // leaves nothing behind
  spectra_container* c = new_container(f);
  if (!c) return nullptr;
  const uint64_t chunk = chunk_size(chunk_bytes);
  Pinned stage[2];
  for (int i = 0; i < 2; ++i) {
    const hipError_t e = pinned_malloc(&stage[i].p, chunk);
    if (e != hipSuccess) {
      drop_container(c);
      set_error(hip_msg("pinned staging buffer", e), SPECTRA_E_NOMEM);
      return nullptr;
    }
  }
  hipStream_t s = nullptr;
  if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) {
    drop_container(c);
    set_error("stream creation failed", SPECTRA_E_HIP);
    return nullptr;
  }
  hipEvent_t done[2] = {nullptr, nullptr};
  for (int i = 0; i < 2; ++i) (void)hipEventCreateWithFlags(&done[i], hipEventDisableTiming);
  // mask and perm are kept on the host as they pass, for the final check
  std::vector<unsigned char> meta(f.lay.codes - f.lay.mask);
  int st = SPECTRA_OK;
  bool used[2] = {false, false};
  for (uint64_t pos = 0, k = 0; st == SPECTRA_OK && pos < bytes; pos += chunk, ++k) {
    const int b = (int)(k & 1);
    const uint64_t n = bytes - pos < chunk ? bytes - pos : chunk;
    // the buffer's previous upload must be done before it is refilled
    if (used[b] && hipEventSynchronize(done[b]) != hipSuccess) {
      st = fail(SPECTRA_E_HIP, "staging upload failed");
      break;
    }
    unsigned char* buf = static_cast<unsigned char*>(stage[b].p);
    if (fread(buf, 1, n, in.fp) != n) {
      st = fail(SPECTRA_E_IO, std::string("read of ") + path + " failed");
      break;
    }
    if (check_range(f, pos, buf, n) != SPECTRA_OK) {
      st = SPECTRA_E_INVAL;
      break;
    }
    const uint64_t mlo = pos > f.lay.mask ? pos : f.lay.mask;
    const uint64_t mhi = pos + n < f.lay.codes ? pos + n : f.lay.codes;
    if (mlo < mhi) memcpy(meta.data() + (mlo - f.lay.mask), buf + (mlo - pos), mhi - mlo);
    hipError_t e = hipMemcpyAsync(c->dev + pos, buf, n, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipEventRecord(done[b], s);
    if (e != hipSuccess) {
      st = fail(SPECTRA_E_HIP, hip_msg("upload of the image", e));
      break;
    }
    used[b] = true;
  }
  if (hipStreamSynchronize(s) != hipSuccess && st == SPECTRA_OK) st = fail(SPECTRA_E_HIP, "upload failed");
  if (st == SPECTRA_OK)
    st = check_meta(f, reinterpret_cast<const uint32_t*>(meta.data()),
                    reinterpret_cast<const int32_t*>(meta.data() + (f.lay.perm - f.lay.mask)));
  for (int i = 0; i < 2; ++i)
    if (done[i]) (void)hipEventDestroy(done[i]);
  (void)hipStreamDestroy(s);
  if (st != SPECTRA_OK) {
    drop_container(c);
    return nullptr;
  }
  return containers().publish(c);
}

spectra_kv* spectra_kv_create(int64_t capacity, int32_t heads, int32_t head_dim) {
  if (capacity < 1 || capacity > ((int64_t)1 << 31) || !kv_shape_supported(heads, head_dim)) {
    set_error("KV cache: capacity in [1, 2^31], heads in [1, 1024], head_dim 64, 128 or 256", SPECTRA_E_INVAL);
    return nullptr;
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_error(hip_msg("hipGetDevice", e), SPECTRA_E_HIP);
    return nullptr;
  }
  const uint64_t G = (uint64_t)head_dim / 32;
  const uint64_t n = (uint64_t)capacity * (uint64_t)heads * G;  // groups per plane
  const uint64_t rec = align_up(16 * n), sc = align_up(2 * n), zb = align_up(n / 2);
  spectra_kv* kv = new (std::nothrow) spectra_kv();
  if (!kv) {
    set_error("host allocation of the KV handle failed", SPECTRA_E_NOMEM);
    return nullptr;
  }
  void* p = nullptr;
  e = dev_malloc(&p, 2 * (rec + sc + zb));
  if (e != hipSuccess) {
    delete kv;
    set_error(hip_msg("hipMalloc (KV cache)", e), SPECTRA_E_NOMEM);
    return nullptr;
  }
  unsigned char* b = static_cast<unsigned char*>(p);
  kv->device = dev;
  kv->length = 0;
  kv->dev = b;
  kv->plane_bytes[0] = rec;
  kv->plane_bytes[1] = sc;
  kv->plane_bytes[2] = zb;
  KvView& v = kv->view;
  v.k.codes = reinterpret_cast<uint4*>(b);
  v.k.scales = reinterpret_cast<uint16_t*>(b + rec);
  v.k.zeros = b + rec + sc;
  unsigned char* b2 = b + rec + sc + zb;
  v.v.codes = reinterpret_cast<uint4*>(b2);
  v.v.scales = reinterpret_cast<uint16_t*>(b2 + rec);
  v.v.zeros = b2 + rec + sc;
  v.cap = capacity;
  v.H = heads;
  v.D = head_dim;
  v.G = (int32_t)G;
  return kvs().publish(kv);
}

int spectra_kv_append(spectra_kv* h, const void* k, const void* v, int64_t T, void* stream) {
  spectra_kv* kv = kvs().get(h);
  if (!kv) return fail(SPECTRA_E_INVAL, "invalid or freed KV cache");
  if (T < 0) return fail(SPECTRA_E_INVAL, "T < 0");
  if (T > kv->view.cap - kv->length) return fail(SPECTRA_E_INVAL, "append past the KV cache capacity");
  if (T == 0) return SPECTRA_OK;
  if (!k || !v) return fail(SPECTRA_E_INVAL, "null k or v");
  if ((reinterpret_cast<uintptr_t>(k) & 15) || (reinterpret_cast<uintptr_t>(v) & 15))
    return fail(SPECTRA_E_INVAL, "k and v must be 16-byte aligned");
  const hipError_t e = launch_kv_append(kv->view, static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                                        T, kv->length, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SPECTRA_E_HIP, hip_msg("KV append launch", e));
  kv->length += T;
  return SPECTRA_OK;
}

int spectra_kv_attend(const spectra_kv* h, const void* q, int32_t q_heads, void* out, void* stream) {
  const spectra_kv* kv = kvs().get(h);
  if (!kv) return fail(SPECTRA_E_INVAL, "invalid or freed KV cache");
  if (kv->length < 1) return fail(SPECTRA_E_INVAL, "attention over an empty KV cache");
  if (kv->length > kv_max_attend_length())
    return fail(SPECTRA_E_UNSUPPORTED, "attention over more than 524288 cached tokens");
  if (!q || !out) return fail(SPECTRA_E_INVAL, "null q or out");
  if ((reinterpret_cast<uintptr_t>(q) & 3) || (reinterpret_cast<uintptr_t>(out) & 3))
    return fail(SPECTRA_E_INVAL, "q and out must be 4-byte aligned");
  const int H = kv->view.H;
  if (q_heads < H || q_heads % H != 0 || q_heads / H > kv_max_rep())
    return fail(SPECTRA_E_INVAL, "q_heads must be heads times 1 .. 16");
  const int rep = q_heads / H;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  hipError_t e = stream_workspace(kv->device, s, kv_attend_workspace_bytes(kv->view, rep, kv->length), &ws);
  if (e != hipSuccess) return fail(SPECTRA_E_NOMEM, hip_msg("KV attention workspace", e));
  e = launch_kv_attend(kv->view, static_cast<const uint16_t*>(q), rep, kv->length, static_cast<uint16_t*>(out),
                       ws, s);
  if (e != hipSuccess) return fail(SPECTRA_E_HIP, hip_msg("KV attention launch", e));
  return SPECTRA_OK;
}

int64_t spectra_kv_length(const spectra_kv* h) {
  const spectra_kv* kv = kvs().get(h);
  return kv ? kv->length : -1;
}

int spectra_kv_reset(spectra_kv* h) {
  spectra_kv* kv = kvs().get(h);
  if (!kv) return fail(SPECTRA_E_INVAL, "invalid or freed KV cache");
  kv->length = 0;
  return SPECTRA_OK;
}

int spectra_kv_export(const spectra_kv* h, void* host_dst, uint64_t cap) {
  const spectra_kv* kv = kvs().get(h);
  if (!kv) return fail(SPECTRA_E_INVAL, "invalid or freed KV cache");
  if (!host_dst) return fail(SPECTRA_E_INVAL, "null destination");
  const uint64_t n = (uint64_t)kv->length * (uint64_t)kv->view.H * (uint64_t)kv->view.G;
  const uint64_t part[3] = {16 * n, 2 * n, n / 2};
  if (cap < 2 * (part[0] + part[1] + part[2])) return fail(SPECTRA_E_INVAL, "destination too small");
  unsigned char* dst = static_cast<unsigned char*>(host_dst);
  const unsigned char* planes[2] = {kv->dev, kv->dev + kv->plane_bytes[0] + kv->plane_bytes[1] + kv->plane_bytes[2]};
  for (int pl = 0; pl < 2; ++pl) {
    uint64_t off = 0;
    for (int i = 0; i < 3; ++i) {
      const hipError_t e = hipMemcpy(dst, planes[pl] + off, part[i], hipMemcpyDeviceToHost);
      if (e != hipSuccess) return fail(SPECTRA_E_HIP, hip_msg("KV export copy", e));
      dst += part[i];
      off += kv->plane_bytes[i];
    }
  }
  return SPECTRA_OK;
}

void spectra_kv_free(spectra_kv* h) {
  spectra_kv* kv = kvs().retire(h);
  if (!kv) return;
  int cur = -1;
  (void)hipGetDevice(&cur);
  if (cur != kv->device) (void)hipSetDevice(kv->device);
  (void)hipFree(kv->dev);
  if (cur >= 0 && cur != kv->device) (void)hipSetDevice(cur);
  delete kv;
}

spectra_step* spectra_step_create(const spectra_step_phase* phases, int32_t nphases) {
  set_error("", SPECTRA_E_INVAL);
  if (!phases) {
    set_error("null phases", SPECTRA_E_INVAL);
    return nullptr;
  }
  if (nphases < 1 || nphases > 4096) {
    set_error("phase count out of range [1, 4096]", SPECTRA_E_INVAL);
    return nullptr;
  }
  std::vector<StepPhaseSpec> spec((size_t)nphases);
  int device = -1;
  for (int p = 0; p < nphases; ++p) {
    const spectra_step_phase& ph = phases[p];
    StepPhaseSpec& sp = spec[(size_t)p];
    if (ph.ntasks < 1 || ph.ntasks > SPECTRA_STEP_MAX_TASKS) {
      set_error("tasks per phase out of range [1, 4]", SPECTRA_E_INVAL);
      return nullptr;
    }
    sp.ntasks = ph.ntasks;
    for (int i = 0; i < ph.ntasks; ++i) {
      const spectra_container* c = cont(ph.c[i]);
      if (!c) {
        set_error("invalid or freed container in a phase", SPECTRA_E_INVAL);
        return nullptr;
      }
      if (device < 0) device = c->device;
      if (c->device != device) {
        set_error("the containers of a decode step must share one device", SPECTRA_E_INVAL);
        return nullptr;
      }
      sp.t[i].v = c->view();
      sp.t[i].y = static_cast<uint16_t*>(ph.y[i]);
    }
    if (ph.input < -1 || ph.input >= p) {
      set_error("a phase's input must be -1 (external x) or an earlier phase", SPECTRA_E_INVAL);
      return nullptr;
    }
    sp.input = ph.input;
    sp.x = static_cast<const uint16_t*>(ph.x);
    sp.x_scale = ph.x_scale;
  }
  int cur = -1;
  (void)hipGetDevice(&cur);
  if (cur != device && hipSetDevice(device) != hipSuccess) {
    set_error("cannot make the containers' device current", SPECTRA_E_HIP);
    return nullptr;
  }
  StepPlan* plan = nullptr;
  const int st = step_plan_create(spec.data(), nphases, device, &plan);
  if (cur >= 0 && cur != device) (void)hipSetDevice(cur);
  if (st != SPECTRA_OK) return nullptr;
  spectra_step* obj = new (std::nothrow) spectra_step();
  if (!obj) {
    step_plan_free(plan);
    set_error("host allocation of the step handle failed", SPECTRA_E_NOMEM);
    return nullptr;
  }
  obj->plan = plan;
  return steps().publish(obj);
}

int spectra_step_run(spectra_step* h, void* stream) {
  spectra_step* st = steps().get(h);
  if (!st) return fail(SPECTRA_E_INVAL, "invalid or freed decode step");
  const hipError_t e = step_plan_run(st->plan, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SPECTRA_E_HIP, hip_msg("decode step launch", e));
  return SPECTRA_OK;
}

int spectra_step_status(spectra_step* h, void* stream) {
  spectra_step* st = steps().get(h);
  if (!st) return fail(SPECTRA_E_INVAL, "invalid or freed decode step");
  const int r = step_plan_check(st->plan, static_cast<hipStream_t>(stream));
  if (r < 0) return r;
  if (r > 0) return fail(SPECTRA_E_TIMEOUT, "a wait inside the decode step gave up; its outputs are invalid");
  return SPECTRA_OK;
}

int spectra_step_test_hooks(spectra_step* h, uint32_t poll_limit, uint32_t tag_skew) {
  spectra_step* st = steps().get(h);
  if (!st) return fail(SPECTRA_E_INVAL, "invalid or freed decode step");
  return step_plan_test_hooks(st->plan, poll_limit, tag_skew);
}

void spectra_step_free(spectra_step* h) {
  spectra_step* st = steps().retire(h);
  if (!st) return;
  int cur = -1;
  (void)hipGetDevice(&cur);
  const int dev = step_plan_device(st->plan);
  if (cur != dev) (void)hipSetDevice(dev);
  step_plan_free(st->plan);
  if (cur >= 0 && cur != dev) (void)hipSetDevice(cur);
  delete st;
}

}  // extern "C"
