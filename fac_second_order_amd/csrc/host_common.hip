// Host-side plumbing of libkfac: status text, thread-local error text, device
// check, descriptor upload by kernel arguments and opt-in per-kernel event timing.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "common.hpp"

namespace kfac {

static thread_local char g_err[512] = "";

kfac_status fail(kfac_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

kfac_status hip_fail(hipError_t e, const char* what) {
  return fail(KFAC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

kfac_status check_device() {
  static int state[64];  // 0 unknown, 1 gfx950, 2 other (benign race: idempotent)
  int dev = 0;
  KFAC_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return fail(KFAC_ERR_UNSUPPORTED, "device index %d out of range", dev);
  if (state[dev] == 0) {
    hipDeviceProp_t prop;
    KFAC_HIP(hipGetDeviceProperties(&prop, dev));
    state[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
  }
  if (state[dev] != 1) return fail(KFAC_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
  return KFAC_OK;
}

kfac_status check_workspace(const void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return KFAC_OK;
  if (ws == nullptr) return fail(KFAC_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0)
    return fail(KFAC_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < need)
    return fail(KFAC_ERR_WORKSPACE, "workspace of %zu bytes is too small (%zu needed)", ws_bytes, need);
  return KFAC_OK;
}

// ---- descriptor upload ------------------------------------------------------
// Descriptor tables travel as kernel arguments, up to 1000 words (just under 4 KB of
// arguments) per launch.
struct UploadChunk {
  uint32_t w[1000];
};

__global__ void __launch_bounds__(256) upload_kernel(uint32_t* dst, UploadChunk c, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = c.w[i];
}

kfac_status upload(void* dst_device, const void* src_host, size_t bytes, hipStream_t stream) {
  if (bytes % 4 != 0) return fail(KFAC_ERR_INVALID, "internal: table size not a multiple of 4");
  const uint32_t* src = static_cast<const uint32_t*>(src_host);
  uint32_t* dst = static_cast<uint32_t*>(dst_device);
  size_t words = bytes / 4;
  for (size_t off = 0; off < words; off += 1000) {
    UploadChunk c;
    int n = static_cast<int>(words - off < 1000 ? words - off : 1000);
    std::memcpy(c.w, src + off, n * 4);
    KFAC_LAUNCH(K_UPLOAD, upload_kernel, dim3(1), dim3(256), 0, stream, dst + off, c, n);
    KFAC_CHECK_LAUNCH("upload_kernel");
  }
  return KFAC_OK;
}

kfac_status TableUpload::flush(hipStream_t stream) {
  // tables in carve order, none overlapping the next; runs of tables with gaps of at
  // most 1 KB between them go up as one image (the gaps written with zeros)
  for (size_t a = 1; a < parts_.size(); ++a)
    if (parts_[a].dst < parts_[a - 1].dst + parts_[a - 1].bytes)
      return fail(KFAC_ERR_INVALID, "internal: descriptor tables out of order");
  size_t a = 0;
  while (a < parts_.size()) {
    size_t b = a + 1;
    while (b < parts_.size() && parts_[b].dst - (parts_[b - 1].dst + parts_[b - 1].bytes) <= 1024) ++b;
    char* base = parts_[a].dst;
    const size_t end = static_cast<size_t>(parts_[b - 1].dst - base) + parts_[b - 1].bytes;
    if (end % 4 != 0) return fail(KFAC_ERR_INVALID, "internal: table size not a multiple of 4");
    std::vector<char> image(end, 0);
    for (size_t q = a; q < b; ++q) std::memcpy(image.data() + (parts_[q].dst - base), parts_[q].src, parts_[q].bytes);
    kfac_status st = upload(base, image.data(), end, stream);
    if (st) return st;
    a = b;
  }
  parts_.clear();
  return KFAC_OK;
}

// ---- timing ------------------------------------------------------------------
struct TimingRec {
  int id;
  hipEvent_t start, end;
};

struct TimingState {
  bool on = false;
  int only = -1;  // the one kernel id timed, or -1 for all
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  std::vector<TimingRec> recs;
  hipEvent_t next() {
    if (used == pool.size()) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      pool.push_back(e);
    }
    return pool[used++];
  }
};

static thread_local TimingState g_timing;

TimerScope::TimerScope(int id_, hipStream_t s)
    : id(id_), stream(s), on(g_timing.on && (g_timing.only < 0 || g_timing.only == id_)), ev_end(nullptr) {
  if (!on) return;
  hipEvent_t st = g_timing.next();
  ev_end = g_timing.next();
  if (!st || !ev_end) { on = false; return; }
  hipEventRecord(st, stream);
  g_timing.recs.push_back({id, st, ev_end});
}

TimerScope::~TimerScope() {
  if (on) hipEventRecord(ev_end, stream);
}

static const char* const kKernelNames[K_COUNT] = {
    "upload_kernel",      "syrk_tile_kernel",   "syrk_reduce_kernel", "pack_kernel",
    "unpack_kernel",      "inv_prep_kernel",    "inv_pivot_kernel",   "inv_panel_kernel",
    "inv_update_kernel",  "inv_finish_kernel",  "gemm_tn_kernel",     "bn_partial_kernel",
    "bn_finish_kernel",   "gemm_tn64_kernel",   "refine_elementwise_kernels",
    "refine_residual_gemm_tn64_kernel",         "refine_correction_gemm_tn_kernel",
    "shift_assemble_kernel"};

}  // namespace kfac

using namespace kfac;

extern "C" {

int32_t kfac_version(void) { return 100; }

const char* kfac_status_string(kfac_status s) {
  switch (s) {
    case KFAC_OK: return "ok";
    case KFAC_ERR_INVALID: return "invalid argument";
    case KFAC_ERR_UNSUPPORTED: return "unsupported device or dtype";
    case KFAC_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case KFAC_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* kfac_last_error(void) { return g_err; }

int32_t kfac_timing_kernels(void) { return K_COUNT; }

const char* kfac_kernel_name(int32_t id) {
  return (id >= 0 && id < K_COUNT) ? kKernelNames[id] : "";
}

kfac_status kfac_timing_enable(int32_t on) {
  g_timing.on = on != 0;
  return KFAC_OK;
}

kfac_status kfac_timing_only(int32_t id) {
  if (id < -1 || id >= K_COUNT) return fail(KFAC_ERR_INVALID, "kfac_timing_only: id %d out of range", id);
  g_timing.only = id;
  return KFAC_OK;
}

kfac_status kfac_timing_reset(void) {
  g_timing.recs.clear();
  g_timing.used = 0;
  return KFAC_OK;
}

kfac_status kfac_timing_read(int32_t id, double* total_ms, int64_t* launches) {
  if (id < 0 || id >= K_COUNT || !total_ms || !launches)
    return fail(KFAC_ERR_INVALID, "kfac_timing_read: bad id or NULL output");
  double sum = 0;
  int64_t n = 0;
  for (const TimingRec& r : g_timing.recs) {
    if (r.id != id) continue;
    KFAC_HIP(hipEventSynchronize(r.end));
    float ms = 0;
    KFAC_HIP(hipEventElapsedTime(&ms, r.start, r.end));
    sum += ms;
    ++n;
  }
  *total_ms = sum;
  *launches = n;
  return KFAC_OK;
}

}  // extern "C"
