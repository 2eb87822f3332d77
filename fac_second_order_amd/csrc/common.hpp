// Shared internals of libkfac: error reporting, device check, workspace carving,
// descriptor-table upload and per-kernel event timing. gfx950 (CDNA4) only.
#pragma once
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <vector>

#include "kfac.h"

namespace kfac {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

// ---- errors (thread-local text) -------------------------------------------
kfac_status fail(kfac_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
kfac_status hip_fail(hipError_t e, const char* what);
#define KFAC_HIP(call)                                   \
  do {                                                   \
    hipError_t e_ = (call);                              \
    if (e_ != hipSuccess) return ::kfac::hip_fail(e_, #call); \
  } while (0)

// Returns KFAC_OK when the current device is gfx950 (cached per device).
kfac_status check_device();

// ---- workspace carving ----------------------------------------------------
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* b = nullptr) : base(static_cast<char*>(b)) {}
  // Reserves `bytes` (256-byte aligned); returns nullptr when only sizing.
  template <class T>
  T* take(size_t count) {
    size_t off = used;
    used += align256(count * sizeof(T));
    return base ? reinterpret_cast<T*>(base + off) : nullptr;
  }
};

kfac_status check_workspace(const void* ws, size_t ws_bytes, size_t need);

// ---- descriptor tables ----------------------------------------------------
// Copies a host table into device memory by kernel arguments (2 KB per launch):
// stream-ordered, needs no pinned host memory and keeps no host pointer.
kfac_status upload(void* dst_device, const void* src_host, size_t bytes, hipStream_t stream);

// The descriptor tables of one call, carved one after another from the workspace,
// sent as one image (the alignment gaps between them are written with zeros), so a
// call pays for as few upload launches as its total table size needs.
class TableUpload {
 public:
  void add(void* dst_device, const void* src_host, size_t bytes) {
    if (bytes) parts_.push_back({static_cast<char*>(dst_device), static_cast<const char*>(src_host), bytes});
  }
  kfac_status flush(hipStream_t stream);

 private:
  struct Part {
    char* dst;
    const char* src;
    size_t bytes;
  };
  std::vector<Part> parts_;
};

// ---- per-kernel timing ----------------------------------------------------
enum KernelId {
  K_UPLOAD = 0,
  K_SYRK,
  K_SYRK_REDUCE,
  K_PACK,
  K_UNPACK,
  K_INV_PREP,
  K_INV_PIVOT,
  K_INV_PANEL,
  K_INV_UPDATE,
  K_INV_FINISH,
  K_GEMM,
  K_BN_PARTIAL,
  K_BN_FINISH,
  K_GEMM64,        // gemm_tn64_kernel of the preconditioning (fp64 sums)
  K_REFINE_EW,     // refine_init_kernel and refine_apply_kernel
  K_REFINE_RES,    // gemm_tn64_kernel forming the residual of the refinement
  K_REFINE_CORR,   // gemm_tn_kernel forming the correction of the refinement
  K_SHIFT_ASM,     // shift_assemble_kernel (3x3 activation factors from shift products)
  K_COUNT
};

// Records a start/end event pair around a launch when timing is enabled on the
// calling thread; a no-op otherwise.
struct TimerScope {
  int id;
  hipStream_t stream;
  bool on;
  hipEvent_t ev_end;
  TimerScope(int id_, hipStream_t s);
  ~TimerScope();
};

#define KFAC_LAUNCH(id, kernel, grid, block, shmem, stream, ...)                 \
  do {                                                                         \
    ::kfac::TimerScope ts_(id, stream);                                        \
    hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);       \
  } while (0)

#define KFAC_CHECK_LAUNCH(what)                                   \
  do {                                                            \
    hipError_t e_ = hipGetLastError();                            \
    if (e_ != hipSuccess) return ::kfac::hip_fail(e_, what);      \
  } while (0)

// ---- global address space -----------------------------------------------------
// Pointers read from descriptor tables are generic; casting them to the global
// address space makes the compiler emit global_* instead of flat_* accesses, whose
// completion is tracked apart from LDS (flat loads would also hold LDS waits).
#define KG __attribute__((address_space(1)))
template <class T>
__device__ __forceinline__ const KG T* gp(const T* p) {
  return (const KG T*)(p);
}
template <class T>
__device__ __forceinline__ KG T* gp(T* p) {
  return (KG T*)(p);
}

// ---- small device helpers --------------------------------------------------
// Maps a hardware block id to a virtual work id so that XCD x (blocks b with
// b % 8 == x, the order in which the dispatcher deals blocks to the 8 XCDs) runs the
// contiguous range [x*per, (x+1)*per) and work items that share operands share that
// XCD's L2. The grid is a multiple of 8; returns -1 for padding. Only for launches
// whose work items cost about the same.
__device__ inline int xcd_virtual(int b, int grid, int total) {
  const int per = grid / 8;
  const int v = (b % 8) * per + b / 8;
  return v < total ? v : -1;
}
inline unsigned xcd_grid(int64_t total) { return static_cast<unsigned>((total + 7) / 8 * 8); }

// Work items split into 8 contiguous segments, one per XCD, chosen by the host so
// that the segments cost about the same (they differ in item count). Block b runs
// on XCD b % 8 and takes that segment's item b / 8; a block past its segment's end
// gets -1. Launch 8 * (longest segment) blocks.
struct XcdSegs {
  int32_t begin[8];
  int32_t len[8];
};
__device__ inline int seg_item(int b, const XcdSegs& sg) {
  const int x = b & 7, slot = b >> 3;
  return slot < sg.len[x] ? sg.begin[x] + slot : -1;
}

// Index of the problem owning work item `w`: largest p with begin[p] <= w.
__device__ inline int find_problem(const int32_t* begin, int count, int w) {
  int lo = 0, hi = count - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (begin[mid] <= w) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Upper-triangle tile t (row-major over i <= j) of an nb x nb tile grid. Row i starts
// at S(i) = i*nb - i(i-1)/2; the row is the root of S(i) = t (a float estimate, exact to
// within a few rows for any grid of fewer than 2^12 blocks per side), then corrected.
__device__ inline void upper_tile(int t, int nb, int& ti, int& tj) {
  const float b = 2.f * static_cast<float>(nb) + 1.f;
  int i = static_cast<int>((b - sqrtf(fmaxf(b * b - 8.f * static_cast<float>(t), 0.f))) * 0.5f);
  i = max(0, min(i, nb - 1));
  auto row_start = [nb](int r) { return r * nb - (r * (r - 1)) / 2; };
  while (i > 0 && row_start(i) > t) --i;
  while (i + 1 < nb && row_start(i + 1) <= t) ++i;
  ti = i;
  tj = i + (t - row_start(i));
}

// Offset of (i, j), i <= j, in the row-by-row upper-triangle packing of order n.
__host__ __device__ inline int64_t packed_off(int64_t i, int64_t j, int64_t n) {
  return i * n - (i * (i - 1)) / 2 + (j - i);
}

}  // namespace kfac
