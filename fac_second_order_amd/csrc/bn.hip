// BatchNorm diagonal Fisher for all BN layers in two launches.
// Osawa et al. (CVPR 2019), Section 1 contributions: BatchNorm's Fisher is taken
// diagonal; the diagonal is that of the empirical Fisher of Section 3.1, eq. (3),
// over the per-sample gradients of gamma and beta.
//
// Stage 1 (bn_partial_kernel) streams x-hat and the output gradient once from HBM
// with 16-byte loads along the channel dimension (NHWC, channels contiguous). A work
// item is (layer, sample, spatial chunk, channel block); it writes the chunk's
// per-channel partial sums (sum g*x, sum g) to the workspace.
// Stage 2 (bn_finish_kernel), 8 lanes per channel over the samples, adds the chunks
// of each sample in a fixed order (deterministic), squares the per-sample sums,
// averages over samples, blends with the stored Fisher when asked and divides; with
// parameters given it also applies the update of eq. (8), gamma/beta -= lr * precond.
#include <mutex>

#include "common.hpp"

namespace kfac {

struct BnDesc {
  const void* xhat;
  const void* gout;
  float* fisher;
  float* precond;
  v2f* partial;     // [n][nchunk][c] (sum g*x, sum g)
  float* params;    // [2][c] gamma, beta updated in place, or NULL
  float lr;
  int32_t n, hw, c;
  int32_t vl;       // vector lanes per row segment (<= 256)
  int32_t rowpar;   // rows processed side by side (256 / vl)
  int32_t cblocks;  // channel blocks of vl*ev channels
  int32_t rows_per_chunk, nchunk;
  int32_t vec;      // 1: 16-byte vectors along channels
  int32_t pad_;
};

template <class T>
struct Vec16;
template <>
struct Vec16<_Float16> {
  static constexpr int ev = 8;
};
template <>
struct Vec16<float> {
  static constexpr int ev = 4;
};

template <class T, int EV>
__device__ inline void load_vec(const T* p, float* out) {
  if constexpr (EV == 1) {
    out[0] = static_cast<float>(gp(p)[0]);
  } else if constexpr (sizeof(T) == 2) {
    v8h v = *reinterpret_cast<const KG v8h*>(gp(p));
#pragma unroll
    for (int q = 0; q < 8; ++q) out[q] = static_cast<float>(v[q]);
  } else {
    v4f v = *reinterpret_cast<const KG v4f*>(gp(p));
#pragma unroll
    for (int q = 0; q < 4; ++q) out[q] = v[q];
  }
}

template <class T, int EV>
__device__ void bn_partial_body(const BnDesc& d, int item) {
  // item -> (sample, chunk, channel block)
  const int cb = item % d.cblocks;
  const int rest = item / d.cblocks;
  const int chunk = rest % d.nchunk;
  const int s = rest / d.nchunk;
  const int lane = threadIdx.x % d.vl;
  const int rp = threadIdx.x / d.vl;
  const int c0 = cb * d.vl * EV + lane * EV;
  const int r_begin = chunk * d.rows_per_chunk;
  const int r_end = min(d.hw, r_begin + d.rows_per_chunk);
  float sg[EV], sb[EV];
#pragma unroll
  for (int q = 0; q < EV; ++q) sg[q] = sb[q] = 0.f;
  const bool active = rp < d.rowpar && c0 < d.c;
  if (active) {
    const T* X = static_cast<const T*>(d.xhat) + (int64_t(s) * d.hw) * d.c + c0;
    const T* G = static_cast<const T*>(d.gout) + (int64_t(s) * d.hw) * d.c + c0;
    // four rows' loads in flight before their sums; rows are still added in order
    constexpr int U = 4;
    int r = r_begin + rp;
    for (; r + (U - 1) * d.rowpar < r_end; r += U * d.rowpar) {
      float x[U][EV], g[U][EV];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        load_vec<T, EV>(X + int64_t(r + u * d.rowpar) * d.c, x[u]);
        load_vec<T, EV>(G + int64_t(r + u * d.rowpar) * d.c, g[u]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int q = 0; q < EV; ++q) {
          sg[q] = fmaf(g[u][q], x[u][q], sg[q]);
          sb[q] += g[u][q];
        }
    }
    for (; r < r_end; r += d.rowpar) {
      float x[EV], g[EV];
      load_vec<T, EV>(X + int64_t(r) * d.c, x);
      load_vec<T, EV>(G + int64_t(r) * d.c, g);
#pragma unroll
      for (int q = 0; q < EV; ++q) {
        sg[q] = fmaf(g[q], x[q], sg[q]);
        sb[q] += g[q];
      }
    }
  }
  // reduce the rowpar partial rows that share a channel through LDS
  __shared__ float2 red[256 * 8];
#pragma unroll
  for (int q = 0; q < EV; ++q) red[threadIdx.x * EV + q] = make_float2(sg[q], sb[q]);
  __syncthreads();
  const int width = d.vl * EV;  // channels in this block
  for (int ch = threadIdx.x; ch < width; ch += blockDim.x) {
    const int c = cb * width + ch;
    if (c >= d.c) continue;
    const int l = ch / EV, q = ch % EV;
    float a = 0.f, b = 0.f;
    for (int r = 0; r < d.rowpar; ++r) {
      float2 v = red[(r * d.vl + l) * EV + q];
      a += v.x;
      b += v.y;
    }
    gp(d.partial)[(int64_t(s) * d.nchunk + chunk) * d.c + c] = v2f{a, b};
  }
}

__global__ void __launch_bounds__(256) bn_partial_kernel(const BnDesc* __restrict__ desc,
                                                         const int32_t* __restrict__ begin,
                                                         int count, int f32) {
  const int p = find_problem(begin, count, blockIdx.x);
  const BnDesc d = desc[p];
  const int item = blockIdx.x - begin[p];
  if (f32) {
    if (d.vec) bn_partial_body<float, 4>(d, item);
    else bn_partial_body<float, 1>(d, item);
  } else {
    if (d.vec) bn_partial_body<_Float16, 8>(d, item);
    else bn_partial_body<_Float16, 1>(d, item);
  }
}

// One block per 32 channels of a layer; 8 lanes per channel split the samples. Each
// lane forms the per-sample sums s_n (chunks added in order) and accumulates s_n^2 and
// s_n; the 8 lanes are then added in a fixed order, so the result is deterministic.
constexpr int FIN_CH = 32, FIN_LANES = 8;

__global__ void __launch_bounds__(256) bn_finish_kernel(const BnDesc* __restrict__ desc,
                                                        const int32_t* __restrict__ gbegin,
                                                        int count, float decay, float shift) {
  const int p = find_problem(gbegin, count, blockIdx.x);
  const BnDesc d = desc[p];
  const int c = (blockIdx.x - gbegin[p]) * FIN_CH + (threadIdx.x % FIN_CH);
  const int q = threadIdx.x / FIN_CH;
  float fg = 0.f, fb = 0.f, gg = 0.f, gb = 0.f;
  if (c < d.c) {
    // this lane's (sample, chunk) pairs in order, samples q, q + 8, ..., eight loads
    // in flight; a sample's chunks are added in chunk order
    const int total = (d.n - q + FIN_LANES - 1) / FIN_LANES * d.nchunk;
    float a = 0.f, b = 0.f;
    int k = 0;
    for (int base = 0; base < total; base += 8) {
      v2f v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int idx = base + u;
        const int s = q + FIN_LANES * (idx / d.nchunk), kk = idx % d.nchunk;
        v[u] = idx < total ? gp(d.partial)[(int64_t(s) * d.nchunk + kk) * d.c + c] : v2f{0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (base + u >= total) break;
        a += v[u].x;
        b += v[u].y;
        if (++k == d.nchunk) {
          fg = fmaf(a, a, fg);
          fb = fmaf(b, b, fb);
          gg += a;
          gb += b;
          a = b = 0.f;
          k = 0;
        }
      }
    }
  }
  __shared__ float4 red[256];
  red[threadIdx.x] = make_float4(fg, fb, gg, gb);
  __syncthreads();
  if (q != 0 || c >= d.c) return;
  for (int l = 1; l < FIN_LANES; ++l) {
    const float4 v = red[l * FIN_CH + threadIdx.x];
    fg += v.x; fb += v.y; gg += v.z; gb += v.w;
  }
  const float inv_n = 1.0f / static_cast<float>(d.n);
  fg *= inv_n;
  fb *= inv_n;
  gg *= inv_n;
  gb *= inv_n;
  if (decay != 0.f) {
    fg = decay * gp(d.fisher)[c] + (1.f - decay) * fg;
    fb = decay * gp(d.fisher)[d.c + c] + (1.f - decay) * fb;
  }
  gp(d.fisher)[c] = fg;
  gp(d.fisher)[d.c + c] = fb;
  const float pg = gg / (fg + shift), pb = gb / (fb + shift);
  gp(d.precond)[c] = pg;
  gp(d.precond)[d.c + c] = pb;
  if (d.params) {
    gp(d.params)[c] = fmaf(-d.lr, pg, gp(d.params)[c]);
    gp(d.params)[d.c + c] = fmaf(-d.lr, pb, gp(d.params)[d.c + c]);
  }
}

// Plans one layer: 16-byte vectors along channels when `vec`, else scalar loads.
static BnDesc plan_layer(const kfac_bn& L, int esize, bool vec) {
  BnDesc d{};
  d.n = L.n;
  d.hw = L.hw;
  d.c = L.c;
  const int ev_full = 16 / esize;
  d.vec = (vec && d.c % ev_full == 0) ? 1 : 0;
  const int ev = d.vec ? ev_full : 1;
  const int groups = (d.c + ev - 1) / ev;
  d.vl = groups < 256 ? groups : 256;
  d.rowpar = 256 / d.vl;
  d.cblocks = (groups + d.vl - 1) / d.vl;
  const int64_t row_bytes = int64_t(d.vl) * ev * esize;
  int64_t rpc = (128 * 1024) / row_bytes;  // about 128 KB of each tensor per work item
  if (rpc < d.rowpar) rpc = d.rowpar;
  rpc = (rpc / d.rowpar) * d.rowpar;
  if (rpc > d.hw) rpc = d.hw;
  d.rows_per_chunk = static_cast<int32_t>(rpc);
  d.nchunk = static_cast<int32_t>((d.hw + rpc - 1) / rpc);
  return d;
}

static size_t partial_count(const BnDesc& d) { return size_t(d.n) * d.nchunk * d.c; }

// Workspace: descriptors, two offset tables, then the partial sums. The bound takes
// the larger partial buffer of the vector and scalar plans of each layer for either
// input dtype, so any alignment seen at call time fits.
static size_t bn_ws_bound(const kfac_bn* L, int count) {
  size_t part = 0;
  for (int l = 0; l < count; ++l) {
    size_t m = 0;
    for (int esize : {2, 4})
      for (bool vec : {true, false}) {
        size_t c = partial_count(plan_layer(L[l], esize, vec));
        m = c > m ? c : m;
      }
    part += m;
  }
  return align256(sizeof(BnDesc) * count) + 2 * align256(sizeof(int32_t) * count) +
         align256(sizeof(v2f) * part);
}

}  // namespace kfac

using namespace kfac;

static kfac_status bn_validate(const kfac_bn* L, int32_t count, kfac_dtype dt) {
  if (count < 0) return fail(KFAC_ERR_INVALID, "count must be >= 0");
  if (count > 0 && !L) return fail(KFAC_ERR_INVALID, "layers is NULL");
  if (dt != KFAC_F16 && dt != KFAC_F32) return fail(KFAC_ERR_UNSUPPORTED, "dtype %d not supported", dt);
  for (int l = 0; l < count; ++l) {
    if (L[l].n < 1 || L[l].hw < 1 || L[l].c < 1)
      return fail(KFAC_ERR_INVALID, "bn layer %d: n, hw, c must be >= 1", l);
    if (int64_t(L[l].n) * L[l].hw * L[l].c >= (int64_t(1) << 40))
      return fail(KFAC_ERR_INVALID, "bn layer %d too large", l);
  }
  return KFAC_OK;
}

extern "C" kfac_status kfac_bn_diag_workspace(const kfac_bn* layers, int32_t count, size_t* bytes) {
  if (!bytes) return fail(KFAC_ERR_INVALID, "bytes is NULL");
  kfac_status st = bn_validate(layers, count, KFAC_F16);
  if (st) return st;
  *bytes = count ? bn_ws_bound(layers, count) : 0;
  return KFAC_OK;
}

// A validated call: per layer its plan with the caller's pointers, and the number of
// partial-sum pairs it needs.
struct BnCall {
  std::vector<BnDesc> desc;
  std::vector<size_t> part;
  int f32 = 0;
};

// Workspace of the layers [l0, l1) of a call: descriptors, two offset tables, partials.
static size_t bn_need(const BnCall& c, int l0, int l1) {
  size_t part = 0;
  for (int l = l0; l < l1; ++l) part += c.part[l];
  const int k = l1 - l0;
  return align256(sizeof(BnDesc) * k) + 2 * align256(sizeof(int32_t) * k) + align256(sizeof(v2f) * part);
}

// Argument checks and plans (nothing enqueued). kfac_bn_diag, and with params the
// update of eq. (8).
static kfac_status bn_prepare(const kfac_bn* layers, int32_t count, kfac_dtype in_dtype, const void* const* xhat,
                              const void* const* gout, float* const* fisher, float* const* precond,
                              float* const* params, float lr, float ema_decay, float shift, BnCall& call) {
  kfac_status st = bn_validate(layers, count, in_dtype);
  if (st) return st;
  if (params && !(lr - lr == 0.f)) return fail(KFAC_ERR_INVALID, "lr must be finite");
  if (!(ema_decay >= 0.f && ema_decay <= 1.f)) return fail(KFAC_ERR_INVALID, "ema_decay must be in [0, 1]");
  if (!(shift == shift)) return fail(KFAC_ERR_INVALID, "shift is NaN");
  if (count == 0) return KFAC_OK;
  if (!xhat || !gout || !fisher || !precond) return fail(KFAC_ERR_INVALID, "NULL pointer array");
  const int esize = in_dtype == KFAC_F16 ? 2 : 4;
  call.f32 = in_dtype == KFAC_F32 ? 1 : 0;
  call.desc.resize(count);
  call.part.resize(count);
  for (int l = 0; l < count; ++l) {
    if (!xhat[l] || !gout[l] || !fisher[l] || !precond[l] || (params && !params[l]))
      return fail(KFAC_ERR_INVALID, "bn layer %d: NULL pointer", l);
    if (params && (reinterpret_cast<uintptr_t>(params[l]) & 3))
      return fail(KFAC_ERR_INVALID, "bn layer %d: misaligned pointer", l);
    if (params && (params[l] == precond[l] || params[l] == fisher[l]))
      return fail(KFAC_ERR_INVALID, "bn layer %d: params overlaps fisher or precond", l);
    const uintptr_t a = reinterpret_cast<uintptr_t>(xhat[l]) | reinterpret_cast<uintptr_t>(gout[l]);
    if (a % esize || (reinterpret_cast<uintptr_t>(fisher[l]) | reinterpret_cast<uintptr_t>(precond[l])) & 3)
      return fail(KFAC_ERR_INVALID, "bn layer %d: misaligned pointer", l);
    BnDesc& d = call.desc[l];
    d = plan_layer(layers[l], esize, a % 16 == 0);
    d.xhat = xhat[l];
    d.gout = gout[l];
    d.fisher = fisher[l];
    d.precond = precond[l];
    d.params = params ? params[l] : nullptr;
    d.lr = lr;
    call.part[l] = partial_count(d);
  }
  return KFAC_OK;
}

// Enqueues layers [l0, l1) of a call with their tables and partial sums carved from
// `ws` (at least bn_need bytes): one table upload, the partial and the finish launch.
static kfac_status bn_launch(BnCall& c, int l0, int l1, void* ws, float ema_decay, float shift, hipStream_t s) {
  const int count = l1 - l0;
  std::vector<int32_t> begin(count), cbegin(count);
  int64_t items = 0, channels = 0;
  for (int l = 0; l < count; ++l) {
    const BnDesc& d = c.desc[l0 + l];
    begin[l] = static_cast<int32_t>(items);
    items += int64_t(d.n) * d.nchunk * d.cblocks;
    cbegin[l] = static_cast<int32_t>(channels);
    channels += (d.c + FIN_CH - 1) / FIN_CH;  // finish blocks
  }
  if (items >= (int64_t(1) << 31) || channels >= (int64_t(1) << 31))
    return fail(KFAC_ERR_INVALID, "bn problem too large");
  Carver cv(ws);
  BnDesc* d_desc = cv.take<BnDesc>(count);
  int32_t* d_begin = cv.take<int32_t>(count);
  int32_t* d_cbegin = cv.take<int32_t>(count);
  size_t part = 0;
  for (int l = l0; l < l1; ++l) part += c.part[l];
  v2f* partial = cv.take<v2f>(part);
  size_t off = 0;
  for (int l = l0; l < l1; ++l) {
    c.desc[l].partial = partial + off;
    off += c.part[l];
  }
  TableUpload tu;
  tu.add(d_desc, c.desc.data() + l0, sizeof(BnDesc) * count);
  tu.add(d_begin, begin.data(), sizeof(int32_t) * count);
  tu.add(d_cbegin, cbegin.data(), sizeof(int32_t) * count);
  kfac_status st = tu.flush(s);
  if (st) return st;
  KFAC_LAUNCH(K_BN_PARTIAL, bn_partial_kernel, dim3(static_cast<unsigned>(items)), dim3(256), 0, s,
              d_desc, d_begin, count, c.f32);
  KFAC_CHECK_LAUNCH("bn_partial_kernel");
  KFAC_LAUNCH(K_BN_FINISH, bn_finish_kernel, dim3(static_cast<unsigned>(channels)), dim3(256), 0, s, d_desc,
              d_cbegin, count, ema_decay, shift);
  KFAC_CHECK_LAUNCH("bn_finish_kernel");
  return KFAC_OK;
}

static kfac_status bn_impl(const kfac_bn* layers, int32_t count, kfac_dtype in_dtype, const void* const* xhat,
                           const void* const* gout, float* const* fisher, float* const* precond,
                           float* const* params, float lr, float ema_decay, float shift, void* workspace,
                           size_t ws_bytes, void* stream) {
  BnCall call;
  kfac_status st = bn_prepare(layers, count, in_dtype, xhat, gout, fisher, precond, params, lr, ema_decay, shift,
                              call);
  if (st || count == 0) return st;
  st = check_device();
  if (st) return st;
  st = check_workspace(workspace, ws_bytes, bn_need(call, 0, count));
  if (st) return st;
  return bn_launch(call, 0, count, workspace, ema_decay, shift, static_cast<hipStream_t>(stream));
}

// ---- the variant that allocates nothing -------------------------------------------
// Its scratch (tables and partial sums) is this file-scope device array, one copy per
// GPU, held until the process ends. Its device address is looked up once per device
// (hipGetSymbolAddress with that device current) and only that address is used from
// the host. A call whose layers need more than the array holds runs in passes of
// consecutive layers, each pass reusing the array after the previous pass's kernels
// (stream order). Every partial sum a finish block reads was written by the partial
// launch of its own pass, so nothing needs clearing between calls.
constexpr size_t kBnScratchBytes = KFAC_BN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kBnScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64];

static kfac_status scratch_address(void** out) {
  int dev = 0;
  KFAC_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return fail(KFAC_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    KFAC_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(KFAC_ERR_HIP, "hipGetSymbolAddress returned NULL for the BN scratch");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KFAC_OK;
}

extern "C" kfac_status kfac_bn_diag(const kfac_bn* layers, int32_t count, kfac_dtype in_dtype,
                                    const void* const* xhat, const void* const* gout,
                                    float* const* fisher, float* const* precond, float ema_decay,
                                    float shift, void* workspace, size_t ws_bytes, void* stream) {
  return bn_impl(layers, count, in_dtype, xhat, gout, fisher, precond, nullptr, 0.f, ema_decay, shift, workspace,
                 ws_bytes, stream);
}

extern "C" kfac_status kfac_bn_update(const kfac_bn* layers, int32_t count, kfac_dtype in_dtype,
                                      const void* const* xhat, const void* const* gout,
                                      float* const* fisher, float* const* precond, float* const* params,
                                      float lr, float ema_decay, float shift, void* workspace, size_t ws_bytes,
                                      void* stream) {
  if (count > 0 && !params) return fail(KFAC_ERR_INVALID, "NULL parameter array");
  return bn_impl(layers, count, in_dtype, xhat, gout, fisher, precond, params, lr, ema_decay, shift, workspace,
                 ws_bytes, stream);
}

extern "C" kfac_status kfac_bn_diag_noalloc(const kfac_bn* layers, int32_t count, kfac_dtype in_dtype,
                                            const void* const* xhat, const void* const* gout,
                                            float* const* fisher, float* const* precond, float* const* params,
                                            float lr, float ema_decay, float shift, void* stream) {
  BnCall call;
  kfac_status st = bn_prepare(layers, count, in_dtype, xhat, gout, fisher, precond, params, lr, ema_decay, shift,
                              call);
  if (st || count == 0) return st;
  for (int l = 0; l < count; ++l)
    if (bn_need(call, l, l + 1) > kBnScratchBytes)
      return fail(KFAC_ERR_INVALID,
                  "kfac_bn_diag_noalloc: bn layer %d needs %zu bytes of scratch, more than the %zu of the "
                  "static buffer (use kfac_bn_diag with a workspace)",
                  l, bn_need(call, l, l + 1), kBnScratchBytes);
  st = check_device();
  if (st) return st;
  void* ws = nullptr;
  if ((st = scratch_address(&ws))) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  int l0 = 0;
  while (l0 < count) {  // the longest run of layers from l0 that fits
    int l1 = l0 + 1;
    while (l1 < count && bn_need(call, l0, l1 + 1) <= kBnScratchBytes) ++l1;
    if ((st = bn_launch(call, l0, l1, ws, ema_decay, shift, s))) return st;
    l0 = l1;
  }
  return KFAC_OK;
}
