// Tile engine on fp32 operands: a 512-thread block accumulates a 128x128 fp32 tile
// C[m][n] += sum_k A[k][m] * B[k][n] with both operands read as rows of k
// ("A^T B" form). While the MFMAs work on one staged chunk of k out of one LDS buffer,
// the global loads of the next two chunks are in flight in registers, and the next
// chunk then lands in the other LDS buffer, so there is one barrier per chunk. Eight
// waves share the tile, wave w owning rows 32*(w/2) .. +32 and columns 64*(w%2) .. +64
// (two 32x32 MFMA blocks); two blocks per compute unit give every SIMD four waves, so
// the tile load and store of one block overlap the other block's MFMAs.
//
// The fp32 product (oct_gemm) runs on bf16 MFMA with exactly split operands (below);
// the fp32 staging (oct_fetch, oct_stage: chunks of 32 fp32 values of k) feeds the
// fp64 engine.
//
// Accumulator layout (v_mfma_f32_32x32x16_bf16 and v_mfma_f32_32x32x2f32, wave64):
// register e of lane l holds row 8*(e/4) + 4*(l/32) + e%4, column l%32 of the 32x32
// block.
#pragma once
#include "common.hpp"

namespace kfac {

constexpr int TB = 128;       // tile edge
constexpr int KT = 32;        // k per LDS chunk
constexpr int LDP = TB + 4;   // LDS pitch of staged chunks [k][m] (floats, 16-byte rows)
constexpr int LDT = TB + 1;   // pitch of full 128x128 LDS tiles used outside the engine
constexpr int CHUNK = KT * LDP;  // floats per staged operand chunk

// One operand read as rows: element (k, m) of the logical [K][M] operand is
// src[k*ld + m]. Columns m0.. of the tile; valid k < kv, m < mv.
struct Operand {
  const void* src;
  int64_t ld;
  int kv, m0, mv;
};

__device__ inline Operand op_rows(const float* src, int64_t ld, int kv, int m0, int mv) {
  return Operand{src, ld, kv, m0, mv};
}
__device__ inline Operand op_rows_h(const _Float16* src, int64_t ld, int kv, int m0, int mv) {
  return Operand{src, ld, kv, m0, mv};
}

// Load forms of an operand: 16-byte groups (fp32 rows on a 4-byte aligned base, m0 %
// 4 == 0; a group may run past a row's end into the next row, or past the buffer's
// range, which a raw buffer load reads as zeros dword by dword), single fp32 values,
// single fp16 values.
constexpr int LD_V4 = 0, LD_F32 = 1, LD_F16 = 2;

// Raw buffer over rows [0, kv) of a rows-form operand (callers guarantee that
// kv * ld * element size < 2^31). The base and size are made wave-uniform explicitly
// so that the resource lives in scalar registers.
template <int MODE>
__device__ inline __amdgpu_buffer_rsrc_t op_rsrc(const Operand& o) {
  constexpr uint32_t es = MODE == LD_F16 ? 2u : 4u;
  const uint64_t a = reinterpret_cast<uint64_t>(o.src);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  const uint32_t bytes = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(o.kv) * static_cast<uint32_t>(o.ld) * es);
  void* base = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, 0x00020000);
}

// ---- the engine ------------------------------------------------------------
struct Oct {
  v16f c[2];
};

__device__ inline void oct_zero(Oct& o) {
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) o.c[b][e] = 0.f;
}

__device__ inline int oct_row(int lane, int e) {
  return 32 * ((threadIdx.x >> 6) >> 1) + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
}
__device__ inline int oct_col(int lane, int b) { return 64 * ((threadIdx.x >> 6) & 1) + 32 * b + (lane & 31); }

// Tile <-> global (row-major, leading dimension ld), rows < rvalid, cols < cvalid.
__device__ inline void oct_load(Oct& o, const float* src, int64_t ld, int rvalid, int cvalid) {
  const int lane = threadIdx.x & 63;
  if (rvalid >= TB && cvalid >= TB) {
    const KG float* s = gp(src) + int64_t(oct_row(lane, 0)) * ld + oct_col(lane, 0);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) o.c[b][e] = s[int64_t(8 * (e >> 2) + (e & 3)) * ld + 32 * b];
    return;
  }
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = oct_row(lane, e), c = oct_col(lane, b);
      o.c[b][e] = (r < rvalid && c < cvalid) ? gp(src)[int64_t(r) * ld + c] : 0.f;
    }
}

__device__ inline void oct_store(const Oct& o, float* dst, int64_t ld, int rvalid, int cvalid) {
  const int lane = threadIdx.x & 63;
  if (rvalid >= TB && cvalid >= TB) {
    KG float* d = gp(dst) + int64_t(oct_row(lane, 0)) * ld + oct_col(lane, 0);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) d[int64_t(8 * (e >> 2) + (e & 3)) * ld + 32 * b] = o.c[b][e];
    return;
  }
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = oct_row(lane, e), c = oct_col(lane, b);
      if (r < rvalid && c < cvalid) gp(dst)[int64_t(r) * ld + c] = o.c[b][e];
    }
}

// dst += alpha * tile (row-major, leading dimension ld), rows < rvalid, cols < cvalid.
__device__ inline void oct_axpy(const Oct& o, float* dst, int64_t ld, int rvalid, int cvalid, float alpha) {
  const int lane = threadIdx.x & 63;
  if (rvalid >= TB && cvalid >= TB) {
    // Full tile: all 32 reads in flight before the first write.
    KG float* d = gp(dst) + int64_t(oct_row(lane, 0)) * ld + oct_col(lane, 0);
    float v[2][16];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) v[b][e] = d[int64_t(8 * (e >> 2) + (e & 3)) * ld + 32 * b];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) d[int64_t(8 * (e >> 2) + (e & 3)) * ld + 32 * b] = fmaf(alpha, o.c[b][e], v[b][e]);
    return;
  }
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = oct_row(lane, e), c = oct_col(lane, b);
      if (r < rvalid && c < cvalid) {
        KG float* x = gp(dst) + int64_t(r) * ld + c;
        *x = fmaf(alpha, o.c[b][e], *x);
      }
    }
}

// Transposed store through LDS (coalesced): dst[c*ld + r] = tile[r][c] for r < rvalid,
// c < cvalid. lds needs TB*LDT floats; ends with a barrier.
__device__ inline void oct_store_t(const Oct& o, float* dst, int64_t ld, int rvalid, int cvalid, float* lds) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) lds[oct_col(lane, b) * LDT + oct_row(lane, e)] = o.c[b][e];
  __syncthreads();
  for (int e = threadIdx.x; e < TB * TB; e += 512) {
    const int c = e / TB, r = e % TB;  // output row c, column r: contiguous in r
    if (r < rvalid && c < cvalid) gp(dst)[int64_t(c) * ld + r] = lds[c * LDT + r];
  }
  __syncthreads();
}

// Staging: thread (kg = tid/32, mg = tid%32) loads k = 2kg, 2kg+1 and m = 4mg..4mg+3
// of a chunk, branch-free through a raw buffer in the load form MODE: every load is
// issued, and one outside the operand (k >= kv or m >= mv) gets an offset past the
// buffer's range, for which it returns zeros without touching memory. With the same
// loads on every path, the wait before an LDS store covers only its own chunk. LD_V4
// reads each 4-group that starts below mv whole: its entries at or past mv (row
// padding, the next row's first entries, or zeros past the buffer's range) reach only
// output rows or columns >= mv, which callers never store.
template <int MODE = LD_V4>
__device__ inline void oct_fetch(const Operand& o, __amdgpu_buffer_rsrc_t rs, int k0, float4 (&r)[2]) {
  const int kg = threadIdx.x >> 5, mg = threadIdx.x & 31;
  const int m = o.m0 + 4 * mg;
  const int ld = static_cast<int>(o.ld);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int k = k0 + 2 * kg + q;
    const bool rok = k < o.kv;
    if constexpr (MODE == LD_V4) {
      const unsigned off = static_cast<unsigned>(k * ld + m) * 4u;
      const v4u x = __builtin_amdgcn_raw_buffer_load_b128(rs, (rok & (m < o.mv)) ? off : 0x80000000u, 0, 0);
      const v4f f = __builtin_bit_cast(v4f, x);
      r[q] = make_float4(f.x, f.y, f.z, f.w);
    } else {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool ok = rok & (m + u < o.mv);
        if constexpr (MODE == LD_F32) {
          const unsigned off = static_cast<unsigned>(k * ld + m + u) * 4u;
          v[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, ok ? off : 0x80000000u, 0, 0));
        } else {
          const unsigned off = static_cast<unsigned>(k * ld + m + u) * 2u;
          const unsigned short h = __builtin_amdgcn_raw_buffer_load_b16(rs, ok ? off : 0x80000000u, 0, 0);
          v[u] = static_cast<float>(__builtin_bit_cast(_Float16, h));
        }
      }
      r[q] = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

__device__ inline void oct_stage(float* lds, const float4 (&r)[2]) {
  const int kg = threadIdx.x >> 5, mg = threadIdx.x & 31;
#pragma unroll
  for (int q = 0; q < 2; ++q) *reinterpret_cast<float4*>(lds + (2 * kg + q) * LDP + 4 * mg) = r[q];
}

// ---- the bf16x3 product ------------------------------------------------------
// Every fp32 operand value x is split exactly into three bf16 parts, x = x0 + x1 + x2:
// x0 = x rounded to bf16 (8 significant bits), x1 = the remainder rounded the same
// way, x2 = what is left, which has at most 8 significant bits and so is a bf16 value
// itself (round to nearest leaves each remainder at most half a unit of the last
// place kept). A product a*b is then formed from the six partial products
// a0b0 + a0b1 + a1b0 + a0b2 + a1b1 + a2b0 on v_mfma_f32_32x32x16_bf16 with fp32 sums;
// the three dropped ones (a1b2, a2b1, a2b2) are each at most 2^-24 |ab|, the size of
// an fp32 rounding, so the result carries fp32 accuracy. bf16 MFMA has 16 times the
// flop rate of fp32 MFMA; with six products per multiply that leaves about 2.7 times
// the throughput of v_mfma_f32_32x32x2f32.
//
// Staging: K is consumed in chunks of XK = 16. Thread (kr = tid/32, mg = tid%32) loads
// k = kr, m = 4mg..4mg+3 of each operand (one 16-byte group or four single values,
// branch-free as in oct_fetch), splits the four values and writes each part to its own
// LDS plane [k][m] of bf16, one 8-byte store per plane. The 8-byte groups of a plane
// row are XOR-swizzled by (k % 4) * 8 so that the transposing reads below hit 32
// distinct bank pairs per half wave. Double-buffered planes take 48 KB: two blocks per
// compute unit, as with the fp32 staging.
//
// MFMA operands: lane l of v_mfma_f32_32x32x16_bf16 holds A(m = l%32, k = 8(l/32)..+7)
// (likewise B(k, n = l%32)); ds_read_b64_tr_b16 gathers them from the [k][m] planes:
// within a group of 16 lanes, lane s supplies the address of 4 consecutive m at row
// s/4 and receives the 4 k values of column s, so two reads (rows +0 and +4) give a
// lane its 8 k values. The accumulator layout is that of v_mfma_f32_32x32x2f32 (Oct).
constexpr int XK = 16;                        // k per staged chunk
constexpr int XPLANE = XK * TB;               // bf16 per plane
constexpr int XOP = 3 * XPLANE;               // one operand: three planes
constexpr int XCH = 2 * XOP;                  // one chunk: A and B
constexpr int X3_LDS_BYTES = 2 * XCH * 2;     // double-buffered (49152)
static_assert(X3_LDS_BYTES <= 4 * CHUNK * 4, "callers size their LDS for the fp32 staging");

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4bf lds_v4bf;

template <int MODE>
__device__ inline v4f x3_fetch(const Operand& o, __amdgpu_buffer_rsrc_t rs, int k0) {
  const int k = k0 + (threadIdx.x >> 5), m = o.m0 + 4 * (threadIdx.x & 31);
  const int ld = static_cast<int>(o.ld);
  const bool rok = k < o.kv;
  if constexpr (MODE == LD_V4) {
    const unsigned off = static_cast<unsigned>(k * ld + m) * 4u;
    return __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rs, (rok & (m < o.mv)) ? off : 0x80000000u, 0, 0));
  } else {
    v4f v;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool ok = rok & (m + u < o.mv);
      if constexpr (MODE == LD_F32) {
        const unsigned off = static_cast<unsigned>(k * ld + m + u) * 4u;
        v[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, ok ? off : 0x80000000u, 0, 0));
      } else {
        const unsigned off = static_cast<unsigned>(k * ld + m + u) * 2u;
        const unsigned short h = __builtin_amdgcn_raw_buffer_load_b16(rs, ok ? off : 0x80000000u, 0, 0);
        v[u] = static_cast<float>(__builtin_bit_cast(_Float16, h));
      }
    }
    return v;
  }
}

// bf16 offset of plane element (k, m), m a multiple of 4
__device__ __forceinline__ int x3_swz(int k, int m) { return k * TB + ((((m >> 2) ^ ((k & 3) << 3))) << 2); }

__device__ inline void x3_stage(__bf16* planes, v4f x) {
  v4bf p0, p1, p2;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const __bf16 h0 = static_cast<__bf16>(x[u]);
    const float r1 = x[u] - static_cast<float>(h0);
    const __bf16 h1 = static_cast<__bf16>(r1);
    p0[u] = h0;
    p1[u] = h1;
    p2[u] = static_cast<__bf16>(r1 - static_cast<float>(h1));
  }
  const int o = x3_swz(threadIdx.x >> 5, 4 * (threadIdx.x & 31));
  *reinterpret_cast<v4bf*>(planes + o) = p0;
  *reinterpret_cast<v4bf*>(planes + XPLANE + o) = p1;
  *reinterpret_cast<v4bf*>(planes + 2 * XPLANE + o) = p2;
}

// operand registers of the 32 columns c0.. of one plane, k 0..15 of the chunk
__device__ __forceinline__ v8bf x3_operand(const __bf16* plane, int c0) {
  const int lane = threadIdx.x & 63, s = lane & 15;
  const int m = c0 + 16 * ((lane >> 4) & 1) + 4 * (s & 3);
  const int k = 8 * (lane >> 5) + (s >> 2);
  const v4bf lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf*)(plane + x3_swz(k, m)));
  const v4bf hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf*)(plane + x3_swz(k + 4, m)));
  return v8bf{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// acc += A^T B over one staged chunk: A planes at pa, B planes at pb (XPLANE apart)
__device__ inline void x3_mma(Oct& o, const __bf16* pa, const __bf16* pb) {
  const int wave = threadIdx.x >> 6;
  const int wm = 32 * (wave >> 1), wn = 64 * (wave & 1);
  v8bf a[3], b[2][3];
#pragma unroll
  for (int p = 0; p < 3; ++p) a[p] = x3_operand(pa + p * XPLANE, wm);
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int p = 0; p < 3; ++p) b[j][p] = x3_operand(pb + p * XPLANE, wn + 32 * j);
#pragma unroll
  for (int j = 0; j < 2; ++j) {  // small parts first
    o.c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2], b[j][0], o.c[j], 0, 0, 0);
    o.c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[j][1], o.c[j], 0, 0, 0);
    o.c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[j][2], o.c[j], 0, 0, 0);
    o.c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[j][0], o.c[j], 0, 0, 0);
    o.c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[j][1], o.c[j], 0, 0, 0);
    o.c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[j][0], o.c[j], 0, 0, 0);
  }
}

// acc += sign * A^T B over k in [0, K) for two rows-form operands loaded in the forms
// MA and MB, each spanning less than 2^31 bytes (callers check), with the bf16x3
// products: loads two chunks ahead in registers, double-buffered LDS planes
// (X3_LDS_BYTES of lds), one barrier per chunk, K padded to an even chunk count with
// zeros. Ends with a barrier.
template <int MA = LD_V4, int MB = LD_V4>
__device__ inline void oct_gemm(Oct& o, const Operand& A, const Operand& B, int K, float sign, float* lds_f) {
  __bf16* lds = reinterpret_cast<__bf16*>(lds_f);
  const int npair = (K + 2 * XK - 1) / (2 * XK);
  const __amdgpu_buffer_rsrc_t rsa = op_rsrc<MA>(A);
  const __amdgpu_buffer_rsrc_t rsb = op_rsrc<MB>(B);
  v4f ra0 = x3_fetch<MA>(A, rsa, 0), rb0 = x3_fetch<MB>(B, rsb, 0);
  v4f ra1 = x3_fetch<MA>(A, rsa, XK), rb1 = x3_fetch<MB>(B, rsb, XK);
  x3_stage(lds, ra0 * sign);
  x3_stage(lds + XOP, rb0);
  ra0 = x3_fetch<MA>(A, rsa, 2 * XK);
  rb0 = x3_fetch<MB>(B, rsb, 2 * XK);
  __syncthreads();
  auto step = [&](int c, v4f& ra, v4f& rb) {
    x3_mma(o, lds + (c & 1) * XCH, lds + (c & 1) * XCH + XOP);
    __bf16* nxt = lds + ((c + 1) & 1) * XCH;
    x3_stage(nxt, ra * sign);
    x3_stage(nxt + XOP, rb);
    ra = x3_fetch<MA>(A, rsa, (c + 3) * XK);
    rb = x3_fetch<MB>(B, rsb, (c + 3) * XK);
    __syncthreads();
  };
  for (int c = 0; c < 2 * npair; c += 2) {
    step(c, ra1, rb1);
    step(c + 1, ra0, rb0);
  }
}

// acc += Y^T Y for one rows-form operand Y (16-byte load form, kv rows, under 2^31
// bytes) with the bf16x3 products: each chunk is staged once and read as both
// operands, into a single set of planes (X3_GRAM_LDS_BYTES of lds), with the next
// chunk's loads in flight during the MFMAs. Rows past kv read as zeros. Ends with a
// barrier.
constexpr int X3_GRAM_LDS_BYTES = XOP * 2;
__device__ inline void oct_gram(Oct& o, const Operand& Y, __bf16* lds) {
  const int nch = (Y.kv + XK - 1) / XK;
  const __amdgpu_buffer_rsrc_t rs = op_rsrc<LD_V4>(Y);
  v4f r = x3_fetch<LD_V4>(Y, rs, 0);
  for (int c = 0; c < nch; ++c) {
    x3_stage(lds, r);
    r = x3_fetch<LD_V4>(Y, rs, (c + 1) * XK);
    __syncthreads();
    x3_mma(o, lds, lds);
    __syncthreads();
  }
}

}  // namespace kfac
