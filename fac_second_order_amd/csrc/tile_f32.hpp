// fp32 MFMA tile engine: a 512-thread block accumulates a 128x128 fp32 tile
// C[m][n] += sum_k A[k][m] * B[k][n] with both operands read as rows of k
// ("A^T B" form). K is consumed in chunks of 32: while the MFMAs work on chunk c out
// of one LDS buffer, the global loads of chunks c+1 and c+2 are in flight in
// registers, and chunk c+1 then lands in the other LDS buffer, so there is one
// barrier per chunk. Eight waves share the tile, wave w owning rows 32*(w/2) .. +32
// and columns 64*(w%2) .. +64 (two v_mfma_f32_32x32x2f32 blocks); two blocks per
// compute unit give every SIMD four waves, so the tile load and store of one block
// overlap the other block's MFMAs.
//
// MFMA lane layout (v_mfma_f32_32x32x2f32, wave64): A operand element (m, k) sits
// in lane m + 32k, B operand element (k, n) in lane n + 32k; accumulator register e
// of lane l holds row 8*(e/4) + 4*(l/32) + e%4, column l%32 of the 32x32 block.
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

// Load forms of an operand: 16-byte groups (fp32 rows whose pitch is a multiple of 4
// floats on a 16-byte aligned base, m0 % 4 == 0), single fp32 values, single fp16
// values.
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
// reads each 4-group that starts below mv whole: its entries at or past mv are row
// padding and reach only output rows or columns >= mv, which callers never store.
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

// acc += sign * As^T Bs over one staged chunk, LDS reads four k-steps ahead of the
// MFMAs (explicit schedule groups: left to itself the scheduler puts each read right
// before its MFMAs, which exposes the LDS latency on every k-step).
__device__ inline void oct_mma(Oct& o, const float* As, const float* Bs, float sign) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ml = lane & 31, kh = lane >> 5;
  float a0[KT / 2], b0[KT / 2], b1[KT / 2];
#pragma unroll
  for (int t = 0; t < KT / 2; ++t) {
    const float* ar = As + (2 * t + kh) * LDP + wm * 32 + ml;
    const float* br = Bs + (2 * t + kh) * LDP + wn * 64 + ml;
    a0[t] = ar[0]; b0[t] = br[0]; b1[t] = br[32];
  }
#pragma unroll
  for (int t = 0; t < KT / 2; ++t) {
    const float x0 = a0[t] * sign;
    o.c[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(x0, b0[t], o.c[0], 0, 0, 0);
    o.c[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(x0, b1[t], o.c[1], 0, 0, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
  for (int t = 0; t < KT / 2 - 4; ++t) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
}

// acc += sign * A^T B over k in [0, K) for two rows-form operands loaded in the forms
// MA and MB, each spanning less than 2^31 bytes (callers check): loads two chunks
// ahead in registers, double-buffered LDS of 4*CHUNK floats, one barrier per chunk,
// K padded to an even chunk count with zeros. Ends with a barrier.
template <int MA = LD_V4, int MB = LD_V4>
__device__ inline void oct_gemm(Oct& o, const Operand& A, const Operand& B, int K, float sign, float* lds) {
  const int npair = (K + 2 * KT - 1) / (2 * KT);
  const __amdgpu_buffer_rsrc_t rsa = op_rsrc<MA>(A);
  const __amdgpu_buffer_rsrc_t rsb = op_rsrc<MB>(B);
  auto fa = [&](int k0, float4 (&r)[2]) { oct_fetch<MA>(A, rsa, k0, r); };
  auto fb = [&](int k0, float4 (&r)[2]) { oct_fetch<MB>(B, rsb, k0, r); };
  float4 ra0[2], rb0[2], ra1[2], rb1[2];
  fa(0, ra0);
  fb(0, rb0);
  fa(KT, ra1);
  fb(KT, rb1);
  oct_stage(lds, ra0);
  oct_stage(lds + CHUNK, rb0);
  fa(2 * KT, ra0);
  fb(2 * KT, rb0);
  __syncthreads();
  auto step = [&](int c, float4 (&ra)[2], float4 (&rb)[2]) {
    const float* cur = lds + (c & 1) * 2 * CHUNK;
    oct_mma(o, cur, cur + CHUNK, sign);
    float* nxt = lds + ((c + 1) & 1) * 2 * CHUNK;
    oct_stage(nxt, ra);
    oct_stage(nxt + CHUNK, rb);
    fa((c + 3) * KT, ra);
    fb((c + 3) * KT, rb);
    __syncthreads();
  };
  for (int c = 0; c < 2 * npair; c += 2) {
    step(c, ra1, rb1);
    step(c + 1, ra0, rb0);
  }
}

}  // namespace kfac
