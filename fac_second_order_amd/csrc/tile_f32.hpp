// fp32 MFMA tile engine: a 256-thread block accumulates a 128x128 fp32 tile
// C[m][n] += sum_k A[k][m] * B[k][n] with both operands read as rows of k
// ("A^T B" form). K is consumed in chunks of 32: while the MFMAs work on chunk c out
// of one LDS buffer, the global loads of chunk c+1 are in flight into registers and
// then land in the other LDS buffer, so there is one barrier per chunk. Each thread
// stages a 4(k) x 4(m) patch per operand with 16-byte loads when the rows are
// 16-byte aligned (scalar loads otherwise). Four waves each own a 64x64 quadrant
// made of 2x2 v_mfma_f32_32x32x2f32 blocks.
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

// Thread index within the 256-thread engine group: blocks of 512 threads run two
// engines side by side (threads 0..255 and 256..511).
__device__ __forceinline__ int etid() { return threadIdx.x & 255; }

struct Quad {
  v16f c[2][2];
};

__device__ inline void quad_zero(Quad& q) {
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) q.c[a][b][e] = 0.f;
}

// Row (within the 128 tile) held by accumulator register e of block (a, .) in this lane.
__device__ inline int quad_row(int wm, int a, int e, int lane) {
  return wm * 64 + a * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
}
__device__ inline int quad_col(int wn, int b, int lane) { return wn * 64 + b * 32 + (lane & 31); }

// One operand: element (k, m) of the logical [K][M] operand is src[k*ld + m] (rows),
// or src[m*ld + k] when trans. Columns m0.. of the tile; valid k < kv, m < mv.
struct Operand {
  const void* src;
  int64_t ld;
  int kv, m0, mv;
  bool f16, trans, vec4;  // vec4: rows are 16-byte aligned (rows form, fp32 only)
};

__device__ inline Operand op_rows(const float* src, int64_t ld, int kv, int m0, int mv) {
  Operand o{src, ld, kv, m0, mv, false, false,
            (ld % 4 == 0) && (reinterpret_cast<uintptr_t>(src) % 16 == 0) && (m0 % 4 == 0)};
  return o;
}
__device__ inline Operand op_rows_h(const _Float16* src, int64_t ld, int kv, int m0, int mv) {
  Operand o{src, ld, kv, m0, mv, true, false, false};
  return o;
}
__device__ inline Operand op_cols(const float* src, int64_t ld, int kv, int m0, int mv) {
  Operand o{src, ld, kv, m0, mv, false, true, false};
  return o;
}

// Thread (kg = tid/32, mg = tid%32) stages k = 4kg..4kg+3 and m = 4mg..4mg+3 of a chunk.
__device__ inline void op_fetch(const Operand& o, int k0, float4 (&r)[4]) {
  const int kg = etid() >> 5, mg = etid() & 31;
  const int m = o.m0 + 4 * mg;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int k = k0 + 4 * kg + q;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (k < o.kv) {
      if (o.vec4 && m + 3 < o.mv) {
        const v4f x = *reinterpret_cast<const KG v4f*>(gp(static_cast<const float*>(o.src)) + k * o.ld + m);
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
      } else if (o.trans) {
        const KG float* s = gp(static_cast<const float*>(o.src));
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (m + u < o.mv) v[u] = s[int64_t(m + u) * o.ld + k];
      } else if (o.f16) {
        const KG _Float16* s = gp(static_cast<const _Float16*>(o.src)) + k * o.ld;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (m + u < o.mv) v[u] = static_cast<float>(s[m + u]);
      } else {
        const KG float* s = gp(static_cast<const float*>(o.src)) + k * o.ld;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (m + u < o.mv) v[u] = s[m + u];
      }
    }
    r[q] = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// Fast path for fp32 rows whose pitch is padded to a multiple of 4 floats, with src
// 16-byte aligned and m0 % 4 == 0 (checked by the caller): each 4-group starting
// below mv is read whole with one 16-byte load. Entries of a group at or beyond mv
// are row padding: they only reach output rows or columns >= mv, which callers
// never store.
__device__ inline void op_fetch_rows4(const Operand& o, int k0, float4 (&r)[4]) {
  const int kg = etid() >> 5, mg = etid() & 31;
  const int m = o.m0 + 4 * mg;
  const KG float* base = gp(static_cast<const float*>(o.src)) + m;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int k = k0 + 4 * kg + q;
    v4f x = {0.f, 0.f, 0.f, 0.f};
    if (k < o.kv && m < o.mv) x = *reinterpret_cast<const KG v4f*>(base + k * o.ld);
    r[q] = make_float4(x.x, x.y, x.z, x.w);
  }
}

// Load forms of a rows-form operand in the buffer pipeline: 16-byte groups (fp32 rows
// as for op_fetch_rows4), single fp32 values, single fp16 values.
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

// Branch-free staging loads through a raw buffer: every load is issued, and a load
// outside the operand (k >= kv or m >= mv) gets an offset past the buffer's range, for
// which it returns zeros without touching memory. With the same number of loads on
// every path, the wait before an LDS store covers only the chunk being stored.
// LD_V4 reads each 4-group starting below mv whole (the rows are padded, as for
// op_fetch_rows4); the other forms read element by element.
template <int MODE>
__device__ inline void op_fetch_buf(const Operand& o, __amdgpu_buffer_rsrc_t rs, int k0, float4 (&r)[4]) {
  const int kg = etid() >> 5, mg = etid() & 31;
  const int m = o.m0 + 4 * mg;
  const int ld = static_cast<int>(o.ld);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int k = k0 + 4 * kg + q;
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

template <bool ROWS4>
__device__ inline void fetch(const Operand& o, int k0, float4 (&r)[4]) {
  if constexpr (ROWS4) op_fetch_rows4(o, k0, r);
  else op_fetch(o, k0, r);
}

__device__ inline void op_store(float* lds, const float4 (&r)[4]) {
  const int kg = etid() >> 5, mg = etid() & 31;
#pragma unroll
  for (int q = 0; q < 4; ++q) *reinterpret_cast<float4*>(lds + (4 * kg + q) * LDP + 4 * mg) = r[q];
}

// acc += sign * As^T Bs over one staged chunk (KT values of k), pitches in floats.
// The LDS reads run four k-steps ahead of the MFMAs that use them (explicit schedule
// groups: left to itself the scheduler puts each read right before its MFMAs, which
// exposes the LDS latency on every k-step).
__device__ inline void quad_mma_p(Quad& q, const float* As, int apitch, const float* Bs, int bpitch,
                                  float sign) {
  const int lane = etid() & 63, wave = etid() >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ml = lane & 31, kh = lane >> 5;
  float a0[KT / 2], a1[KT / 2], b0[KT / 2], b1[KT / 2];
#pragma unroll
  for (int t = 0; t < KT / 2; ++t) {
    const float* ar = As + (2 * t + kh) * apitch + wm * 64 + ml;
    const float* br = Bs + (2 * t + kh) * bpitch + wn * 64 + ml;
    a0[t] = ar[0]; a1[t] = ar[32]; b0[t] = br[0]; b1[t] = br[32];
  }
#pragma unroll
  for (int t = 0; t < KT / 2; ++t) {
    const float x0 = a0[t] * sign, x1 = a1[t] * sign;
    q.c[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(x0, b0[t], q.c[0][0], 0, 0, 0);
    q.c[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(x0, b1[t], q.c[0][1], 0, 0, 0);
    q.c[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(x1, b0[t], q.c[1][0], 0, 0, 0);
    q.c[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(x1, b1[t], q.c[1][1], 0, 0, 0);
  }
  // schedule: reads of 4 k-steps ahead, then per k-step 4 MFMAs and the reads of step t+4
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
  for (int t = 0; t < KT / 2 - 4; ++t) {
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
}

// acc += sign * A^T B over k in [0, K), pipelined. lds holds 4*CHUNK floats
// (two buffers of the A and B chunks). Global loads run two chunks ahead of the
// MFMAs in two register stages used alternately: while the MFMAs read chunk c from
// one LDS buffer, chunks c+1 and c+2 are in flight; after the MFMAs, chunk c+1 goes
// to the other buffer and its registers take chunk c+3. One barrier per chunk; ends
// with a barrier. ROWS4: both operands qualify for op_fetch_rows4.
template <bool ROWS4 = false>
__device__ inline void quad_gemm(Quad& q, const Operand& A, const Operand& B, int K, float sign,
                                 float* lds) {
  const int nchunk = (K + KT - 1) / KT;
  float4 ra0[4], rb0[4], ra1[4], rb1[4];
  fetch<ROWS4>(A, 0, ra0);
  fetch<ROWS4>(B, 0, rb0);
  if (nchunk > 1) {
    fetch<ROWS4>(A, KT, ra1);
    fetch<ROWS4>(B, KT, rb1);
  }
  op_store(lds, ra0);
  op_store(lds + CHUNK, rb0);
  if (nchunk > 2) {
    fetch<ROWS4>(A, 2 * KT, ra0);
    fetch<ROWS4>(B, 2 * KT, rb0);
  }
  __syncthreads();
  // ra/rb: the stage holding chunk c+1
  auto step = [&](int c, float4 (&ra)[4], float4 (&rb)[4]) {
    const float* cur = lds + (c & 1) * 2 * CHUNK;
    quad_mma_p(q, cur, LDP, cur + CHUNK, LDP, sign);
    if (c + 1 < nchunk) {
      float* nxt = lds + ((c + 1) & 1) * 2 * CHUNK;
      op_store(nxt, ra);
      op_store(nxt + CHUNK, rb);
      if (c + 3 < nchunk) {
        fetch<ROWS4>(A, (c + 3) * KT, ra);
        fetch<ROWS4>(B, (c + 3) * KT, rb);
      }
    }
    __syncthreads();
  };
  for (int c = 0; c < nchunk; c += 2) {
    step(c, ra1, rb1);
    if (c + 1 < nchunk) step(c + 1, ra0, rb0);
  }
}

// quad_gemm for two rows-form operands, each spanning less than 2^31 bytes, loaded in
// the forms MA and MB. Same pipeline, but every chunk load is issued unconditionally
// (op_fetch_buf; chunks past K read as zeros, and K is padded to an even chunk count),
// so that each LDS store waits only for its own chunk while the next one stays in
// flight.
template <int MA = LD_V4, int MB = LD_V4>
__device__ inline void quad_gemm_buf(Quad& q, const Operand& A, const Operand& B, int K, float sign,
                                     float* lds) {
  const int npair = (K + 2 * KT - 1) / (2 * KT);
  const __amdgpu_buffer_rsrc_t rsa = op_rsrc<MA>(A), rsb = op_rsrc<MB>(B);
  float4 ra0[4], rb0[4], ra1[4], rb1[4];
  op_fetch_buf<MA>(A, rsa, 0, ra0);
  op_fetch_buf<MB>(B, rsb, 0, rb0);
  op_fetch_buf<MA>(A, rsa, KT, ra1);
  op_fetch_buf<MB>(B, rsb, KT, rb1);
  op_store(lds, ra0);
  op_store(lds + CHUNK, rb0);
  op_fetch_buf<MA>(A, rsa, 2 * KT, ra0);
  op_fetch_buf<MB>(B, rsb, 2 * KT, rb0);
  __syncthreads();
  // ra/rb: the stage holding chunk c+1; afterwards it takes chunk c+3
  auto step = [&](int c, float4 (&ra)[4], float4 (&rb)[4]) {
    const float* cur = lds + (c & 1) * 2 * CHUNK;
    quad_mma_p(q, cur, LDP, cur + CHUNK, LDP, sign);
    float* nxt = lds + ((c + 1) & 1) * 2 * CHUNK;
    op_store(nxt, ra);
    op_store(nxt + CHUNK, rb);
    op_fetch_buf<MA>(A, rsa, (c + 3) * KT, ra);
    op_fetch_buf<MB>(B, rsb, (c + 3) * KT, rb);
    __syncthreads();
  };
  for (int c = 0; c < 2 * npair; c += 2) {
    step(c, ra1, rb1);
    step(c + 1, ra0, rb0);
  }
}

// Same with the B operand already resident in LDS as rows [k][n] (pitch bpitch), and
// an A operand of fp32 rows with 16-byte groups spanning less than 2^31 bytes: its
// chunks come through the branch-free buffer loads (zeros past K), two ahead of the
// MFMAs (one in LDS, one in registers). Ends with a barrier.
__device__ inline void quad_gemm_lds_b(Quad& q, const Operand& A, const float* Bl, int bpitch, int K,
                                       float sign, float* lds) {
  const int nchunk = (K + KT - 1) / KT;
  const __amdgpu_buffer_rsrc_t rs = op_rsrc<LD_V4>(A);
  float4 ra[4];
  op_fetch_buf<LD_V4>(A, rs, 0, ra);
  op_store(lds, ra);
  op_fetch_buf<LD_V4>(A, rs, KT, ra);
  __syncthreads();
  for (int c = 0; c < nchunk; ++c) {
    float* cur = lds + (c & 1) * CHUNK;
    float* nxt = lds + ((c + 1) & 1) * CHUNK;
    quad_mma_p(q, cur, LDP, Bl + c * KT * bpitch, bpitch, sign);
    op_store(nxt, ra);
    op_fetch_buf<LD_V4>(A, rs, (c + 2) * KT, ra);
    __syncthreads();
  }
}

// ---- 512-thread variant ("oct"): eight waves share one 128x128 tile, wave w owning
// rows 32*(w/2) .. +32 and columns 64*(w%2) .. +64 (two 32x32 blocks). With half the
// accumulators and half the staging per thread, two blocks give every SIMD four waves,
// so the tile load and store of one block overlap the other block's MFMAs. Same
// chunking, LDS layout and pipeline as the 256-thread engine.
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
// of a chunk, branch-free through a raw buffer in the load form MODE, as op_fetch_buf.
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

// The same through plain loads with per-element checks, for operands of any size
// (rows, fp32 or fp16; no transposed form).
__device__ inline void oct_fetch_plain(const Operand& o, int k0, float4 (&r)[2]) {
  const int kg = threadIdx.x >> 5, mg = threadIdx.x & 31;
  const int m = o.m0 + 4 * mg;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int64_t k = k0 + 2 * kg + q;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (k < o.kv) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (m + u < o.mv)
          v[u] = o.f16 ? static_cast<float>(gp(static_cast<const _Float16*>(o.src))[k * o.ld + m + u])
                       : gp(static_cast<const float*>(o.src))[k * o.ld + m + u];
    }
    r[q] = make_float4(v[0], v[1], v[2], v[3]);
  }
}

__device__ inline void oct_stage(float* lds, const float4 (&r)[2]) {
  const int kg = threadIdx.x >> 5, mg = threadIdx.x & 31;
#pragma unroll
  for (int q = 0; q < 2; ++q) *reinterpret_cast<float4*>(lds + (2 * kg + q) * LDP + 4 * mg) = r[q];
}

// acc += sign * As^T Bs over one staged chunk, LDS reads four k-steps ahead of the
// MFMAs (explicit schedule groups, as in quad_mma_p).
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
// MA and MB, each spanning less than 2^31 bytes: the quad_gemm_buf pipeline (two
// chunks ahead in registers, double-buffered LDS of 4*CHUNK floats, one barrier per
// chunk, K padded to an even chunk count with zeros). With PLAIN, plain loads with
// per-element checks instead (operands of any size). Ends with a barrier.
template <int MA = LD_V4, int MB = LD_V4, bool PLAIN = false>
__device__ inline void oct_gemm(Oct& o, const Operand& A, const Operand& B, int K, float sign, float* lds) {
  const int npair = (K + 2 * KT - 1) / (2 * KT);
  // (unused with PLAIN: an empty range)
  const __amdgpu_buffer_rsrc_t rsa = PLAIN ? __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(A.src), 0, 0, 0x00020000)
                                           : op_rsrc<MA>(A);
  const __amdgpu_buffer_rsrc_t rsb = PLAIN ? __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(B.src), 0, 0, 0x00020000)
                                           : op_rsrc<MB>(B);
  auto fa = [&](int k0, float4 (&r)[2]) {
    if constexpr (PLAIN) oct_fetch_plain(A, k0, r);
    else oct_fetch<MA>(A, rsa, k0, r);
  };
  auto fb = [&](int k0, float4 (&r)[2]) {
    if constexpr (PLAIN) oct_fetch_plain(B, k0, r);
    else oct_fetch<MB>(B, rsb, k0, r);
  };
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

// Tile <-> global (row-major, leading dimension ld), rows < rvalid, cols < cvalid.
__device__ inline void quad_load(Quad& q, const float* src, int64_t ld, int rvalid, int cvalid) {
  const int lane = etid() & 63, wave = etid() >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  if (rvalid >= TB && cvalid >= TB) {  // interior tile: no per-element checks
    const KG float* s = gp(src) + int64_t(quad_row(wm, 0, 0, lane)) * ld + quad_col(wn, 0, lane);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          q.c[a][b][e] = s[int64_t(a * 32 + 8 * (e >> 2) + (e & 3)) * ld + b * 32];
    return;
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = quad_row(wm, a, e, lane), c = quad_col(wn, b, lane);
        q.c[a][b][e] = (r < rvalid && c < cvalid) ? gp(src)[int64_t(r) * ld + c] : 0.f;
      }
}

// q += tile loaded from global.
__device__ inline void quad_add_global(Quad& q, const float* src, int64_t ld, int rvalid, int cvalid) {
  const int lane = etid() & 63, wave = etid() >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = quad_row(wm, a, e, lane), c = quad_col(wn, b, lane);
        if (r < rvalid && c < cvalid) q.c[a][b][e] += gp(src)[int64_t(r) * ld + c];
      }
}

__device__ inline void quad_store(const Quad& q, float* dst, int64_t ld, int rvalid, int cvalid,
                                  float scale = 1.f) {
  const int lane = etid() & 63, wave = etid() >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  if (rvalid >= TB && cvalid >= TB) {  // interior tile
    KG float* o = gp(dst) + int64_t(quad_row(wm, 0, 0, lane)) * ld + quad_col(wn, 0, lane);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          o[int64_t(a * 32 + 8 * (e >> 2) + (e & 3)) * ld + b * 32] = q.c[a][b][e] * scale;
    return;
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = quad_row(wm, a, e, lane), c = quad_col(wn, b, lane);
        if (r < rvalid && c < cvalid) gp(dst)[int64_t(r) * ld + c] = q.c[a][b][e] * scale;
      }
}

// Upper-triangle store of a square tile: entries r <= c < nvalid.
__device__ inline void quad_store_upper(const Quad& q, float* dst, int64_t ld, int nvalid) {
  const int lane = etid() & 63, wave = etid() >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = quad_row(wm, a, e, lane), c = quad_col(wn, b, lane);
        if (r <= c && c < nvalid) gp(dst)[int64_t(r) * ld + c] = q.c[a][b][e];
      }
}

// Transposed store through LDS (coalesced): dst[c*ld + r] = tile[r][c] for r < rvalid,
// c < cvalid. lds needs TB*LDT floats; ends with a barrier (256-thread blocks only).
__device__ inline void quad_store_t(const Quad& q, float* dst, int64_t ld, int rvalid, int cvalid,
                                    float* lds) {
  const int lane = etid() & 63, wave = etid() >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        lds[quad_col(wn, b, lane) * LDT + quad_row(wm, a, e, lane)] = q.c[a][b][e];
  __syncthreads();
  for (int e = etid(); e < TB * TB; e += 256) {
    const int c = e / TB, r = e % TB;  // output row c, column r: contiguous in r
    if (r < rvalid && c < cvalid) gp(dst)[int64_t(c) * ld + r] = lds[c * LDT + r];
  }
  __syncthreads();
}

// Tile -> LDS [TB][pitch] (rows r, columns c), all 128x128 entries.
__device__ inline void quad_to_lds(const Quad& q, float* lds, int pitch) {
  const int lane = etid() & 63, wave = etid() >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        lds[quad_row(wm, a, e, lane) * pitch + quad_col(wn, b, lane)] = q.c[a][b][e];
}

}  // namespace kfac
