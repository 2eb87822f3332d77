// Kronecker factors A = E[a a^T] and G = E[g g^T] of many layers in one launch.
// Osawa et al. (CVPR 2019), Section 3.2, eq. (5): G comes from the loss gradients
// with respect to a layer's outputs, A from the layer's inputs; E is the mini-batch
// mean of eq. (1), taken here over all N*H_out*W_out patch rows. Section 1
// (contributions): the factors are symmetric, so only the upper triangle is formed
// and stored, and the products use half precision.
//
// Each factor is S = X^T X / R for a virtual row matrix X[R, d]. For A, X is the
// im2col patch matrix of the NHWC activation and is never written out: each
// 16-byte fp16 vector of 8 patch columns (one kernel tap, 8 channels) is gathered
// straight from the activation tensor into registers, transposed in registers and
// stored column-major (XOR-swizzled) into LDS, where the MFMA operands are read with
// 16-byte LDS loads. For G, X is the output-gradient tensor viewed as [R, C_out].
//
// Work item = (factor, row split, upper tile ti <= tj of 128x128). Waves compute
// 64x64 quadrants with v_mfma_f32_32x32x16_f16 (fp16 in, fp32 accumulate); the
// quadrant strictly below the diagonal of a diagonal tile is skipped. The bias
// column (constant 1) is not multiplied: its entries are column sums, accumulated
// by the diagonal tiles from the same LDS data, and R for the corner. Row splits
// write fp32 partial tiles that a second kernel adds in split order, so results
// are deterministic. The epilogue multiplies by fp32(1/R), optionally blends with
// the stored factor (exponential moving average), and writes the packed upper
// triangle. Work items are renumbered so that each of the 8 XCDs runs a contiguous
// range (tiles of one row split share that XCD's L2).
//
// The activation factor of a 3x3 convolution with stride 1 and padding 1 is not
// formed from its 9C patch columns but from 13 shift products of the C channels
// (a block-Toeplitz structure, see shift_assemble_kernel): the same work items and
// tile loop compute them as rectangular C x 13C products, and a last kernel
// assembles the packed factor, about a third of the multiplications of the patch Gram.
//
// fp32 inputs take a plain path (element gathers, v_mfma_f32_32x32x2f32).
#include <algorithm>
#include <cmath>

#include "common.hpp"

namespace kfac {

constexpr int ST = 128;           // output tile edge
constexpr int KC = 128;           // patch rows per LDS operand buffer (fp16)
constexpr int LDK = KC + 8;       // LDS row pitch in halves (272 B)
constexpr int RPT = KC / 8;       // patch rows each staging thread gathers
constexpr int KC32 = 32;          // patch rows per LDS chunk (fp32 path)
constexpr int LDN32 = ST + 4;     // LDS row pitch in floats (fp32 path)

// LDS operand layout [column m][patch row k] (fp16, pitch LDK = 68 dwords), with
// the 16-byte group of 8 rows XOR-swizzled by (m/8 ^ m/16). A thread stores the 8
// rows of one column per 16-byte write; of the swizzles measured on gfx950 this one
// gave the fastest factor pass (transposing stores conflict-free, MFMA operand reads
// of 16 consecutive m in one aligned 16-byte group each).
__device__ __forceinline__ int xoff(int m, int k) {
  return m * LDK + ((((k >> 3) ^ (m >> 3) ^ (m >> 4)) & 7) << 3) + (k & ~63) + (k & 7);
}

struct SyrkDesc {
  const void* src;
  float* out;      // packed upper triangle, d(d+1)/2
  float* partial;  // [splits][nt][ST*ST] when splits > 1
  float* pcol;     // [splits][nb][ST] bias column partial sums
  int32_t mode;    // 0: rows [R, ld]; 1: im2col of NHWC [n, H, W, C]
  int32_t vec;     // 16-byte gathers (buffer loads) allowed
  int32_t padded;  // > 0: rows written out by im2row job padded-1, zeros from d_core to ld
  int32_t nbytes;  // input tensor bytes when vec (< 2^31): the buffer range
  int32_t d_core;  // columns of X (without the bias column)
  int32_t d;       // factor order (d_core + bias)
  int32_t bias;
  int32_t R;
  int32_t H, W, C, Ho, Wo, kh, kw, sh, sw, ph, pw;
  int32_t ld;
  int32_t nb, nt, splits, rows_per_split;
  float inv_r, r_f;
  double rhw, rwo;  // 1 / (Ho Wo) and 1 / Wo for the row decode
  // kind 1, a shift product: T[c][t*C + c'] = sum over the rows' pixels p of
  // x[p][c] * x[p + (tdh[t], tdw[t])][c'] (zero outside the image), raw fp32 sums in
  // `out` (dense, leading dimension c_col), and the column sums of the row operand
  // (sum over p of x[p][c]) in csum. The rows are the pixels of an Ho x Wo window at
  // (-ph, -pw) of every image (mode 1 with stride 1 and a negative padding).
  int32_t kind;          // 0: a factor (packed upper triangle), 1: a shift product
  int32_t ntap;          // kind 1: column taps
  int32_t c_row, c_col;  // kind 1: C and ntap * C
  int32_t nbr, nbc;      // kind 1: 128-blocks along the rows and the columns of T
  float* csum;
  int8_t tdh[16], tdw[16];
  // 256x256 tiles (syrk_big_kernel): 256-blocks of the factor (kind 0) or of the rows
  // and the columns of T (kind 1), and the tiles per row split
  int32_t nb2, nbr2, nbc2, nt2;
  int32_t big;  // the problem's items run in syrk_big_kernel
  int32_t pad2_;
  // kind 0: when not NULL, every entry (i, j >= i) written to `out` is also written to
  // full[i * d + j] (row-major d x d; the strict lower triangle is not written)
  float* full;
};

// Value of X[row][c] (0 outside the image or beyond d_core), any input dtype
// (plain path for fp32 inputs).
template <class T>
__device__ inline float x_elem(const SyrkDesc& d, int row, int c) {
  if (c >= d.d_core) return 0.f;
  const KG T* src = gp(static_cast<const T*>(d.src));
  if (d.mode == 0) return static_cast<float>(src[int64_t(row) * d.ld + c]);
  const int hw = d.Ho * d.Wo;
  const int n = row / hw;
  const int rem = row - n * hw;
  const int oh = rem / d.Wo, ow = rem - (rem / d.Wo) * d.Wo;
  const int tap = c / d.C, ci = c - tap * d.C;
  const int ki = tap / d.kw, kj = tap - ki * d.kw;
  const int ih = oh * d.sh + ki - d.ph, iw = ow * d.sw + kj - d.pw;
  if (ih < 0 || ih >= d.H || iw < 0 || iw >= d.W) return 0.f;
  return static_cast<float>(src[((int64_t(n) * d.H + ih) * d.W + iw) * d.C + ci]);
}

// Row decode of one chunk of patch rows, shared through LDS: element offset of the
// row's (ih0, iw0) pixel and the top-left input coordinates of its receptive field
// (ih0 = oh*sh - ph, iw0 = ow*sw - pw). Rows past the end get an ih0 that fails every
// bounds check. In row mode (G factors, 1x1 stride-1 convolutions) the offset is
// row*ld and ih0 = iw0 = 0 with H = W = 1.
// n / dv for 0 <= n < 2^31 and dv > 0, with rdv = 1/dv rounded to fp64: the product
// is within one of the quotient, and one correction step each way makes it exact.
__device__ __forceinline__ int fast_div(int n, int dv, double rdv) {
  int q = static_cast<int>(static_cast<double>(n) * rdv);
  const int r = n - q * dv;
  q += (r >= dv) - (r < 0);
  return q;
}

struct RowTab {
  int32_t lo[2 * KC];  // element offset (input tensors span less than 2^31 bytes)
  int32_t ih[2 * KC];
  int32_t iw[2 * KC];
};

constexpr int32_t kNoRow = -(1 << 29);

__device__ inline void fill_rowtab_at(const SyrkDesc& d, RowTab& t, int r0, int r_end, int rows, int tid) {
  if (tid >= rows) return;
  const int row = r0 + tid;
  if (row >= r_end) {
    t.lo[tid] = 0;
    t.ih[tid] = kNoRow;
    t.iw[tid] = 0;
    return;
  }
  if (d.mode == 0) {
    t.lo[tid] = row * d.ld;
    t.ih[tid] = 0;
    t.iw[tid] = 0;
    return;
  }
  const int hw = d.Ho * d.Wo;
  const int n = fast_div(row, hw, d.rhw);
  const int rem = row - n * hw;
  const int oh = fast_div(rem, d.Wo, d.rwo);
  const int ow = rem - oh * d.Wo;
  const int ih0 = oh * d.sh - d.ph, iw0 = ow * d.sw - d.pw;
  t.lo[tid] = ((n * d.H + ih0) * d.W + iw0) * d.C;
  t.ih[tid] = ih0;
  t.iw[tid] = iw0;
}

__device__ inline void fill_rowtab(const SyrkDesc& d, RowTab& t, int r0, int r_end, int rows) {
  fill_rowtab_at(d, t, r0, r_end, rows, threadIdx.x);
}

// Per-thread column data for its 8 columns [c0, c0+8): tap offsets inside the input
// tensor and tap coordinates for the bounds checks (constant over rows).
struct ColTab {
  int32_t coff[8];
  int32_t ki[8];
  int32_t kj[8];
};

__device__ inline void fill_coltab(const SyrkDesc& d, int op, int c0, ColTab& ct) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int c = c0 + q;
    if (d.kind == 1) {  // op 0: the pixel's own channels; op 1: channel c % C of tap c / C
      if (c >= (op ? d.c_col : d.c_row)) {
        ct.coff[q] = 0;
        ct.ki[q] = kNoRow;
        ct.kj[q] = 0;
      } else if (op == 0) {
        ct.coff[q] = c;
        ct.ki[q] = 0;
        ct.kj[q] = 0;
      } else {
        const int tap = c / d.C, ci = c - tap * d.C;
        const int dh = d.tdh[tap], dw = d.tdw[tap];
        ct.coff[q] = (dh * d.W + dw) * d.C + ci;
        ct.ki[q] = dh;
        ct.kj[q] = dw;
      }
    } else if (c >= d.d_core) {
      ct.coff[q] = 0;
      ct.ki[q] = kNoRow;
      ct.kj[q] = 0;
    } else if (d.mode == 0) {
      ct.coff[q] = c;
      ct.ki[q] = 0;
      ct.kj[q] = 0;
    } else {
      const int tap = c / d.C, ci = c - tap * d.C;
      const int ki = tap / d.kw, kj = tap - ki * d.kw;
      ct.coff[q] = (ki * d.W + kj) * d.C + ci;
      ct.ki[q] = ki;
      ct.kj[q] = kj;
    }
  }
}

// 8 consecutive columns of the chunk row rr as fp16 (zeros outside the image, past
// the last row or past d_core), element by element (inputs whose channel count or
// alignment rules out 16-byte vectors).
__device__ inline v8h gather8_elem(const SyrkDesc& d, const RowTab& t, int rr, const ColTab& ct) {
  const KG _Float16* src = gp(static_cast<const _Float16*>(d.src));
  const int ih = t.ih[rr], iw = t.iw[rr];
  const int off = t.lo[rr];
  v8h v;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const bool ok = unsigned(ih + ct.ki[q]) < unsigned(d.H) && unsigned(iw + ct.kj[q]) < unsigned(d.W);
    v[q] = ok ? src[off + ct.coff[q]] : static_cast<_Float16>(0.f);
  }
  return v;
}

// The same when the 8 columns share one tap (d.vec), for the N consecutive chunk
// rows rr0.. at once: one 16-byte buffer load per row. A padding tap, a row past the
// end or columns past d_core get an offset beyond the buffer's range, for which the
// load returns zeros without touching memory. All table entries are read before any
// address is formed (one LDS round trip instead of one per row).
template <int N>
__device__ __forceinline__ void gather8_vec(__amdgpu_buffer_rsrc_t rsrc, int H, int W, const RowTab& t,
                                            int rr0, const ColTab& ct, v8h (&v)[N]) {
  int lo[N], ih[N], iw[N];
#pragma unroll
  for (int q = 0; q < N; q += 4) {
    const v4i a = *reinterpret_cast<const v4i*>(t.lo + rr0 + q);
    const v4i b = *reinterpret_cast<const v4i*>(t.ih + rr0 + q);
    const v4i c = *reinterpret_cast<const v4i*>(t.iw + rr0 + q);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      lo[q + u] = a[u];
      ih[q + u] = b[u];
      iw[q + u] = c[u];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < N; ++q) {
    const bool ok = (unsigned(ih[q] + ct.ki[0]) < unsigned(H)) & (unsigned(iw[q] + ct.kj[0]) < unsigned(W));
    const unsigned off = static_cast<unsigned>(lo[q] + ct.coff[0]) * 2u;
    const v4u x = __builtin_amdgcn_raw_buffer_load_b128(rsrc, ok ? off : 0x80000000u, 0, 0);
    v[q] = __builtin_bit_cast(v8h, x);
  }
}

__device__ inline float blend(float v, const float* out, int64_t o, float decay) {
  return decay != 0.f ? decay * gp(out)[o] + (1.f - decay) * v : v;
}

// Entry (i, j >= i) of a factor: the packed store at o and, when asked for, the full one.
__device__ inline void put_entry(const SyrkDesc& d, int64_t o, int i, int j, float v) {
  gp(d.out)[o] = v;
  if (d.full) gp(d.full)[int64_t(i) * d.d + j] = v;
}

// Writes the bias column entries (column sums) and the bias corner of a direct tile.
__device__ inline void write_bias_direct(const SyrkDesc& d, int ti, int t, float colsum,
                                         float decay) {
  const int tid = threadIdx.x;
  if (tid < ST) {
    const int i = ti * ST + tid;
    if (i < d.d_core) {
      const int64_t o = packed_off(i, d.d_core, d.d);
      put_entry(d, o, i, d.d_core, blend(colsum * d.inv_r, d.out, o, decay));
    }
  }
  if (t == 0 && tid == 0) {
    const int64_t o = packed_off(d.d_core, d.d_core, d.d);
    put_entry(d, o, d.d_core, d.d_core, blend(d.r_f * d.inv_r, d.out, o, decay));
  }
}

// Main loop of a tile over patch rows [r_begin, r_end): gathers of the next chunk
// overlap the MFMAs of the current one. An off-diagonal tile stages its two operands
// (row block ti into X0, tj into X1) over chunks of KC rows; a diagonal tile has one
// operand and stages chunks of 2 KC rows, the first KC in X0 and the rest in X1, so
// that every thread gathers the same 8 rows x 8 columns in both kinds. VEC: 16-byte
// buffer-load gathers. want_col: thread tid < 128 adds up column tid of the row
// operand. mma_on (wave-uniform): this wave's 64x64 quadrant is needed (not the one
// below a diagonal tile's diagonal, not past the last row of a shift product).
template <bool DIAG, bool VEC>
__device__ __forceinline__ void syrk_rows(const SyrkDesc& d, RowTab* tab, _Float16* X0, _Float16* X1,
                                          const ColTab& ct, int r_begin, int r_end, bool want_col,
                                          bool mma_on, v16f (&acc)[2][2], float& colsum) {
  constexpr int CK = DIAG ? 2 * KC : KC;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // staging: thread = (half op, column group cg of 8, row group rg of RPT)
  const int op = tid >> 7, cg = tid & 15, rg = (tid >> 4) & 7;
  const int rrow = (DIAG ? op * KC : 0) + rg * RPT;
  _Float16* Xo = op ? X1 : X0;
  // raw buffer over the input tensor (used by the VEC gathers only)
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(d.src), 0, d.nbytes, 0x00020000);
  const int H = d.H, W = d.W;
  // rows rr0.. of the chunk into v[0 .. NV)
  auto gather = [&](const RowTab& t, int rr0, v8h(&v)[VEC ? RPT : 8]) {
    if constexpr (VEC) {
      gather8_vec<RPT>(rsrc, H, W, t, rr0, ct, v);
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = gather8_elem(d, t, rr0 + q, ct);
    }
  };
  auto mma = [&](const _Float16* A, const _Float16* B) {
#pragma unroll
    for (int ks = 0; ks < KC / 16; ++ks) {
      const int ko = ks * 16 + (lane >> 5) * 8;
      const v8h a0 = *reinterpret_cast<const v8h*>(A + xoff(wm * 64 + (lane & 31), ko));
      const v8h a1 = *reinterpret_cast<const v8h*>(A + xoff(wm * 64 + 32 + (lane & 31), ko));
      const v8h b0 = *reinterpret_cast<const v8h*>(B + xoff(wn * 64 + (lane & 31), ko));
      const v8h b1 = *reinterpret_cast<const v8h*>(B + xoff(wn * 64 + 32 + (lane & 31), ko));
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1, acc[1][1], 0, 0, 0);
    }
  };
  fill_rowtab(d, tab[0], r_begin, r_end, CK);
  __syncthreads();
  // rows held across the MFMAs: all RPT with 16-byte gathers; the element gathers
  // (one register per fp16 value in flight) prefetch the first 8 and fetch the rest
  // after storing them
  constexpr int NV = VEC ? RPT : 8;
  v8h v[NV];
  gather(tab[0], rrow, v);
  int c = 0;
  for (int r0 = r_begin; r0 < r_end; r0 += CK, ++c) {
    const bool more = r0 + CK < r_end;
    __syncthreads();  // the previous chunk's LDS operands are consumed
#pragma unroll
    for (int g = 0; g < RPT / 8; ++g) {
      const int gv = VEC ? g : 0;
      if (!VEC && g > 0) gather(tab[c & 1], rrow + 8 * g, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const v8h w = {v[8 * gv][e],     v[8 * gv + 1][e], v[8 * gv + 2][e], v[8 * gv + 3][e],
                       v[8 * gv + 4][e], v[8 * gv + 5][e], v[8 * gv + 6][e], v[8 * gv + 7][e]};
        *reinterpret_cast<v8h*>(Xo + xoff(cg * 8 + e, rg * RPT + 8 * g)) = w;
      }
    }
    if (more) fill_rowtab(d, tab[(c + 1) & 1], r0 + CK, r_end, CK);
    __syncthreads();
    if (more) {  // next chunk's global loads overlap this chunk's MFMAs
      gather(tab[(c + 1) & 1], rrow, v);
    }
    if constexpr (DIAG) {
      if (want_col) {  // all 2 KC rows of column tid, in swizzled order
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int k = 0; k < KC; k += 8) {
            v8h cv = *reinterpret_cast<const v8h*>((h ? X1 : X0) + tid * LDK + k);
#pragma unroll
            for (int q = 0; q < 8; ++q) colsum += static_cast<float>(cv[q]);
          }
      }
      if (mma_on) {
        mma(X0, X0);
        mma(X1, X1);
      }
    } else {
      if (want_col) {  // the KC rows of column tid of the row operand, in swizzled order
#pragma unroll
        for (int k = 0; k < KC; k += 8) {
          v8h cv = *reinterpret_cast<const v8h*>(X0 + tid * LDK + k);
#pragma unroll
          for (int q = 0; q < 8; ++q) colsum += static_cast<float>(cv[q]);
        }
      }
      if (mma_on) mma(X0, X1);
    }
  }
}

__global__ void __launch_bounds__(256) syrk_f16_kernel(const SyrkDesc* __restrict__ desc,
                                                       const int32_t* __restrict__ begin, int count,
                                                       int32_t* __restrict__ next_item, int total, float decay) {
  __shared__ int s_item;  // the next item from the counter, longest items first
  if (threadIdx.x == 0) s_item = atomicAdd(next_item, 1);
  __syncthreads();
  const int v = s_item;
  if (v >= total) return;
  const int p = find_problem(begin, count, v);
  const SyrkDesc& d = desc[p];
  const int local = v - begin[p];
  const int t = local % d.nt, s = local / d.nt;
  const bool shp = d.kind == 1;  // a shift product: a rectangular grid of tiles
  int ti, tj;
  if (shp) {
    ti = t % d.nbr;
    tj = t / d.nbr;
  } else {
    upper_tile(t, d.nb, ti, tj);
  }
  const bool diag = !shp && ti == tj;

  __shared__ __attribute__((aligned(16))) _Float16 lds[2][ST * LDK];
  __shared__ RowTab tab[2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const bool skip = diag && wm > wn;  // quadrant strictly below the diagonal
  // rows of a shift product past C (C = 64: the lower half of the tile)
  const bool idle = shp && ti * ST + wm * 64 >= d.c_row;
  // a quadrant whose rows or columns all lie past the factor's last (order 64: three
  // of a diagonal tile's quadrants) multiplies zeros only
  const bool past = ti * ST + wm * 64 >= (shp ? d.c_row : d.d_core) || tj * ST + wn * 64 >= (shp ? d.c_col : d.d_core);
  ColTab ct;  // the 8 columns this thread stages: of row block tj in threads 128.. of an
              // off-diagonal tile, else of row block ti
  const int op = diag ? 0 : (tid >> 7);
  fill_coltab(d, op, (op ? tj : ti) * ST + (tid & 15) * 8, ct);
  const int r_begin = s * d.rows_per_split;
  const int r_end = min(d.R, r_begin + d.rows_per_split);
  const bool want_col = tid < ST && (shp ? tj == 0 : diag && d.bias);

  v16f acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;
  float colsum = 0.f;
  const bool mma_on = !skip && !idle && !past;
  // block-uniform specialisations of the main loop
  if (diag) {
    if (d.vec) syrk_rows<true, true>(d, tab, lds[0], lds[1], ct, r_begin, r_end, want_col, mma_on, acc, colsum);
    else syrk_rows<true, false>(d, tab, lds[0], lds[1], ct, r_begin, r_end, want_col, mma_on, acc, colsum);
  } else {
    if (d.vec) syrk_rows<false, true>(d, tab, lds[0], lds[1], ct, r_begin, r_end, want_col, mma_on, acc, colsum);
    else syrk_rows<false, false>(d, tab, lds[0], lds[1], ct, r_begin, r_end, want_col, mma_on, acc, colsum);
  }

  if (d.splits == 1) {
    // the descriptor's fields copied first (the stores could alias the table, which
    // the compiler would otherwise reload after every store); row offsets per row
    const int c_row = d.c_row, c_col = d.c_col, d_core = d.d_core;
    const int64_t dd = d.d;
    const float inv_r = d.inv_r;
    KG float* const out = gp(d.out);
    KG float* const full = gp(d.full);
    const int jb = tj * ST + wn * 64 + (lane & 31);
    if (shp) {  // raw sums into T, rows < C, columns < ntap * C
      if (!idle) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int i = ti * ST + wm * 64 + a * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
            KG float* const row = out + int64_t(i) * c_col;
#pragma unroll
            for (int b = 0; b < 2; ++b) {
              const int j = jb + b * 32;
              if (i < c_row && j < c_col) row[j] = acc[a][b][e];
            }
          }
      }
      if (want_col && ti * ST + tid < c_row) gp(d.csum)[ti * ST + tid] = colsum;
    } else {
      if (!skip) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int i = ti * ST + wm * 64 + a * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
            KG float* const row = out + (int64_t(i) * dd - (int64_t(i) * (i - 1)) / 2 - i);  // row[j] for j >= i
            KG float* const frow = full + int64_t(i) * dd;
#pragma unroll
            for (int b = 0; b < 2; ++b) {
              const int j = jb + b * 32;
              if (i <= j && j < d_core) {
                const float x = acc[a][b][e] * inv_r;
                const float v = decay != 0.f ? decay * row[j] + (1.f - decay) * x : x;
                row[j] = v;
                if (full) frow[j] = v;
              }
            }
          }
      }
      if (diag && d.bias) write_bias_direct(d, ti, t, colsum, decay);
    }
  } else {
    float* P = d.partial + (int64_t(s) * d.nt + t) * (ST * ST);
    if (!skip && !idle) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int r = wm * 64 + a * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
            const int cc = wn * 64 + b * 32 + (lane & 31);
            gp(P)[r * ST + cc] = acc[a][b][e];
          }
    }
    if (want_col) gp(d.pcol)[(int64_t(s) * d.nb + ti) * ST + tid] = colsum;
  }
}

// ---- 256x256 tiles ----------------------------------------------------------------
// Factors of order 256 and more and the shift products of 3x3 layers with 256 or more
// channels run on 256x256 output tiles: each 16-byte gather then feeds twice the MFMAs
// of a 128x128 tile (the 128x128 tiles are bound by issuing their gathers). A block of
// 512 threads (eight waves, each a 128x64 slab: rows wm*128.., columns wn*64..) stages
// 64-row chunks of its two 256-column operands (a diagonal tile: 128-row chunks of its
// one operand, halves in the two operand slots) in double-buffered LDS: the gathers of
// chunk c+2 and the stores of chunk c+1 run during the MFMAs of chunk c, with one
// barrier per chunk. The LDS layout and the 8x8 register transpose are those of the
// 128x128 tiles at a 64-row pitch. Results go out as the 128x128 sub-tiles of the
// other kernel (packed factor, dense T, or split partials in the same layout), so the
// split reduction and the shift assembly read them unchanged.
constexpr int BT = 256;      // big tile edge
constexpr int KB = 64;       // patch rows per LDS operand buffer (big tiles)
constexpr int LDB = KB + 8;  // LDS row pitch in halves (144 B)
constexpr int BT_LDS_HALVES = 2 * 2 * BT * LDB;  // [buffer][operand][column][row]

__device__ __forceinline__ int xoffb(int m, int k) {
  return m * LDB + ((((k >> 3) ^ (m >> 3) ^ (m >> 4)) & 7) << 3) + (k & 7);
}

// Row loop of a big tile over patch rows [r_begin, r_end), 16-byte gathers only.
// mma_on (wave-uniform): the wave's slab is needed; lo_on: its lower 64 rows too (not
// when they lie below the diagonal of a diagonal sub-tile or past the last row).
template <bool DIAG>
__device__ __forceinline__ void big_rows(const SyrkDesc& d, RowTab* tab, _Float16* lds, const ColTab& ct,
                                         int r_begin, int r_end, bool want_col, bool mma_on, bool lo_on,
                                         v16f (&acc)[4][2], float& colsum) {
  constexpr int CK = DIAG ? 2 * KB : KB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  // staging: thread = (operand slot op, column group cg of 8, row group rg of 8)
  const int op = tid >> 8, cg = tid & 31, rg = (tid >> 5) & 7;
  const int rrow = (DIAG ? op * KB : 0) + rg * 8;
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(d.src), 0, d.nbytes, 0x00020000);
  const int H = d.H, W = d.W;
  auto slot = [&](int b, int o) { return lds + (b * 2 + o) * (BT * LDB); };
  auto stage = [&](const v8h(&v)[8], int b) {
    _Float16* X = slot(b, op);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const v8h w = {v[0][e], v[1][e], v[2][e], v[3][e], v[4][e], v[5][e], v[6][e], v[7][e]};
      *reinterpret_cast<v8h*>(X + xoffb(cg * 8 + e, rg * 8)) = w;
    }
  };
  // one 16-deep step of the slab: the upper 64 rows' operands first, the lower 64
  // rows' read while the upper MFMAs run (fewer operand registers live at once)
  auto step = [&](const _Float16* A, const _Float16* B, int ks) {
    const int ko = ks * 16 + (lane >> 5) * 8;
    v8h a[2], b[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = *reinterpret_cast<const v8h*>(B + xoffb(wn * 64 + 32 * j + (lane & 31), ko));
#pragma unroll
    for (int i = 0; i < 2; ++i) a[i] = *reinterpret_cast<const v8h*>(A + xoffb(wm * 128 + 32 * i + (lane & 31), ko));
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    if (lo_on) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const v8h*>(A + xoffb(wm * 128 + 64 + 32 * i + (lane & 31), ko));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[2 + i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[2 + i][j], 0, 0, 0);
    }
  };
  const int nch = (r_end - r_begin + CK - 1) / CK;
  fill_rowtab(d, tab[0], r_begin, r_end, CK);
  if (nch > 1) fill_rowtab(d, tab[1], r_begin + CK, r_end, CK);
  __syncthreads();
  v8h v[8];
  gather8_vec<8>(rsrc, H, W, tab[0], rrow, ct, v);
  stage(v, 0);
  if (nch > 1) gather8_vec<8>(rsrc, H, W, tab[1], rrow, ct, v);
  if (nch > 2) fill_rowtab(d, tab[2], r_begin + 2 * CK, r_end, CK);
  __syncthreads();
  // Each 16-deep step's MFMAs are followed by a share of the staging, which runs while
  // the matrix unit works on them (and the other wave on the SIMD fills the gaps): after
  // step 0 and 1 the stores of chunk c+1 (columns 0-3, 4-7 of each thread's 8x8 block)
  // into the other buffer, last read before the previous barrier; after step 2 the
  // gathers of chunk c+2; after step 3 every wave's share of chunk c+3's row table (its
  // slot last read for chunk c); after the last step the column sums of the row operand
  // (a column per thread, half the chunk's rows each). Nothing here depends on chunk c's
  // products; the barrier at the end of the chunk orders everything across waves.
  constexpr int NS = DIAG ? 8 : 4;  // 16-deep steps per chunk
  const int tl = lane < CK / 8 ? wave * (CK / 8) + lane : CK;  // this thread's table entry (CK: none)
  const int chalf = tid >> 8;
  for (int c = 0; c < nch; ++c) {
    const int cur = c & 1;
    const bool st = c + 1 < nch, ga = c + 2 < nch, tb = c + 3 < nch;
    _Float16* Xs = slot(cur ^ 1, op);
#pragma unroll
    for (int ks = 0; ks < NS; ++ks) {
      const _Float16* A = slot(cur, (DIAG && ks >= 4) ? 1 : 0);
      const _Float16* B = DIAG ? A : slot(cur, 1);
      if (mma_on) step(A, B, ks & 3);
      __builtin_amdgcn_sched_barrier(0);
      if ((ks == 0 || ks == 1) && st) {
#pragma unroll
        for (int e = 4 * ks; e < 4 * ks + 4; ++e) {
          const v8h w = {v[0][e], v[1][e], v[2][e], v[3][e], v[4][e], v[5][e], v[6][e], v[7][e]};
          *reinterpret_cast<v8h*>(Xs + xoffb(cg * 8 + e, rg * 8)) = w;
        }
      }
      if (ks == 2 && ga) gather8_vec<8>(rsrc, H, W, tab[(c + 2) % 3], rrow, ct, v);
      if (ks == 3 && tb) fill_rowtab_at(d, tab[c % 3], r_begin + (c + 3) * CK, r_end, CK, tl);
      if (ks == NS - 1 && want_col) {
        const _Float16* X = slot(cur, DIAG ? chalf : 0) + (tid & (BT - 1)) * LDB + (DIAG ? 0 : 32 * chalf);
#pragma unroll
        for (int k = 0; k < (DIAG ? KB : KB / 2); k += 8) {
          const v8h cv = *reinterpret_cast<const v8h*>(X + k);
#pragma unroll
          for (int q = 0; q < 8; ++q) colsum += static_cast<float>(cv[q]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
  }
  if (want_col) {  // threads t and t + 256 summed the two halves of column t
    float* part = reinterpret_cast<float*>(tab);
    if (tid >= BT) part[tid - BT] = colsum;
    __syncthreads();
    if (tid < BT) colsum += part[tid];
  }
}

__global__ void __launch_bounds__(512) syrk_big_kernel(const SyrkDesc* __restrict__ desc,
                                                       const int32_t* __restrict__ begin, int count,
                                                       int32_t* __restrict__ next_item, int total, float decay) {
  __shared__ int s_item;
  if (threadIdx.x == 0) s_item = atomicAdd(next_item, 1);
  __syncthreads();
  const int v = s_item;
  if (v >= total) return;
  const int p = find_problem(begin, count, v);
  const SyrkDesc& d = desc[p];
  const int local = v - begin[p];
  const int t = local % d.nt2, s = local / d.nt2;
  const bool shp = d.kind == 1;
  int TI, TJ;
  if (shp) {
    TI = t % d.nbr2;
    TJ = t / d.nbr2;
  } else {
    upper_tile(t, d.nb2, TI, TJ);
  }
  const bool diag = !shp && TI == TJ;

  __shared__ __attribute__((aligned(16))) _Float16 lds[BT_LDS_HALVES];
  __shared__ RowTab tab[3];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int rlim = shp ? d.c_row : d.d_core, clim = shp ? d.c_col : d.d_core;
  const int row0 = TI * BT + wm * 128, col0 = TJ * BT + wn * 64;
  // the slab below the diagonal of a diagonal tile, or past the valid rows or columns
  const bool mma_on = !(diag && wm == 1 && wn < 2) && row0 < rlim && col0 < clim;
  // rows 64.. of the slab: below the diagonal of a diagonal sub-tile, or past the rows
  const bool lo_on = !(diag && wm == (wn >> 1) && (wn & 1) == 0) && row0 + 64 < rlim;
  ColTab ct;  // the 8 columns this thread stages
  const int op = diag ? 0 : (tid >> 8);
  fill_coltab(d, op, (op ? TJ : TI) * BT + (tid & 31) * 8, ct);
  const int r_begin = s * d.rows_per_split;
  const int r_end = min(d.R, r_begin + d.rows_per_split);
  const bool want_cols = shp ? TJ == 0 : diag && d.bias;  // the block forms column sums
  const bool want_col = tid < BT && want_cols;               // this thread holds column tid's

  v16f acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;
  float colsum = 0.f;
  if (diag) big_rows<true>(d, tab, lds, ct, r_begin, r_end, want_cols, mma_on, lo_on, acc, colsum);
  else big_rows<false>(d, tab, lds, ct, r_begin, r_end, want_cols, mma_on, lo_on, acc, colsum);

  const int na = lo_on ? 4 : 2;
  if (d.splits == 1) {
    if (mma_on) {
      // Branch-free stores through a raw buffer over the output (under 2^31 bytes, as
      // the host checks): an entry outside the valid part gets an offset beyond the
      // buffer's range and is dropped. Row offsets once per accumulator row, in 32 bits.
      // The descriptor's fields are copied first: the stores could alias the table, so
      // the compiler would otherwise reload them after every store.
      const int c_row = d.c_row, c_col = d.c_col, d_core = d.d_core, dd = d.d;
      const float inv_r = d.inv_r;
      const unsigned lim = shp ? unsigned(c_row) * unsigned(c_col) : unsigned(dd) * unsigned(dd + 1) / 2u;
      const __amdgpu_buffer_rsrc_t orsrc =
          __builtin_amdgcn_make_buffer_rsrc(d.out, 0, static_cast<int>(lim * 4u), 0x00020000);
      const int jl = col0 + (lane & 31);
      // entry (a, b, e) of the slab: row i = i0 + a*32 + 8*(e/4) + e%4, column jl + b*32
      const int i0 = row0 + 4 * (lane >> 5);
      auto each = [&](auto&& put) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
          if (a < na)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int i = i0 + a * 32 + 8 * (e >> 2) + (e & 3);
#pragma unroll
              for (int b = 0; b < 2; ++b) put(i, jl + b * 32, acc[a][b][e]);
            }
      };
      if (shp) {  // raw sums of T, row i at i * c_col
        each([&](int i, int j, float x) {
          const bool ok = i < c_row && j < c_col;
          const unsigned off = ok ? (unsigned(i) * unsigned(c_col) + unsigned(j)) * 4u : 0x80000000u;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), orsrc, off, 0, 0);
        });
      } else {  // the factor scaled by 1/R, entry (i, j >= i) at i*d - i(i-1)/2 + j - i
        auto off_of = [&](int i, int j) {
          const unsigned ui = static_cast<unsigned>(i);
          const bool ok = i <= j && j < d_core;
          return ok ? (ui * unsigned(dd) - (ui * (ui - 1u)) / 2u - ui + unsigned(j)) * 4u : 0x80000000u;
        };
        // the full matrix's rows from the slab's first one: a buffer based there, so that
        // the offsets stay small (under 128 rows of the factor)
        KG float* const full = gp(d.full);
        const int64_t fbytes = int64_t(dd - row0) * dd * 4;  // <= 0 for a slab past the last row
        const unsigned frec = fbytes <= 0 ? 0u : fbytes > 0x7fffff00 ? 0x7fffff00u : unsigned(fbytes);
        const __amdgpu_buffer_rsrc_t frsrc = __builtin_amdgcn_make_buffer_rsrc(
            full + int64_t(row0) * dd, 0, static_cast<int>(frec), 0x00020000);
        auto foff_of = [&](int i, int j) {
          const bool ok = i <= j && j < d_core;
          return ok ? (unsigned(i - row0) * unsigned(dd) + unsigned(j)) * 4u : 0x80000000u;
        };
        if (decay == 0.f && full) {
          each([&](int i, int j, float x) {
            const unsigned v = __float_as_uint(x * inv_r);
            __builtin_amdgcn_raw_buffer_store_b32(v, orsrc, off_of(i, j), 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(v, frsrc, foff_of(i, j), 0, 0);
          });
        } else if (decay == 0.f) {
          each([&](int i, int j, float x) {
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x * inv_r), orsrc, off_of(i, j), 0, 0);
          });
        } else {  // blended with the stored factor
          each([&](int i, int j, float x) {
            const unsigned off = off_of(i, j);
            const float old = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(orsrc, off, 0, 0));
            const unsigned v = __float_as_uint(decay * old + (1.f - decay) * (x * inv_r));
            __builtin_amdgcn_raw_buffer_store_b32(v, orsrc, off, 0, 0);
            if (full) __builtin_amdgcn_raw_buffer_store_b32(v, frsrc, foff_of(i, j), 0, 0);
          });
        }
      }
    }
    if (shp) {
      if (want_col && TI * BT + tid < d.c_row) gp(d.csum)[TI * BT + tid] = colsum;
    } else if (want_col) {  // the bias column and, from the first tile, the corner
      const int i = TI * BT + tid;
      if (i < d.d_core) {
        const int64_t o = packed_off(i, d.d_core, d.d);
        put_entry(d, o, i, d.d_core, blend(colsum * d.inv_r, d.out, o, decay));
      }
      if (TI == 0 && tid == 0) {
        const int64_t o = packed_off(d.d_core, d.d_core, d.d);
        put_entry(d, o, d.d_core, d.d_core, blend(d.r_f * d.inv_r, d.out, o, decay));
      }
    }
  } else {
    // the slab's 128x128 sub-tile (si, sj) in the partial layout of the other kernel
    const int si = 2 * TI + wm, sj = 2 * TJ + (wn >> 1);
    const bool valid = shp ? (si < d.nbr && sj < d.nbc) : (si <= sj && sj < d.nb);
    if (mma_on && valid) {
      const int t128 = shp ? si + sj * d.nbr : si * d.nb - (si * (si - 1)) / 2 + (sj - si);
      float* P = d.partial + (int64_t(s) * d.nt + t128) * (ST * ST);
#pragma unroll
      for (int a = 0; a < 4; ++a)
        if (a < na)
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int r = a * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
              const int cc = (wn & 1) * 64 + b * 32 + (lane & 31);
              gp(P)[r * ST + cc] = acc[a][b][e];
            }
    }
    if (want_col) {
      const int bi = 2 * TI + (tid >> 7);
      if (bi < d.nb) gp(d.pcol)[(int64_t(s) * d.nb + bi) * ST + (tid & (ST - 1))] = colsum;
    }
  }
}

// fp32 inputs: element gathers into LDS laid out [k][column], fp32 MFMA.
__global__ void __launch_bounds__(256) syrk_f32_kernel(const SyrkDesc* __restrict__ desc,
                                                       const int32_t* __restrict__ begin,
                                                       int count, XcdSegs segs, float decay) {
  const int v = seg_item(blockIdx.x, segs);
  if (v < 0) return;
  const int p = find_problem(begin, count, v);
  const SyrkDesc& d = desc[p];
  const int local = v - begin[p];
  const int t = local % d.nt, s = local / d.nt;
  int ti, tj;
  upper_tile(t, d.nb, ti, tj);
  const bool diag = ti == tj;

  __shared__ float la[KC32 * LDN32], lb[KC32 * LDN32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const bool skip = diag && wm > wn;
  const int r_begin = s * d.rows_per_split;
  const int r_end = min(d.R, r_begin + d.rows_per_split);
  const bool want_col = diag && d.bias && tid < ST;

  v16f acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;
  float colsum = 0.f;

  for (int r0 = r_begin; r0 < r_end; r0 += KC32) {
    __syncthreads();
    for (int e = tid; e < KC32 * ST; e += 256) {
      const int k = e / ST, c = e % ST;
      const int row = r0 + k;
      const bool ok = row < r_end;
      la[k * LDN32 + c] = ok ? x_elem<float>(d, row, ti * ST + c) : 0.f;
      lb[k * LDN32 + c] = ok ? x_elem<float>(d, row, tj * ST + c) : 0.f;
    }
    __syncthreads();
    if (want_col)
      for (int k = 0; k < KC32; ++k) colsum += la[k * LDN32 + tid];
    if (!skip) {
      for (int k = 0; k < KC32; k += 2) {
        const int kk = k + (lane >> 5);
        const float a0 = la[kk * LDN32 + wm * 64 + (lane & 31)];
        const float a1 = la[kk * LDN32 + wm * 64 + 32 + (lane & 31)];
        const float b0 = lb[kk * LDN32 + wn * 64 + (lane & 31)];
        const float b1 = lb[kk * LDN32 + wn * 64 + 32 + (lane & 31)];
        acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
        acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
        acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
      }
    }
  }
  if (d.splits == 1) {
    if (!skip) {
      for (int a = 0; a < 2; ++a)
        for (int b = 0; b < 2; ++b)
          for (int e = 0; e < 16; ++e) {
            const int i = ti * ST + wm * 64 + a * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
            const int j = tj * ST + wn * 64 + b * 32 + (lane & 31);
            if (i <= j && j < d.d_core) {
              const int64_t o = packed_off(i, j, d.d);
              put_entry(d, o, i, j, blend(acc[a][b][e] * d.inv_r, d.out, o, decay));
            }
          }
    }
    if (diag && d.bias) write_bias_direct(d, ti, t, colsum, decay);
  } else {
    float* P = d.partial + (int64_t(s) * d.nt + t) * (ST * ST);
    if (!skip) {
      for (int a = 0; a < 2; ++a)
        for (int b = 0; b < 2; ++b)
          for (int e = 0; e < 16; ++e) {
            const int r = wm * 64 + a * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
            const int c = wn * 64 + b * 32 + (lane & 31);
            gp(P)[r * ST + c] = acc[a][b][e];
          }
    }
    if (want_col) gp(d.pcol)[(int64_t(s) * d.nb + ti) * ST + tid] = colsum;
  }
}

// Adds the row-split partial tiles in split order, scales, blends and packs. One
// block per 1024 entries of a tile (RED_PARTS blocks per tile), 4 entries per thread.
constexpr int RED_PARTS = ST * ST / 1024;

__global__ void __launch_bounds__(256) syrk_reduce_kernel(const SyrkDesc* __restrict__ desc,
                                                          const int32_t* __restrict__ rbegin,
                                                          const int32_t* __restrict__ rprob,
                                                          int rcount, float decay) {
  const int q = find_problem(rbegin, rcount, blockIdx.x);
  const SyrkDesc& d = desc[rprob[q]];
  const int local = blockIdx.x - rbegin[q];
  const int t = local / RED_PARTS, part = local % RED_PARTS;
  if (d.kind == 1) {  // a shift product: dense raw sums, and the row operand's column sums
    const int ti = t % d.nbr, tj = t / d.nbr;
    const int64_t tstride = int64_t(d.nt) * ST * ST;
    const int e0 = part * 1024 + threadIdx.x * 4;
    const int i = ti * ST + e0 / ST, j0 = tj * ST + e0 % ST;
    if (i < d.c_row && j0 < d.c_col) {
      const KG float* P = gp(d.partial) + int64_t(t) * ST * ST + e0;
      v4f sum = {0.f, 0.f, 0.f, 0.f};
      constexpr int U = 8;
      int s = 0;
      for (; s + U <= d.splits; s += U) {
        v4f x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = *reinterpret_cast<const KG v4f*>(P + (s + u) * tstride);
#pragma unroll
        for (int u = 0; u < U; ++u) sum += x[u];
      }
      for (; s < d.splits; ++s) sum += *reinterpret_cast<const KG v4f*>(P + s * tstride);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (j0 + u < d.c_col) gp(d.out)[int64_t(i) * d.c_col + j0 + u] = sum[u];
    }
    if (part == 0 && tj == 0 && threadIdx.x < ST && ti * ST + int(threadIdx.x) < d.c_row) {
      const KG float* pc = gp(d.pcol) + int64_t(ti) * ST + threadIdx.x;
      const int64_t sstride = int64_t(d.nb) * ST;
      float sum = 0.f;
      for (int s = 0; s < d.splits; ++s) sum += pc[s * sstride];
      gp(d.csum)[ti * ST + threadIdx.x] = sum;
    }
    return;
  }
  int ti, tj;
  upper_tile(t, d.nb, ti, tj);  const int64_t tstride = int64_t(d.nt) * ST * ST;
  const int e0 = part * 1024 + threadIdx.x * 4;
  const int i = ti * ST + e0 / ST, j0 = tj * ST + e0 % ST;
  if (i < d.d_core && j0 + 3 >= i && j0 < d.d_core) {
    const float* P = d.partial + int64_t(t) * ST * ST + e0;
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
    // eight splits' loads in flight, then added in split order
    constexpr int U = 8;
    int s = 0;
    for (; s + U <= d.splits; s += U) {
      v4f x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) x[u] = *reinterpret_cast<const KG v4f*>(gp(P) + (s + u) * tstride);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        sum.x += x[u].x; sum.y += x[u].y; sum.z += x[u].z; sum.w += x[u].w;
      }
    }
    for (; s < d.splits; ++s) {
      const v4f x = *reinterpret_cast<const KG v4f*>(gp(P) + s * tstride);
      sum.x += x.x; sum.y += x.y; sum.z += x.z; sum.w += x.w;
    }
    const float v4[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + u;
      if (j >= i && j < d.d_core) {
        const int64_t o = packed_off(i, j, d.d);
        put_entry(d, o, i, j, blend(v4[u] * d.inv_r, d.out, o, decay));
      }
    }
  }
  if (part == 0 && ti == tj && d.bias && threadIdx.x < ST) {
    const int ib = ti * ST + threadIdx.x;
    if (ib < d.d_core) {
      const KG float* pc = gp(d.pcol) + int64_t(ti) * ST + threadIdx.x;
      const int64_t sstride = int64_t(d.nb) * ST;
      float sum = 0.f;
      int s = 0;
      for (; s + 8 <= d.splits; s += 8) {
        float x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = pc[(s + u) * sstride];
#pragma unroll
        for (int u = 0; u < 8; ++u) sum += x[u];
      }
      for (; s < d.splits; ++s) sum += pc[s * sstride];
      const int64_t o = packed_off(ib, d.d_core, d.d);
      put_entry(d, o, ib, d.d_core, blend(sum * d.inv_r, d.out, o, decay));
    }
  }
  if (t == 0 && part == 0 && d.bias && threadIdx.x == 0) {
    const int64_t o = packed_off(d.d_core, d.d_core, d.d);
    put_entry(d, o, d.d_core, d.d_core, blend(d.r_f * d.inv_r, d.out, o, decay));
  }
}

// ---- 3x3 activation factors from shift products ---------------------------------
// For a 3x3 convolution with stride 1 and zero padding 1, column t*C + c of the patch
// matrix is channel c of the pixel o + (i-1, j-1) for tap t = 3i + j and output
// position o. Block (t1, t2) of A sums x[u][c1] x[u + delta][c2], delta = tap t2's offset
// minus tap t1's, over the pixels u that tap t1 sees: all pixels u with u + delta inside
// the image, except that tap row i1 = 0 never sees the last image row and i1 = 2 never
// the first (the same for the columns). With the full-image shift product
//   T_delta[c1][c2] = sum over all pixels u of x[u][c1] x[u + delta][c2]
// (zero outside the image), a block is therefore T_delta minus a one-row strip when
// delta_h = 0 and i1 != 1, minus a one-column strip when delta_w = 0 and j1 != 1, plus
// the corner pixel where both were taken off. With t1 <= t2, delta is one of 13 offsets
// (delta_h = 0, delta_w = 0..2; delta_h = 1, 2, delta_w = -2..2), so A's upper triangle
// needs 13 C x C products over all rows instead of 45 blocks, plus strips over one
// image row or column: about three times fewer multiplications. The bias column is the
// column sum over the pixels each tap sees, formed the same way.
// Per layer the workspace region holds (floats): T [C][13C]; row strips [2][C][3C]
// (top, bottom; taps (0,0), (0,1), (0,2)); column strips [2][C][3C] (left, right; taps
// (0,0), (1,0), (2,0)); corners [4][C][C] (top-left, top-right, bottom-left,
// bottom-right); column sums [9][C] (all pixels, the two row strips, the two column
// strips, the four corners).
constexpr int kShiftTaps = 13;
__host__ __device__ inline int64_t sr_rows(int C) { return int64_t(13) * C * C; }           // row strips
__host__ __device__ inline int64_t sr_cols(int C) { return int64_t(19) * C * C; }           // column strips
__host__ __device__ inline int64_t sr_corners(int C) { return int64_t(25) * C * C; }
__host__ __device__ inline int64_t sr_sums(int C) { return int64_t(29) * C * C; }
__host__ __device__ inline int64_t sr_floats(int C) { return int64_t(29) * C * C + 9 * C; }
__host__ __device__ inline int tap_index(int dh, int dw) { return dh == 0 ? dw : 3 + (dh - 1) * 5 + (dw + 2); }

struct ShiftAsm {
  const float* base;  // the layer's region
  float* out;         // packed A
  float* full;        // NULL, or A row-major d x d: the upper triangle written as well
  int32_t C, d, bias, pad_;
  float inv_r, r_f;
};

// One block per channel c1 of a job (blocks of all jobs numbered by offsets `begin`):
// the nine packed rows i = t1*C + c1 of A (t1 = 0..8), which all read row c1 of T and
// of the strips (cache hits after the first), block 0 also the bias corner. Within a
// row, the columns of one tap t2 are a segment on which delta and the strips that apply
// are fixed: an entry loads only the terms that apply to its segment and forms its
// value in the same order as everywhere (T, minus the row strip, minus the column
// strip, plus the corner). Every entry times fp32(1/R), blended with the stored factor
// when decay != 0, goes to the packed factor and, when asked for, to the full matrix.
__global__ void __launch_bounds__(256) shift_assemble_kernel(const ShiftAsm* __restrict__ jobs,
                                                             const int32_t* __restrict__ begin, int count,
                                                             float decay) {
  const int q = find_problem(begin, count, blockIdx.x);
  const ShiftAsm& a = jobs[q];
  const int c1 = blockIdx.x - begin[q];
  const int C = a.C, d = a.d, tid = threadIdx.x;
  const int64_t C3 = int64_t(3) * C;
  // the region is only read and the factor only written here: restrict lets every
  // group's loads issue before the previous groups' stores
  const KG float* __restrict__ T = gp(a.base) + int64_t(c1) * (kShiftTaps * C);
  const KG float* __restrict__ Su = gp(a.base) + sr_sums(C);
  const KG float* __restrict__ R0 = gp(a.base) + sr_rows(C) + int64_t(c1) * C3;    // + hs*3C^2 + dw*C + c2
  const KG float* __restrict__ C0 = gp(a.base) + sr_cols(C) + int64_t(c1) * C3;    // + ws*3C^2 + dh*C + c2
  const KG float* __restrict__ X0 = gp(a.base) + sr_corners(C) + int64_t(c1) * C;  // + (2hs+ws)*C^2 + c2
  const int64_t cc = int64_t(C) * C;
  KG float* const full = gp(a.full);
  const float inv_r = a.inv_r;
  // j / C by a shift when C is a power of two (block-uniform choice)
  const bool pow2 = (C & (C - 1)) == 0;
  const int lg = 31 - __builtin_clz(static_cast<unsigned>(C));
  // entry (i, j) from its unscaled value: o its packed address, f its full one
  auto put = [&](KG float* o, KG float* f, float v) {
    const float x = v * inv_r;
    const float y = decay != 0.f ? decay * *o + (1.f - decay) * x : x;
    *o = y;
    if (full) *f = y;
  };
  if (a.bias && c1 == 0 && tid == 0)
    put(gp(a.out) + packed_off(d - 1, d - 1, d), full + (int64_t(d) * d - 1), a.r_f);
  for (int t1 = 0; t1 < 9; ++t1) {
    const int i = t1 * C + c1, i1 = t1 / 3, j1 = t1 - 3 * i1;
    const int hs = i1 == 0 ? 1 : 0, ws = j1 == 0 ? 1 : 0;  // strips left out: bottom/top, right/left
    KG float* __restrict__ orow = gp(a.out) + packed_off(i, i, d) - i;  // orow[j] for j >= i
    KG float* __restrict__ frow = full + int64_t(i) * d;
    if (a.bias && tid == 0) {  // the bias column: sum over the pixels tap t1 sees
      float bias_v = Su[c1];
      if (i1 != 1) bias_v -= Su[(1 + hs) * C + c1];
      if (j1 != 1) bias_v -= Su[(3 + ws) * C + c1];
      if (i1 != 1 && j1 != 1) bias_v += Su[(5 + 2 * hs + ws) * C + c1];
      put(orow + (d - 1), frow + (d - 1), bias_v);
    }
    // entries j = i .. 9C-1 of the row, consecutive across the threads (coalesced stores),
    // U per thread with their loads in flight before any store; only the terms that apply
    // to an entry's segment are loaded (the segment changes within a wave only at its
    // boundaries)
    constexpr int U = 8;
    const int jend = 9 * C;
    for (int jb = i + tid; jb < jend; jb += 256 * U) {
      float xt[U], xr[U], xc[U], xx[U];
      bool fr[U], fc[U], fx[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = min(jb + 256 * u, jend - 1);
        const int t2 = pow2 ? (j >> lg) : j / C, c2 = j - t2 * C, i2 = t2 / 3, j2 = t2 - 3 * i2;
        const int dh = i2 - i1, dw = j2 - j1;
        fr[u] = dh == 0 && i1 != 1;
        fc[u] = dw == 0 && j1 != 1;
        fx[u] = fr[u] && fc[u];
        xt[u] = T[tap_index(dh, dw) * C + c2];
        xr[u] = fr[u] ? R0[hs * C3 * C + dw * C + c2] : 0.f;
        xc[u] = fc[u] ? C0[ws * C3 * C + dh * C + c2] : 0.f;
        xx[u] = fx[u] ? X0[(2 * hs + ws) * cc + c2] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = jb + 256 * u;
        if (j >= jend) continue;
        float x = xt[u];
        if (fr[u]) x -= xr[u];
        if (fc[u]) x -= xc[u];
        if (fx[u]) x += xx[u];
        put(orow + j, frow + j, x);
      }
    }
  }
}

// ---- host planning ------------------------------------------------------------
// A patch matrix written out before the factor pass: for fp16 convolutions whose
// channel count rules out 16-byte gathers from the NHWC tensor (e.g. 3 input
// channels), element gathers cost several times the 16-byte ones per patch row, so
// the rows are gathered once into the workspace (row pitch ld = d_core rounded up to
// 8, zeros past d_core) and the factor pass reads them as plain rows with 16-byte
// loads. The conv geometry is kept here; the factor problem becomes a row problem.
struct Im2Row {
  const _Float16* src;
  _Float16* dst;
  int32_t R, ld, d_core, H, W, C, Ho, Wo, kh, kw, sh, sw, ph, pw;
  double rhw, rwo;
};

__global__ void __launch_bounds__(256) im2row_kernel(Im2Row j, int64_t total) {
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;  // (row, group of 8 columns)
  if (e >= total) return;
  const int groups = j.ld / 8;
  const int row = static_cast<int>(e / groups), c0 = static_cast<int>(e - int64_t(row) * groups) * 8;
  const int hw = j.Ho * j.Wo;
  const int n = fast_div(row, hw, j.rhw);
  const int rem = row - n * hw;
  const int oh = fast_div(rem, j.Wo, j.rwo);
  const int ow = rem - oh * j.Wo;
  const int ih0 = oh * j.sh - j.ph, iw0 = ow * j.sw - j.pw;
  const KG _Float16* src = gp(j.src) + int64_t(n) * j.H * j.W * j.C;
  // column c0 decoded once, then stepped: c = (ki * kw + kj) * C + ci
  const int tap = c0 / j.C;
  int ci = c0 - tap * j.C, ki = tap / j.kw, kj = tap - ki * j.kw;
  v8h v;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    _Float16 x = static_cast<_Float16>(0.f);
    const int ih = ih0 + ki, iw = iw0 + kj;
    if (c0 + q < j.d_core && unsigned(ih) < unsigned(j.H) && unsigned(iw) < unsigned(j.W))
      x = src[(int64_t(ih) * j.W + iw) * j.C + ci];
    v[q] = x;
    if (++ci == j.C) {
      ci = 0;
      if (++kj == j.kw) {
        kj = 0;
        ++ki;
      }
    }
  }
  *reinterpret_cast<KG v8h*>(gp(j.dst) + int64_t(row) * j.ld + c0) = v;
}

struct SyrkPlan {
  std::vector<SyrkDesc> desc;
  std::vector<Im2Row> im2row;        // patch matrices written out first (dst set at launch)
  std::vector<int32_t> im2row_prob;  // the problem in desc that reads each
  size_t im2row_bytes = 0;
  std::vector<int32_t> begin;        // work-item offsets (each launch's problems from 0)
  std::vector<int32_t> rbegin, rprob;  // reduce tiles of split problems
  int64_t items = 0, ritems = 0;     // items of the 128x128 launch, reduce blocks
  int64_t items_big = 0;             // items of the 256x256 launch
  int nbig = 0;                      // problems desc[0, nbig) run on 256x256 tiles
  size_t partial_floats = 0;
  XcdSegs segs{};
  int64_t seg_max = 0;               // longest XCD segment (items) of the 128x128 launch
  // 3x3 activation factors formed from shift products: one assembly job per layer,
  // its region (sr_floats(C) floats) carved at launch; problem p of kind 1 belongs to
  // job shift_job[p] as sub-problem shift_sub[p]
  std::vector<ShiftAsm> jobs;
  std::vector<int32_t> jbegin;       // assembly tiles
  std::vector<int32_t> shift_job, shift_sub;
  int64_t jtiles = 0;
  size_t shift_floats = 0;
};

// Whether layer L's activation factor is formed from shift products: fp16 inputs, a
// 3x3 kernel with stride 1 and padding 1, channels in groups of 8.
static bool shift_eligible(const kfac_layer& L, kfac_dtype dt) {
  return dt == KFAC_F16 && L.kh == 3 && L.kw == 3 && L.sh == 1 && L.sw == 1 && L.ph == 1 && L.pw == 1 &&
         L.c_in % 8 == 0 && L.h_out == L.h && L.w_out == L.w && int64_t(L.c_in) * kShiftTaps <= 65536;
}

// Sub-problem `sub` of the shift products of a 3x3 layer: 0 the full image (13 taps),
// 1/2 the top/bottom row, 3/4 the left/right column (3 taps each), 5..8 the corners
// top-left, top-right, bottom-left, bottom-right (1 tap). Its rows are the pixels of
// the window, in mode-1 form: stride 1, padding minus the window's origin.
static SyrkDesc make_shift(const kfac_layer& L, int sub) {
  static const int8_t full_dh[kShiftTaps] = {0, 0, 0, 1, 1, 1, 1, 1, 2, 2, 2, 2, 2};
  static const int8_t full_dw[kShiftTaps] = {0, 1, 2, -2, -1, 0, 1, 2, -2, -1, 0, 1, 2};
  SyrkDesc d{};
  d.kind = 1;
  d.mode = 1;
  d.H = L.h; d.W = L.w; d.C = L.c_in;
  int oh0 = 0, ow0 = 0, ho = L.h, wo = L.w;
  if (sub == 0) {
    d.ntap = kShiftTaps;
    for (int t = 0; t < kShiftTaps; ++t) { d.tdh[t] = full_dh[t]; d.tdw[t] = full_dw[t]; }
  } else if (sub <= 2) {           // row strip
    oh0 = sub == 1 ? 0 : L.h - 1;
    ho = 1;
    d.ntap = 3;
    for (int t = 0; t < 3; ++t) { d.tdh[t] = 0; d.tdw[t] = static_cast<int8_t>(t); }
  } else if (sub <= 4) {           // column strip
    ow0 = sub == 3 ? 0 : L.w - 1;
    wo = 1;
    d.ntap = 3;
    for (int t = 0; t < 3; ++t) { d.tdh[t] = static_cast<int8_t>(t); d.tdw[t] = 0; }
  } else {                         // corner
    const int k = sub - 5;
    oh0 = (k >> 1) ? L.h - 1 : 0;
    ow0 = (k & 1) ? L.w - 1 : 0;
    ho = wo = 1;
    d.ntap = 1;
  }
  d.Ho = ho; d.Wo = wo;
  d.sh = d.sw = 1; d.kh = d.kw = 1;
  d.ph = -oh0; d.pw = -ow0;
  d.R = L.n * ho * wo;
  d.rhw = 1.0 / static_cast<double>(int64_t(ho) * wo);
  d.rwo = 1.0 / static_cast<double>(wo);
  d.c_row = L.c_in;
  d.c_col = d.ntap * L.c_in;
  d.d_core = d.c_col;
  d.d = d.c_col;
  d.nbr = (d.c_row + ST - 1) / ST;
  d.nbc = (d.c_col + ST - 1) / ST;
  d.nb = d.nbr;
  d.nt = d.nbr * d.nbc;
  d.nbr2 = (d.c_row + BT - 1) / BT;
  d.nbc2 = (d.c_col + BT - 1) / BT;
  d.nb2 = d.nbr2;
  d.nt2 = d.nbr2 * d.nbc2;
  return d;
}

// Where sub-problem `sub` writes in a region: (products, column sums), offsets in floats.
static void shift_out(int C, int sub, int64_t& prod, int64_t& sums) {
  const int64_t c2 = int64_t(C) * C;
  if (sub == 0) prod = 0;
  else if (sub <= 2) prod = sr_rows(C) + (sub - 1) * 3 * c2;
  else if (sub <= 4) prod = sr_cols(C) + (sub - 3) * 3 * c2;
  else prod = sr_corners(C) + (sub - 5) * c2;
  sums = sr_sums(C) + int64_t(sub) * C;
}

// One factor problem from a layer (which = 0: A, 1: G).
static SyrkDesc make_problem(const kfac_layer& L, int which) {
  SyrkDesc d{};
  d.R = L.n * L.h_out * L.w_out;
  if (which == 0) {
    d.mode = 1;
    d.H = L.h; d.W = L.w; d.C = L.c_in; d.Ho = L.h_out; d.Wo = L.w_out;
    d.rhw = 1.0 / static_cast<double>(int64_t(L.h_out) * L.w_out);
    d.rwo = 1.0 / static_cast<double>(L.w_out);
    d.kh = L.kh; d.kw = L.kw; d.sh = L.sh; d.sw = L.sw; d.ph = L.ph; d.pw = L.pw;
    d.d_core = L.c_in * L.kh * L.kw;
    d.bias = L.bias ? 1 : 0;
    if (L.kh == 1 && L.kw == 1 && L.sh == 1 && L.sw == 1 && L.ph == 0 && L.pw == 0 &&
        L.h == L.h_out && L.w == L.w_out) {  // 1x1 stride-1: the activation is X itself
      d.mode = 0;
      d.ld = L.c_in;
      d.H = d.W = 1;
    }
  } else {
    d.mode = 0;
    d.d_core = L.c_out;
    d.ld = L.c_out;
    d.H = d.W = 1;
    d.bias = 0;
  }
  d.d = d.d_core + d.bias;
  d.nb = (d.d_core + ST - 1) / ST;
  d.nt = d.nb * (d.nb + 1) / 2;
  d.nb2 = (d.d_core + BT - 1) / BT;
  d.nt2 = d.nb2 * (d.nb2 + 1) / 2;
  d.inv_r = 1.0f / static_cast<float>(d.R);
  d.r_f = static_cast<float>(d.R);
  return d;
}

// Relative cost of one patch row of one tile: 16-byte gathers (fp16 input whose
// channel count and d_core are multiples of 8) against element gathers, as measured
// on gfx950 (about 4x per row).
static double row_cost(const SyrkDesc& d, kfac_dtype dt) {
  const int width = d.mode == 1 ? d.C : d.ld;
  return (dt == KFAC_F16 && width % 8 == 0 && (d.d_core % 8 == 0 || d.padded)) ? 1.0 : 4.0;
}

// Cost of one patch row of a 256x256 tile in units of one patch row of a 128x128
// tile with 16-byte gathers: four times the products for twice the gathers.
constexpr double kBigRowCost = 2.0;
// Smallest factor order (d_core) taken on 256x256 tiles.
constexpr int kBigMinOrder = 1024;
// Set-up, first loads and result stores of a 256x256 item, in patch rows (measured on
// gfx950: about 6 us per item against about 2 us per 64 rows).
constexpr double kBigItemRows = 192.0;

// Whether a problem's shape suits 256x256 tiles: fp16 inputs read with 16-byte
// gathers; a shift product of 256 or more channels (fewer would leave most of a
// 256-row tile idle) or a factor of order kBigMinOrder or more; an output under 2^31
// bytes (32-bit store offsets). A factor of order d does about d/2 flop per input
// byte, against about 540 for the chip's fp16 MFMA rate over its HBM rate: below
// order ~1000 a factor is bound by its loads, which the 128x128 kernel (two blocks
// per compute unit, twice the bytes in flight) streams faster (measured on the
// order-256 factors over 100,352 rows: 82-96 us in 256x256 tiles, less in 128x128).
// The launch also needs the input pointer's 16-byte alignment (SyrkDesc::vec); the
// split plan depends on the shape only, so that the workspace query bounds every call.
static bool big_shape(const SyrkDesc& d, kfac_dtype dt) {
  const int64_t out_floats = d.kind == 1 ? int64_t(d.c_row) * d.c_col : int64_t(d.d) * (d.d + 1) / 2;
  return dt == KFAC_F16 && row_cost(d, dt) == 1.0 && (d.kind == 1 ? d.c_row >= BT : d.d_core >= kBigMinOrder) &&
         out_floats * 4 < (int64_t(1) << 31);
}


// Cost of one patch row of one work item (a tile over a range of rows).
static double item_row_cost(const SyrkDesc& d, kfac_dtype dt) {
  return big_shape(d, dt) ? kBigRowCost : row_cost(d, dt);
}
static int64_t tiles_per_split(const SyrkDesc& d, kfac_dtype dt) { return big_shape(d, dt) ? d.nt2 : d.nt; }

// Row splits: spread the work so that the launches hold about 2048 work items (a
// tile over a range of rows) of about equal cost, and at least 1024 rows each; the
// split count of a factor never exceeds 256. Equal item costs keep the per-XCD
// ranges of items (contiguous, equal in count) equal in time. (Measured on ResNet-50
// at batch 32 with 128x128 tiles only: 2048 items 1.80-1.82 ms plus 0.026 ms of
// split reduction, 4096 items 1.83-1.87 + 0.036, 8192 items 1.81-1.82 + 0.116.)
static void plan_splits(std::vector<SyrkDesc>& ds, kfac_dtype dt) {
  double work = 0;
  for (auto& d : ds) work += double(tiles_per_split(d, dt)) * d.R * item_row_cost(d, dt);
  const double per_cost = work / 2048.0;
  for (auto& d : ds) {
    double per = per_cost / item_row_cost(d, dt);
    if (per < 1024) per = 1024;
    int64_t splits = static_cast<int64_t>((d.R + per - 1) / per);
    if (splits < 1) splits = 1;
    if (splits > 256) splits = 256;
    int64_t rows = (d.R + splits - 1) / splits;
    rows = (rows + 2 * KC - 1) / (2 * KC) * (2 * KC);  // whole chunks of a diagonal tile
    d.rows_per_split = static_cast<int32_t>(rows);
    d.splits = static_cast<int32_t>((d.R + rows - 1) / rows);
  }
}

// Work-item offsets: the problems of the big-tile launch (desc[0, nbig)) and those of
// the 128x128 launch (desc[nbig, ..)) are each numbered from 0.
static void finish_plan(SyrkPlan& pl) {
  pl.begin.clear(); pl.rbegin.clear(); pl.rprob.clear();
  pl.items = pl.items_big = pl.ritems = 0;
  pl.partial_floats = 0;
  for (size_t p = 0; p < pl.desc.size(); ++p) {
    SyrkDesc& d = pl.desc[p];
    if (d.big) {
      pl.begin.push_back(static_cast<int32_t>(pl.items_big));
      pl.items_big += int64_t(d.splits) * d.nt2;
    } else {
      pl.begin.push_back(static_cast<int32_t>(pl.items));
      pl.items += int64_t(d.splits) * d.nt;
    }
    if (d.splits > 1) {
      pl.rbegin.push_back(static_cast<int32_t>(pl.ritems));
      pl.rprob.push_back(static_cast<int32_t>(p));
      pl.ritems += int64_t(d.nt) * RED_PARTS;
      pl.partial_floats += size_t(d.splits) * d.nt * ST * ST + size_t(d.splits) * d.nb * ST;
    }
  }
}

static size_t syrk_ws_bytes(const SyrkPlan& pl) {
  const size_t np = pl.desc.size(), nr = pl.rprob.size(), nj = pl.jobs.size();
  return align256(sizeof(SyrkDesc) * np) + align256(sizeof(int32_t) * np) + align256(sizeof(int32_t) * 2) +
         2 * align256(sizeof(int32_t) * (nr ? nr : 1)) + align256(sizeof(float) * pl.partial_floats) +
         pl.im2row_bytes + align256(sizeof(ShiftAsm) * (nj ? nj : 1)) + align256(sizeof(int32_t) * (nj ? nj : 1)) +
         sizeof(float) * pl.shift_floats;
}

}  // namespace kfac

using namespace kfac;

static kfac_status layers_validate(const kfac_layer* L, int32_t count, kfac_dtype dt) {
  if (count < 0) return fail(KFAC_ERR_INVALID, "count must be >= 0");
  if (count > 0 && !L) return fail(KFAC_ERR_INVALID, "layers is NULL");
  if (dt != KFAC_F16 && dt != KFAC_F32) return fail(KFAC_ERR_UNSUPPORTED, "dtype %d not supported", dt);
  for (int l = 0; l < count; ++l) {
    const kfac_layer& x = L[l];
    if (x.n < 1 || x.h < 1 || x.w < 1 || x.c_in < 1 || x.c_out < 1 || x.kh < 1 || x.kw < 1 ||
        x.sh < 1 || x.sw < 1 || x.ph < 0 || x.pw < 0 || x.h_out < 1 || x.w_out < 1)
      return fail(KFAC_ERR_INVALID, "layer %d: sizes must be positive", l);
    if (x.h_out != (x.h + 2 * x.ph - x.kh) / x.sh + 1 || x.w_out != (x.w + 2 * x.pw - x.kw) / x.sw + 1 ||
        x.h + 2 * x.ph < x.kh || x.w + 2 * x.pw < x.kw)
      return fail(KFAC_ERR_INVALID, "layer %d: h_out/w_out do not match the convolution", l);
    if (x.bias != 0 && x.bias != 1) return fail(KFAC_ERR_INVALID, "layer %d: bias must be 0 or 1", l);
    const int64_t rows = int64_t(x.n) * x.h_out * x.w_out;
    const int64_t da = int64_t(x.c_in) * x.kh * x.kw + x.bias;
    if (rows >= (int64_t(1) << 31) || da > 65536 || x.c_out > 65536)
      return fail(KFAC_ERR_INVALID, "layer %d: too large", l);
    // every input tensor is addressed with 32-bit offsets (raw buffer loads)
    const int64_t es = dt == KFAC_F16 ? 2 : 4;
    if (int64_t(x.n) * x.h * x.w * x.c_in * es >= (int64_t(1) << 31) || rows * x.c_out * es >= (int64_t(1) << 31))
      return fail(KFAC_ERR_UNSUPPORTED, "layer %d: an input tensor of 2^31 bytes or more", l);
  }
  return KFAC_OK;
}

// Problems in call order: A of layer l (or its nine shift products), then G of layer
// l. Row splits are planned over all factors (so the workspace query bounds every
// call); factors whose input pointer is NULL are then dropped.
static kfac_status build_plan(const kfac_layer* L, int32_t count, kfac_dtype dt, const void* const* act,
                              const void* const* gout, float* const* A, float* const* G, float* const* Af,
                              float* const* Gf, SyrkPlan& pl) {
  const int esize = dt == KFAC_F16 ? 2 : 4;
  std::vector<SyrkDesc> all;
  std::vector<Im2Row> geo;            // conv geometry of the problems converted to rows (by index in all)
  std::vector<int32_t> owner, which_of, sub_of;  // layer, factor (0 A, 1 G), shift sub-problem (-1: none)
  for (int l = 0; l < count; ++l)
    for (int which = 0; which < 2; ++which) {
      if (which == 0 && shift_eligible(L[l], dt)) {
        for (int sub = 0; sub < 9; ++sub) {
          all.push_back(make_shift(L[l], sub));
          geo.push_back(Im2Row{});
          owner.push_back(l); which_of.push_back(0); sub_of.push_back(sub);
        }
        continue;
      }
      SyrkDesc d = make_problem(L[l], which);
      Im2Row g{};
      if (dt == KFAC_F16 && d.mode == 1 && d.C % 8 != 0) {
        g = Im2Row{nullptr, nullptr, d.R, (d.d_core + 7) / 8 * 8, d.d_core, d.H, d.W, d.C, d.Ho, d.Wo,
                   d.kh, d.kw, d.sh, d.sw, d.ph, d.pw, d.rhw, d.rwo};
        d.mode = 0;
        d.ld = g.ld;
        d.H = d.W = 1;
        d.padded = 1;
      }
      all.push_back(d);
      geo.push_back(g);
      owner.push_back(l); which_of.push_back(which); sub_of.push_back(-1);
    }
  plan_splits(all, dt);
  std::vector<int32_t> job_of_layer(count, -1);
  for (size_t q = 0; q < all.size(); ++q) {
    const int l = owner[q], which = which_of[q], sub = sub_of[q];
    SyrkDesc d = all[q];
    if (act) {
      const void* src = which == 0 ? act[l] : gout[l];
      if (!src) continue;
      float* out = which == 0 ? A[l] : G[l];
      float* const* fl = which == 0 ? Af : Gf;
      float* full = fl ? fl[l] : nullptr;
      if (!out) return fail(KFAC_ERR_INVALID, "layer %d: output for factor %d is NULL", l, which);
      if (reinterpret_cast<uintptr_t>(src) % esize || reinterpret_cast<uintptr_t>(out) % 4 ||
          reinterpret_cast<uintptr_t>(full) % 4)
        return fail(KFAC_ERR_INVALID, "layer %d: misaligned pointer", l);
      d.src = src;
      d.out = out;  // shift products: replaced by the region at launch
      d.full = sub >= 0 ? nullptr : full;  // a shift product's full copy is its assembly's
      const int width = d.mode == 1 ? d.C : d.ld;
      const int64_t bytes = d.mode == 1 ? int64_t(L[l].n) * d.H * d.W * d.C * esize
                                        : int64_t(d.R) * d.ld * esize;
      d.vec = (dt == KFAC_F16 && width % 8 == 0 &&
               (d.padded || (d.d_core % 8 == 0 && reinterpret_cast<uintptr_t>(src) % 16 == 0))) ? 1 : 0;
      d.nbytes = d.vec ? static_cast<int32_t>(bytes) : 0;
    }
    if (sub >= 0 && sub_of[q] == 0) {  // the layer's assembly job (first sub-problem)
      job_of_layer[l] = static_cast<int32_t>(pl.jobs.size());
      ShiftAsm j{};
      j.out = act ? A[l] : nullptr;
      j.full = act && Af ? Af[l] : nullptr;
      j.C = L[l].c_in;
      j.bias = L[l].bias ? 1 : 0;
      j.d = 9 * j.C + j.bias;
      const int64_t rows = int64_t(L[l].n) * L[l].h_out * L[l].w_out;
      j.inv_r = 1.0f / static_cast<float>(rows);
      j.r_f = static_cast<float>(rows);
      pl.jobs.push_back(j);
      pl.jbegin.push_back(static_cast<int32_t>(pl.jtiles));
      pl.jtiles += j.C;  // one assembly block per channel
      pl.shift_floats += align256(sizeof(float) * sr_floats(j.C)) / sizeof(float);
    }
    if (d.padded) {
      const int64_t pb = int64_t(d.R) * d.ld * 2;
      if (pb < (int64_t(1) << 31)) {  // rows in the workspace, read with 16-byte loads
        Im2Row g = geo[q];
        g.src = static_cast<const _Float16*>(d.src);
        pl.im2row.push_back(g);
        d.padded = static_cast<int32_t>(pl.im2row.size());
        pl.im2row_bytes += align256(static_cast<size_t>(pb));
      } else {  // too large for one buffer range: element gathers from the NHWC tensor
        SyrkDesc c = make_problem(L[l], which);
        c.splits = d.splits;
        c.rows_per_split = d.rows_per_split;
        c.src = d.src;
        c.out = d.out;
        c.full = d.full;
        d = c;
      }
    }
    pl.desc.push_back(d);
    pl.shift_job.push_back(sub >= 0 ? job_of_layer[l] : -1);
    pl.shift_sub.push_back(sub);
  }
  // The big-tile problems first, then the rest; within each launch, problems in
  // decreasing cost per item (stable): each problem's items stay together (its tiles
  // over one row range are neighbours, sharing those rows in L2), and each XCD segment
  // starts with its longest items.
  for (SyrkDesc& d : pl.desc) d.big = (big_shape(d, dt) && d.vec) ? 1 : 0;
  // cost of an item of `rows` rows (per-row cost as in item_row_cost, now that vec is
  // known); a 256x256 item also costs about kBigItemRows rows' worth of set-up, first
  // loads and result stores, so that XCD segments of short items are not overfilled
  auto cost_of = [&](const SyrkDesc& d, int rows) {
    return d.big ? (double(rows) + kBigItemRows) * kBigRowCost
                 : double(rows) * ((dt == KFAC_F16 && d.vec) ? 1.0 : 4.0);
  };
  auto item_cost = [&](const SyrkDesc& d) { return cost_of(d, d.rows_per_split); };
  std::vector<int> order(pl.desc.size());
  for (size_t q = 0; q < order.size(); ++q) order[q] = static_cast<int>(q);
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
    if (pl.desc[a].big != pl.desc[b].big) return pl.desc[a].big > pl.desc[b].big;
    return item_cost(pl.desc[a]) > item_cost(pl.desc[b]);
  });
  {
    std::vector<SyrkDesc> ds(order.size());
    std::vector<int32_t> sj(order.size()), ss(order.size());
    for (size_t q = 0; q < order.size(); ++q) {
      ds[q] = pl.desc[order[q]];
      sj[q] = pl.shift_job[order[q]];
      ss[q] = pl.shift_sub[order[q]];
    }
    pl.desc.swap(ds);
    pl.shift_job.swap(sj);
    pl.shift_sub.swap(ss);
  }
  pl.nbig = 0;
  while (pl.nbig < static_cast<int>(pl.desc.size()) && pl.desc[pl.nbig].big) ++pl.nbig;
  pl.im2row_prob.assign(pl.im2row.size(), 0);
  for (size_t p = 0; p < pl.desc.size(); ++p)
    if (pl.desc[p].padded) pl.im2row_prob[pl.desc[p].padded - 1] = static_cast<int32_t>(p);
  finish_plan(pl);
  if (pl.items >= (int64_t(1) << 31) - 8 || pl.items_big >= (int64_t(1) << 31) - 8 ||
      pl.ritems >= (int64_t(1) << 31) || pl.jtiles >= (int64_t(1) << 31))
    return fail(KFAC_ERR_INVALID, "too many tiles");
  // XCD segments of about equal cost (rows x per-row cost over the items in order),
  // for each launch over its own problems
  auto make_segs = [&](int p0, int p1, XcdSegs& segs, int64_t& seg_max) {
    double total = 0;
    for (int p = p0; p < p1; ++p) {
      const SyrkDesc& d = pl.desc[p];
      for (int sp = 0; sp < d.splits; ++sp)
        total += cost_of(d, std::min(d.rows_per_split, d.R - sp * d.rows_per_split)) * (d.big ? d.nt2 : d.nt);
    }
    int64_t item = 0;
    double acc = 0;
    int x = 0;
    segs.begin[0] = 0;
    for (int p = p0; p < p1; ++p) {
      const SyrkDesc& d = pl.desc[p];
      const int64_t nt = d.big ? d.nt2 : d.nt;
      for (int sp = 0; sp < d.splits; ++sp) {
        const double c = cost_of(d, std::min(d.rows_per_split, d.R - sp * d.rows_per_split));
        int64_t t = 0;
        while (t < nt) {  // a segment starts at the first item reached with acc >= its share
          int64_t k = nt - t;
          if (x < 7) {
            const double thr = total * (x + 1) / 8;
            if (acc >= thr) {
              segs.begin[++x] = static_cast<int32_t>(item);
              continue;
            }
            k = std::min<int64_t>(k, std::max<int64_t>(1, static_cast<int64_t>(std::ceil((thr - acc) / c))));
          }
          acc += double(k) * c;
          item += k;
          t += k;
        }
      }
    }
    while (x < 7) segs.begin[++x] = static_cast<int32_t>(item);
    seg_max = 0;
    for (int k = 0; k < 8; ++k) {
      const int64_t e = k < 7 ? segs.begin[k + 1] : item;
      segs.len[k] = static_cast<int32_t>(e - segs.begin[k]);
      seg_max = std::max<int64_t>(seg_max, segs.len[k]);
    }
  };
  make_segs(pl.nbig, static_cast<int>(pl.desc.size()), pl.segs, pl.seg_max);
  return KFAC_OK;
}

extern "C" kfac_status kfac_factors_workspace(const kfac_layer* layers, int32_t count, kfac_dtype in_dtype,
                                              size_t* bytes) {
  if (!bytes) return fail(KFAC_ERR_INVALID, "bytes is NULL");
  kfac_status st = layers_validate(layers, count, in_dtype);
  if (st) return st;
  if (count == 0) { *bytes = 0; return KFAC_OK; }
  SyrkPlan pl;
  st = build_plan(layers, count, in_dtype, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, pl);
  if (st) return st;
  *bytes = syrk_ws_bytes(pl);
  return KFAC_OK;
}

extern "C" kfac_status kfac_factors_full(const kfac_layer* layers, int32_t count, kfac_dtype in_dtype,
                                         const void* const* act, const void* const* gout,
                                         float* const* A_packed, float* const* G_packed, float* const* A_full,
                                         float* const* G_full, float ema_decay, void* workspace,
                                         size_t ws_bytes, void* stream) {
  kfac_status st = layers_validate(layers, count, in_dtype);
  if (st) return st;
  if (!(ema_decay >= 0.f && ema_decay <= 1.f)) return fail(KFAC_ERR_INVALID, "ema_decay must be in [0, 1]");
  if (count == 0) return KFAC_OK;
  if (!act || !gout || !A_packed || !G_packed) return fail(KFAC_ERR_INVALID, "NULL pointer array");
  SyrkPlan pl;
  st = build_plan(layers, count, in_dtype, act, gout, A_packed, G_packed, A_full, G_full, pl);
  if (st) return st;
  if (pl.desc.empty()) return KFAC_OK;
  st = check_device();
  if (st) return st;
  // The workspace query plans every factor; a call that skips factors needs less.
  const size_t need = syrk_ws_bytes(pl);
  st = check_workspace(workspace, ws_bytes, need);
  if (st) return st;
  const int np = static_cast<int>(pl.desc.size());
  const int nr = static_cast<int>(pl.rprob.size());
  Carver cv(workspace);
  SyrkDesc* d_desc = cv.take<SyrkDesc>(np);
  int32_t* d_begin = cv.take<int32_t>(np);
  int32_t* d_next = cv.take<int32_t>(2);  // item counters of the 256x256 and 128x128 launches
  int32_t* d_rbegin = cv.take<int32_t>(nr ? nr : 1);
  int32_t* d_rprob = cv.take<int32_t>(nr ? nr : 1);
  const int nj = static_cast<int>(pl.jobs.size());
  ShiftAsm* d_jobs = cv.take<ShiftAsm>(nj ? nj : 1);  // tables first: they go up as one image
  int32_t* d_jbegin = cv.take<int32_t>(nj ? nj : 1);
  float* part = cv.take<float>(pl.partial_floats);
  for (size_t q = 0; q < pl.im2row.size(); ++q) {
    Im2Row& g = pl.im2row[q];
    g.dst = cv.take<_Float16>(size_t(g.R) * g.ld);
    pl.desc[pl.im2row_prob[q]].src = g.dst;
  }
  float* regions = cv.take<float>(pl.shift_floats);
  {
    size_t roff = 0;
    for (ShiftAsm& j : pl.jobs) {
      j.base = regions + roff;
      roff += align256(sizeof(float) * sr_floats(j.C)) / sizeof(float);
    }
  }
  size_t off = 0;
  for (size_t q = 0; q < pl.desc.size(); ++q) {
    SyrkDesc& d = pl.desc[q];
    if (d.splits > 1) {
      d.partial = part + off;
      off += size_t(d.splits) * d.nt * ST * ST;
      d.pcol = part + off;
      off += size_t(d.splits) * d.nb * ST;
    }
    if (pl.shift_job[q] >= 0) {  // a shift product writes into its layer's region
      const ShiftAsm& j = pl.jobs[pl.shift_job[q]];
      int64_t prod = 0, sums = 0;
      shift_out(j.C, pl.shift_sub[q], prod, sums);
      d.out = const_cast<float*>(j.base) + prod;
      d.csum = const_cast<float*>(j.base) + sums;
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  TableUpload tu;
  const int32_t zero[2] = {0, 0};
  tu.add(d_desc, pl.desc.data(), sizeof(SyrkDesc) * np);
  tu.add(d_begin, pl.begin.data(), sizeof(int32_t) * np);
  tu.add(d_next, zero, sizeof(zero));
  if (nr) {
    tu.add(d_rbegin, pl.rbegin.data(), sizeof(int32_t) * nr);
    tu.add(d_rprob, pl.rprob.data(), sizeof(int32_t) * nr);
  }
  if (nj) {
    tu.add(d_jobs, pl.jobs.data(), sizeof(ShiftAsm) * nj);
    tu.add(d_jbegin, pl.jbegin.data(), sizeof(int32_t) * nj);
  }
  if ((st = tu.flush(s))) return st;
  for (const Im2Row& g : pl.im2row) {
    const int64_t total = int64_t(g.R) * (g.ld / 8);
    KFAC_LAUNCH(K_SYRK, im2row_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, s, g, total);
    KFAC_CHECK_LAUNCH("im2row_kernel");
  }
  const int nbig = pl.nbig, nsmall = np - nbig;
  if (pl.items_big > 0) {  // problems desc[0, nbig) on 256x256 tiles, one block per item
    KFAC_LAUNCH(K_SYRK, syrk_big_kernel, dim3(static_cast<unsigned>(pl.items_big)), dim3(512), 0, s, d_desc,
                d_begin, nbig, d_next, static_cast<int>(pl.items_big), ema_decay);
    KFAC_CHECK_LAUNCH("syrk_big_kernel");
  }
  if (nsmall > 0 && pl.items > 0) {  // the rest on 128x128 tiles
    const unsigned grid = static_cast<unsigned>(8 * pl.seg_max);
    if (in_dtype == KFAC_F16) {  // one block per item, from the counter
      KFAC_LAUNCH(K_SYRK, syrk_f16_kernel, dim3(static_cast<unsigned>(pl.items)), dim3(256), 0, s, d_desc + nbig,
                  d_begin + nbig, nsmall, d_next + 1, static_cast<int>(pl.items), ema_decay);
    } else {
      KFAC_LAUNCH(K_SYRK, syrk_f32_kernel, dim3(grid), dim3(256), 0, s, d_desc + nbig, d_begin + nbig, nsmall,
                  pl.segs, ema_decay);
    }
    KFAC_CHECK_LAUNCH("syrk kernel");
  }
  if (nr) {
    KFAC_LAUNCH(K_SYRK_REDUCE, syrk_reduce_kernel, dim3(static_cast<unsigned>(pl.ritems)), dim3(256), 0, s,
                d_desc, d_rbegin, d_rprob, nr, ema_decay);
    KFAC_CHECK_LAUNCH("syrk_reduce_kernel");
  }
  if (nj) {
    KFAC_LAUNCH(K_SHIFT_ASM, shift_assemble_kernel, dim3(static_cast<unsigned>(pl.jtiles)), dim3(256), 0, s,
                d_jobs, d_jbegin, nj, ema_decay);
    KFAC_CHECK_LAUNCH("shift_assemble_kernel");
  }
  return KFAC_OK;
}

extern "C" kfac_status kfac_factors(const kfac_layer* layers, int32_t count, kfac_dtype in_dtype,
                                    const void* const* act, const void* const* gout,
                                    float* const* A_packed, float* const* G_packed, float ema_decay,
                                    void* workspace, size_t ws_bytes, void* stream) {
  return kfac_factors_full(layers, count, in_dtype, act, gout, A_packed, G_packed, nullptr, nullptr, ema_decay,
                           workspace, ws_bytes, stream);
}
