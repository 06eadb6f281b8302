// The GPTQ column sweep on one 128-column block, the lazy update of the
// columns to its right, and the small helper kernels around them.
//
// Method: "GPTQ > The GPTQ Algorithm" (one fixed left-to-right column order
// for all rows; lazy batch updates in blocks of 128) and "GPTQ, Line by
// Line", blocks-of-128 question (rank-1 updates inside the block, then
// Err1 * Hinv[block, rest] on the rest).  Quantizer and error scaling:
// gptq_quantize_layer listing of "GPTQ-style round-to-nearest with Hessian
// weighting" (min/max grid per row and group, statistics at the group's first
// column, err = (w - w_hat) / Hinv[j,j]).
//
// gfx950 design of the sweep kernel:
//   * Rows are independent (every row shares the same Hinv), so a workgroup
//     owns 16 rows and the whole 128-column block of them; no inter-workgroup
//     synchronisation exists anywhere in the sweep.
//   * 16 lanes per row, 4 rows per wave.  Lane l holds columns l, l+16, ...,
//     l+112 of its row in registers.  The 128 column steps are unrolled so
//     every register index is a compile-time constant.
//   * Step j: every lane evaluates the quantizer on its register j/16 (only
//     lane j%16 holds column j), the owner's scaled error is broadcast inside
//     the 16-lane group, and each lane applies the rank-1 update to the
//     columns it holds.  Hinv's 128x128 diagonal block is in LDS row by row
//     (lanes of a row read 16 consecutive floats, the four rows of a wave
//     the same ones); entries left of the diagonal are zero, which makes the
//     update of finished columns a no-op.
//   * Group min/max is a per-lane reduction followed by a 4-step xor shuffle
//     across the 16 lanes of the row.
//   * Per-column loss partials are reduced inside the workgroup and written
//     per workgroup; a final kernel adds them in a fixed order.
//   * With groups inside blocks, the workgroup first applies to its rows the
//     errors of the earlier blocks of the same superblock (fp32 MFMA, one
//     128x128 Hinv tile at a time through LDS), so no separate launch carries
//     them.
//
// The lazy update W[:, c0:c1] -= Err[:, k0:k1] Hinv[k0:k1, c0:c1] is an fp32
// MFMA GEMM (v_mfma_f32_16x16x4_f32) on (32*MT)x128 output tiles, K streamed
// through double-buffered LDS in chunks of 32.
#include "common.h"

#include <utility>

namespace gptq {

namespace {

constexpr int BC = kBlock;  // 128 columns per block
constexpr int RL = 16;      // lanes per row
constexpr int CPL = BC / RL;  // columns per lane (8)

__device__ inline float shfl_xor16(float v, int m) { return __shfl_xor(v, m, 16); }

__device__ inline void row_minmax(float& mn, float& mx) {
#pragma unroll
  for (int m = 1; m < RL; m <<= 1) {
    mn = fminf(mn, shfl_xor16(mn, m));
    mx = fmaxf(mx, shfl_xor16(mx, m));
  }
}

__device__ inline void grid_params(float mn, float mx, float qm, float& s, float& z) {
  s = fmaxf((mx - mn) / qm, 1e-8f);
  z = fminf(fmaxf(rintf(-mn / s), 0.f), qm);
}

// x / s correctly rounded (IEEE binary32), given rs = RN(1/s): the residual
// x - q0*s is exact under FMA, and one correction step yields RN(x/s)
// (Markstein's division theorem).  For |x| < 2^-100 the correction may be
// off by an ulp, but then x/s + z rounds to the same integer either way.
__device__ inline float div_rn(float x, float s, float rs) {
  const float q0 = x * rs;
  const float r = __builtin_fmaf(-q0, s, x);
  return __builtin_fmaf(r, rs, q0);
}

// Row min/max of the current group across the 16 lanes of a row and the
// resulting grid; lane 0 of the row records it.
__device__ inline void group_stats(float mn, float mx, float qm, float& s, float& z, float& rs,
                                   bool rv, int l, int64_t row, int64_t ngroups, int64_t gi,
                                   float* __restrict__ scales, float* __restrict__ zeros) {
  row_minmax(mn, mx);
  grid_params(mn, mx, qm, s, z);
  rs = 1.0f / s;
  if (rv && l == 0) {
    scales[row * ngroups + gi] = s;
    zeros[row * ngroups + gi] = z;
  }
}

// Value of `v` held by lane `src + 16*rg` of the wave, for each lane's row
// group rg (src is wave-uniform): four readlanes combined with the lane's 0/1
// row-group masks (branch-free; exact because each product is v or 0).
// Value of v held by lane LJ of this lane's row of 16 (DPP row_newbcast):
// each row of 16 lanes is one row of W, so this is the owner's value.
template <int LJ>
__device__ inline float row_bcast(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + LJ, 0xF, 0xF, true));
}

// Column step j = 16*kj + LJ of the sweep for this lane's row (see sweep_kernel).
template <int LJ>
__device__ inline void sweep_step(int kj, int l, float s, float z, float rs, float qm, float rd,
                                  const float* __restrict__ urow, float (&w)[CPL],
                                  float (&u)[CPL], float (&qc)[CPL], float (&ev)[CPL]) {
  // next step's Hinv row segment, off the dependency chain
  float un[CPL];
  if (LJ + 1 < RL) {
#pragma unroll
    for (int k = kj; k < CPL; ++k) un[k] = urow[(LJ + 1) * BC + l + RL * k];
  }
  const float x = w[kj];
  const float t = div_rn(x, s, rs) + z;
  const float q = fminf(fmaxf(rintf(t), 0.f), qm);
  const float err = __builtin_fmaf(-(q - z), s, x);
  const float eb = row_bcast<LJ>(err * rd);
  if (l == LJ) {
    qc[kj] = q;
    ev[kj] = eb;
  }
#pragma unroll
  for (int k = kj; k < CPL; ++k) w[k] = __builtin_fmaf(-eb, u[k], w[k]);
  if (LJ + 1 < RL) {
#pragma unroll
    for (int k = kj; k < CPL; ++k) u[k] = un[k];
  }
  __builtin_amdgcn_sched_barrier(0);  // keep steps apart: bounded register pressure
}

template <int... LJ>
__device__ inline void sweep_steps(int kj, int l, float s, float z, float rs, float qm, float rd,
                                   const float* __restrict__ urow, float (&w)[CPL],
                                   float (&u)[CPL], float (&qc)[CPL], float (&ev)[CPL],
                                   std::integer_sequence<int, LJ...>) {
  (sweep_step<LJ>(kj, l, s, z, rs, qm, rd, urow, w, u, qc, ev), ...);
}

// G: group size when it divides the block (16, 32, 64, 128); G == 0 means the
// group spans several blocks (groupsize a multiple of 128).
//
// Column j = 16*kj + lj lives in register kj of lane lj.  Both loops are
// unrolled, so every register index and the DPP source lane are compile-time
// constants.  Steps past the end of a short last block run on zero weights
// and zero Hinv entries and change nothing.
// Hinv[r0 + j][i1 + c] for j < nrows, c < nbc (zero elsewhere) as the 16
// float4 this thread moves into a 128x128 LDS tile (row j at U + 128 j).
__device__ inline void hinv_tile_load(float4 (&v)[16], const float* __restrict__ Hinv, int64_t cols,
                                      int64_t r0, int i1, int nbc, int nrows, int tid) {
  const bool vec = (cols % 4 == 0) && (reinterpret_cast<uintptr_t>(Hinv) % 16 == 0);
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int e = tid + 256 * q;  // float4 index: row e/32, columns 4*(e%32)..
    const int j = e >> 5, c = (e & 31) * 4;
    const float* p = Hinv + (r0 + j) * cols + i1 + c;
    float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
    if (j < nrows) {
      if (vec && c + 4 <= nbc) {
        u = *reinterpret_cast<const float4*>(p);
      } else {
        if (c + 0 < nbc) u.x = p[0];
        if (c + 1 < nbc) u.y = p[1];
        if (c + 2 < nbc) u.z = p[2];
        if (c + 3 < nbc) u.w = p[3];
      }
    }
    v[q] = u;
  }
}

// The loaded tile into LDS; with TRI (the block's own diagonal tile) the part
// left of the diagonal is zeroed.
template <bool TRI>
__device__ inline void hinv_tile_store(float* __restrict__ U, const float4 (&v)[16], int tid) {
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int e = tid + 256 * q;
    const int j = e >> 5, c = (e & 31) * 4;
    float4 u = v[q];
    if (TRI) {
      if (c + 0 < j) u.x = 0.f;
      if (c + 1 < j) u.y = 0.f;
      if (c + 2 < j) u.z = 0.f;
      if (c + 3 < j) u.w = 0.f;
    }
    *reinterpret_cast<float4*>(U + j * BC + c) = u;
  }
}

// Err[row0 + r][c0 + c] for the workgroup's 16 rows x 128 columns: 2 float4
// per thread (rows past `rows` read as zero).
__device__ inline void err_slice_load(float4 (&v)[2], const float* __restrict__ Err, int64_t ldk,
                                      int64_t rows, int64_t row0, int c0, int tid) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = tid + 256 * q;
    const int r = e >> 5, c = (e & 31) * 4;
    v[q] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row0 + r < rows) v[q] = *reinterpret_cast<const float4*>(Err + (row0 + r) * ldk + c0 + c);
  }
}

// p0 < i1 (groups inside blocks only): the blocks [p0, i1) of this
// superblock were swept by earlier launches and their errors have not yet
// been applied to this block; the workgroup applies them to its own rows
// first, W[rows, block] -= Err[rows, p0:i1] Hinv[p0:i1, block], one 128x128
// Hinv tile at a time through LDS and fp32 MFMA.  This replaces a separate
// small lazy-update launch per block (the result is the same sum).
template <int G>
__global__ __launch_bounds__(256) void sweep_kernel(float* __restrict__ Wk, int64_t ldk,
                                                    int64_t rows, int64_t cols, int i1, int p0,
                                                    const float* __restrict__ Hinv, int bits,
                                                    int groupsize, uint8_t* __restrict__ codes,
                                                    float* __restrict__ scales,
                                                    float* __restrict__ zeros,
                                                    float* __restrict__ Err,
                                                    float* __restrict__ lpart) {
  __shared__ __attribute__((aligned(16))) float Ub[BC * BC];  // Hinv block, row j at Ub + 128 j
  __shared__ float rdiag[BC];
  __shared__ float lsum[4][BC];
  __shared__ __attribute__((aligned(16))) float Es[kSweepRows * (BC + 4)];  // Err slice / update tile

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l = lane & 15;
  const int rg = lane >> 4;
  const int64_t row = (int64_t)blockIdx.x * kSweepRows + wave * 4 + rg;
  const bool rv = row < rows;
  const int nbc = (int)((cols - i1) < BC ? (cols - i1) : BC);
  const int64_t ngroups = ceil_div(cols, groupsize);

  float w[CPL];
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    const int c = l + RL * k;
    w[k] = (rv && c < nbc) ? Wk[row * ldk + i1 + c] : 0.f;
  }

  float4 hv[16];  // next Hinv tile on its way to LDS
  if (G != 0 && p0 < i1) {
    // pending errors of this superblock: dacc = Err[rows, p0:i1] Hinv[p0:i1, block],
    // wave w forming columns 32w..32w+31 of the 16 rows; the next tile (and
    // finally the block's own diagonal tile) is loaded during each tile's MFMAs
    const int64_t row0 = (int64_t)blockIdx.x * kSweepRows;
    constexpr int EP = BC + 4;
    f32x4 dacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    float4 ev4[2];
    hinv_tile_load(hv, Hinv, cols, p0, i1, nbc, BC, tid);
    err_slice_load(ev4, Err, ldk, rows, row0, p0, tid);
    for (int c0 = p0; c0 < i1; c0 += BC) {
      hinv_tile_store<false>(Ub, hv, tid);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int e = tid + 256 * q;
        *reinterpret_cast<float4*>(Es + (e >> 5) * EP + (e & 31) * 4) = ev4[q];
      }
      __syncthreads();
      if (c0 + BC < i1) {
        hinv_tile_load(hv, Hinv, cols, c0 + BC, i1, nbc, BC, tid);
        err_slice_load(ev4, Err, ldk, rows, row0, c0 + BC, tid);
      } else {
        hinv_tile_load(hv, Hinv, cols, i1, i1, nbc, nbc, tid);  // the diagonal tile
      }
#pragma unroll 8
      for (int s4 = 0; s4 < BC / 4; ++s4) {
        const int kr = 4 * s4 + (lane >> 4);
        const float a = Es[(lane & 15) * EP + kr];
#pragma unroll
        for (int b = 0; b < 2; ++b)
          dacc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, Ub[kr * BC + 32 * wave + 16 * b + (lane & 15)],
                                                        dacc[b], 0, 0, 0);
      }
      __syncthreads();  // Ub and Es are refilled next
    }
    // element i of dacc[b] at lane (n, q) is the update of row 4q + i, column 32w + 16b + n
    // (the fp32 16x16x4 result layout)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        Es[(4 * (lane >> 4) + i) * EP + 32 * wave + 16 * b + (lane & 15)] = dacc[b][i];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < CPL; ++k) w[k] -= Es[(wave * 4 + rg) * EP + l + RL * k];
  } else {
    hinv_tile_load(hv, Hinv, cols, i1, i1, nbc, nbc, tid);
  }
  // Hinv[i1:i1+128, i1:i1+128] with the part left of the diagonal (and past
  // the last column) zeroed
  hinv_tile_store<true>(Ub, hv, tid);
  for (int j = tid; j < BC; j += 256)
    rdiag[j] = (j < nbc) ? 1.f / Hinv[(int64_t)(i1 + j) * cols + i1 + j] : 0.f;

  __syncthreads();

  const float qm = (float)((1 << bits) - 1);
  float s = 1.f, z = 0.f, rs = 1.f;
  if (G == 0) {
    // group of groupsize columns spanning blocks
    const int64_t gi = i1 / groupsize;
    if (i1 % groupsize == 0) {
      float mn = INFINITY, mx = -INFINITY;
#pragma unroll
      for (int k = 0; k < CPL; ++k)
        if (l + RL * k < nbc) {
          mn = fminf(mn, w[k]);
          mx = fmaxf(mx, w[k]);
        }
      const int64_t gend = (i1 + groupsize < cols) ? i1 + groupsize : cols;
      if (rv)
        for (int64_t c = i1 + BC + l; c < gend; c += RL) {
          const float v = Wk[row * ldk + c];
          mn = fminf(mn, v);
          mx = fmaxf(mx, v);
        }
      group_stats(mn, mx, qm, s, z, rs, rv, l, row, ngroups, gi, scales, zeros);
    } else if (rv) {
      s = scales[row * ngroups + gi];
      z = zeros[row * ngroups + gi];
      rs = 1.0f / s;
    }
  }

  float qc[CPL], ev[CPL];
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    qc[k] = 0.f;
    ev[k] = 0.f;
  }

#pragma unroll
  for (int kj = 0; kj < CPL; ++kj) {
    if (RL * kj >= nbc) break;
    if (G != 0 && (RL * kj) % (G > 0 ? G : 1) == 0) {
      // a group starts at column 16*kj: statistics over its current values
      float mn = INFINITY, mx = -INFINITY;
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        const int c = l + RL * k;
        if (k >= kj && k < kj + (G > 0 ? G : RL) / RL && c < nbc) {
          mn = fminf(mn, w[k]);
          mx = fmaxf(mx, w[k]);
        }
      }
      group_stats(mn, mx, qm, s, z, rs, rv, l, row, ngroups, (i1 + RL * kj) / groupsize, scales,
                  zeros);
    }
    // this lane's column 16*kj + l: its 1/Hinv[j][j] (only the owner's is used)
    const float rd = rdiag[RL * kj + l];
    const float* urow = Ub + (RL * kj) * BC;
    float u[CPL];
#pragma unroll
    for (int k = kj; k < CPL; ++k) u[k] = urow[l + RL * k];
    sweep_steps(kj, l, s, z, rs, qm, rd, urow, w, u, qc, ev, std::make_integer_sequence<int, RL>{});
  }

  // outputs
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    const int c = l + RL * k;
    if (rv && c < nbc) {
      codes[row * cols + i1 + c] = (uint8_t)qc[k];
      Err[row * ldk + i1 + c] = ev[k];
    }
  }
  // loss partials: sum of e^2 over this workgroup's rows, per column
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    float v = rv ? ev[k] * ev[k] : 0.f;
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    if (rg == 0) lsum[wave][l + RL * k] = v;
  }
  __syncthreads();
  if (tid < BC) {
    const float tot = (lsum[0][tid] + lsum[1][tid]) + (lsum[2][tid] + lsum[3][tid]);
    if (tid < nbc) lpart[(int64_t)blockIdx.x * ldk + i1 + tid] = 0.5f * tot;
  }
}

// ---------------------------------------------------------------- lazy GEMM
// W[:, c0:c1] -= Err[:, k0:k1] * Hinv[k0:k1, c0:c1]  (fp32, MFMA 16x16x4).
// 128x128 output tiles, 4 waves of 64x64; K streamed in chunks of 32 through
// double-buffered LDS stored k-major (pitch 144 floats: the four k rows an
// operand read touches fall in four different 16-bank groups); the next
// chunk's global loads are issued before the current chunk's MFMAs, and the
// C tile is fetched before the last chunk so its latency overlaps the math.
constexpr int LT = 128;  // output tile edge
constexpr int LK = 32;   // K chunk
constexpr int LP = LT + 16;

// MT: 16x16 MFMA tiles per wave along rows (workgroup tile (32*MT) x 128).
// ALL: K <= 4 chunks, and every chunk's loads and the W tile's loads are
// issued up front (one memory round trip for the whole update instead of
// one per chunk: the small updates inside a superblock are latency-bound).
template <int MT, bool ALL>
__global__ __launch_bounds__(256, 2) void lazy_kernel(float* __restrict__ Wk, int64_t ldk,
                                                   int64_t rows, int64_t cols, int k0, int k1,
                                                   int c0, int c1, const float* __restrict__ Err,
                                                   const float* __restrict__ Hinv) {
  constexpr int TM = 32 * MT;      // rows per workgroup tile
  constexpr int PA = LK + 4;       // A is m-major: a row of 32 k at pitch 36 floats, so
                                   // float4 stores and the operand reads (16 rows x 4 k)
                                   // hit distinct banks
  constexpr int AV = TM * LK / 4 / 256;  // float4 A loads per thread
  __shared__ __attribute__((aligned(16))) float As[2][TM * PA];  // [m][k]
  __shared__ __attribute__((aligned(16))) float Bs[2][LK][LP];   // [k][n]
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t r0 = (int64_t)blockIdx.y * TM;
  const int64_t n0 = (int64_t)c0 + (int64_t)blockIdx.x * LT;
  const int K = k1 - k0;

  f32x4 acc[MT][4];
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Loads read in-bounds addresses unconditionally and keep the raw values;
  // entries past K, past c1 or past the last row are zeroed (or ignored)
  // when the chunk goes to LDS, so no MFMA waits for the next chunk's loads.
  // A = Err[r0.., k0..k1]: the row stride ldk is a multiple of 128 and k0 a
  // multiple of 128, so a whole chunk stays inside each (clamped) row.
  // B = Hinv[k0..k1, n0..]: row and column indices are clamped.
  constexpr int NR = ALL ? 4 : 1;  // register sets of chunk loads in flight
  float4 av[NR][AV], bv[NR][4];
  auto gload = [&](int set, int kc) {
#pragma unroll
    for (int q = 0; q < AV; ++q) {
      const int e = tid + 256 * q;
      const int m = e >> 3, kk = (e & 7) * 4;  // A: 8 float4 per row
      const int64_t gr = (r0 + m < rows) ? r0 + m : rows - 1;
      av[set][q] = *reinterpret_cast<const float4*>(Err + gr * ldk + k0 + kc + kk);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + 256 * q;
      const int kb = e >> 5, nn = (e & 31) * 4;  // B: 32 float4 per k-row
      const int krow = min(k0 + kc + kb, k1 - 1);
      const float* p = Hinv + (int64_t)krow * cols;
      const int64_t gc = n0 + nn;
      const int64_t cl = cols - 1;
      bv[set][q] = make_float4(p[gc < cl ? gc : cl], p[gc + 1 < cl ? gc + 1 : cl],
                               p[gc + 2 < cl ? gc + 2 : cl], p[gc + 3 < cl ? gc + 3 : cl]);
    }
  };
  auto lstore = [&](int set, int buf, int kc) {
#pragma unroll
    for (int q = 0; q < AV; ++q) {
      const int e = tid + 256 * q;
      const int m = e >> 3, kk = (e & 7) * 4;
      const int gk = kc + kk;
      float4 v = av[set][q];
      v.x = (gk + 0 < K) ? v.x : 0.f;
      v.y = (gk + 1 < K) ? v.y : 0.f;
      v.z = (gk + 2 < K) ? v.z : 0.f;
      v.w = (gk + 3 < K) ? v.w : 0.f;
      *reinterpret_cast<float4*>(&As[buf][m * PA + kk]) = v;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + 256 * q;
      const int kb = e >> 5, nn = (e & 31) * 4;
      const bool kv = kc + kb < K;
      const int64_t gc = n0 + nn;
      float4 u = bv[set][q];
      u.x = (kv && gc + 0 < c1) ? u.x : 0.f;
      u.y = (kv && gc + 1 < c1) ? u.y : 0.f;
      u.z = (kv && gc + 2 < c1) ? u.z : 0.f;
      u.w = (kv && gc + 3 < c1) ? u.w : 0.f;
      *reinterpret_cast<float4*>(&Bs[buf][kb][nn]) = u;
    }
  };

  // this lane's output elements: rows rb + 16a + i, columns cb + 16b
  const int64_t rb = r0 + 16 * MT * wm + 4 * (lane >> 4);
  const int64_t cb = n0 + 64 * wn + (lane & 15);
  float* const wbase = Wk + rb * ldk + cb;
  const int ldi = (int)ldk;
  const int nchunks = (K + LK - 1) / LK;
  auto mma_chunk = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < LK; ks += 4) {
      const int kr = ks + (lane >> 4);
      float af[MT], bf[4];
#pragma unroll
      for (int a = 0; a < MT; ++a) af[a] = As[buf][(16 * MT * wm + 16 * a + (lane & 15)) * PA + kr];
#pragma unroll
      for (int b = 0; b < 4; ++b) bf[b] = Bs[buf][kr][64 * wn + 16 * b + (lane & 15)];
#pragma unroll
      for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[a], bf[b], acc[a][b], 0, 0, 0);
    }
  };
  // the W tile this lane updates: rows rb + 16a + i, columns cb + 16b
  float cv[MT][4][4];
  auto wload = [&]() {
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool rv = rb + 16 * a + i < rows;
#pragma unroll
        for (int b = 0; b < 4; ++b) cv[a][i][b] = rv ? wbase[(16 * a + i) * ldi + 16 * b] : 0.f;
      }
  };
  if (ALL) {
    // every chunk (K <= 4 * LK) and the W tile in flight at once
#pragma unroll
    for (int c = 0; c < NR; ++c) gload(c, c * LK);
    wload();
#pragma unroll
    for (int c = 0; c < NR; ++c) {
      if (c < nchunks) {
        lstore(c, c & 1, c * LK);
        __syncthreads();
        mma_chunk(c & 1);
      }
    }
  } else {
    gload(0, 0);
    lstore(0, 0, 0);
    __syncthreads();
    int buf = 0;
    for (int ch = 0; ch < nchunks; ++ch) {
      const bool more = ch + 1 < nchunks;
      if (more) gload(0, (ch + 1) * LK);
      mma_chunk(buf);
      if (more) lstore(0, buf ^ 1, (ch + 1) * LK);
      __syncthreads();
      buf ^= 1;
    }
    wload();
  }
  // W tile update
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool rv = rb + 16 * a + i < rows;
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (rv && cb + 16 * b < c1) wbase[(16 * a + i) * ldi + 16 * b] = cv[a][i][b] - acc[a][b][i];
    }
}

// ---------------------------------------------------------------- helpers
template <typename T>
__global__ __launch_bounds__(256) void convert_kernel(const T* __restrict__ W, int64_t rows,
                                                      int64_t cols, int64_t ldw,
                                                      float* __restrict__ Wk, int64_t ldk) {
  const int64_t r = blockIdx.x;
  for (int64_t c = (int64_t)blockIdx.y * 256 + threadIdx.x; c < ldk; c += (int64_t)gridDim.y * 256)
    Wk[r * ldk + c] = (c < cols) ? (float)W[r * ldw + c] : 0.f;
}

// Act-order variant: Wk[r][j] = W[r][perm[j]] (columns in processing order;
// perm entries clamped into [0, cols)).  One workgroup per row; with `stage`
// the row of W is first copied to LDS (dynamic, cols * sizeof(T) bytes) so
// the gather reads LDS and both global passes are coalesced.
template <typename T>
__global__ __launch_bounds__(256) void convert_perm_kernel(const T* __restrict__ W, int64_t rows,
                                                           int64_t cols, int64_t ldw,
                                                           const int* __restrict__ perm,
                                                           float* __restrict__ Wk, int64_t ldk,
                                                           bool stage) {
  extern __shared__ __attribute__((aligned(16))) uint8_t convert_row[];
  T* rowbuf = reinterpret_cast<T*>(convert_row);
  const int64_t r = blockIdx.x;
  const T* src = W + r * ldw;
  if (stage) {
    for (int64_t c = threadIdx.x; c < cols; c += 256) rowbuf[c] = src[c];
    __syncthreads();
    src = rowbuf;
  }
  const int cmax = (int)(cols - 1);
  for (int64_t c = threadIdx.x; c < ldk; c += 256)
    Wk[r * ldk + c] = (c < cols) ? (float)src[min(max(perm[c], 0), cmax)] : 0.f;
}

// fp16 rows whose start is 16-byte aligned (ldw % 8 == 0): 8 columns per
// thread with one 16-byte load and two 16-byte stores.  ldk is a multiple of
// 128, so every 8-column run of Wk is whole.
__global__ __launch_bounds__(256) void convert_f16x8_kernel(const _Float16* __restrict__ W,
                                                            int64_t cols, int64_t ldw,
                                                            float* __restrict__ Wk, int64_t ldk) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  const int64_t r = blockIdx.x;
  for (int64_t c = ((int64_t)blockIdx.y * 256 + threadIdx.x) * 8; c < ldk;
       c += (int64_t)gridDim.y * 256 * 8) {
    float o[8];
    if (c + 8 <= cols) {
      const h8 v = *reinterpret_cast<const h8*>(W + r * ldw + c);
#pragma unroll
      for (int u = 0; u < 8; ++u) o[u] = (float)v[u];
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) o[u] = (c + u < cols) ? (float)W[r * ldw + c + u] : 0.f;
    }
    float4* dst = reinterpret_cast<float4*>(Wk + r * ldk + c);
    dst[0] = make_float4(o[0], o[1], o[2], o[3]);
    dst[1] = make_float4(o[4], o[5], o[6], o[7]);
  }
}

// losses[c] = sum over parts p of lpart[p][c], in a fixed order: a workgroup
// takes 16 columns; thread (s, c) sums parts s, s+16, ... and the 16 slices
// are added in slice order.
__global__ __launch_bounds__(256) void loss_reduce_kernel(const float* __restrict__ lpart,
                                                          int64_t nparts, int64_t ldk,
                                                          int64_t cols, float* __restrict__ out) {
  __shared__ float part[16][17];
  const int cl = threadIdx.x & 15, sl = threadIdx.x >> 4;
  const int64_t c = (int64_t)blockIdx.x * 16 + cl;
  float acc = 0.f;
  if (c < cols)
    for (int64_t p = sl; p < nparts; p += 16) acc += lpart[p * ldk + c];
  part[sl][cl] = acc;
  __syncthreads();
  if (sl == 0 && c < cols) {
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) tot += part[i][cl];
    out[c] = tot;
  }
}

}  // namespace

hipError_t launch_convert_w(const void* W, int w_dtype, int64_t rows, int64_t cols, int64_t ldw,
                            const int* perm, float* Wk, int64_t ldk, hipStream_t s) {
  dim3 grid((unsigned)rows, (unsigned)((ceil_div(ldk, 256) < 16) ? ceil_div(ldk, 256) : 16));
  if (perm != nullptr) {
    const int64_t rb = cols * (w_dtype == GPTQ_DTYPE_F16 ? 2 : 4);
    const bool stage = rb <= kStageBytes;
    const unsigned lds = stage ? (unsigned)rb : 0u;
    if (w_dtype == GPTQ_DTYPE_F16)
      hipLaunchKernelGGL(convert_perm_kernel<_Float16>, dim3((unsigned)rows), dim3(256), lds, s,
                         reinterpret_cast<const _Float16*>(W), rows, cols, ldw, perm, Wk, ldk,
                         stage);
    else
      hipLaunchKernelGGL(convert_perm_kernel<float>, dim3((unsigned)rows), dim3(256), lds, s,
                         reinterpret_cast<const float*>(W), rows, cols, ldw, perm, Wk, ldk, stage);
    return hipGetLastError();
  }
  const bool v8 = (ldw % 8 == 0) && ((reinterpret_cast<uintptr_t>(W) & 15) == 0) &&
                  ((reinterpret_cast<uintptr_t>(Wk) & 15) == 0);
  if (w_dtype == GPTQ_DTYPE_F16 && v8)
    hipLaunchKernelGGL(convert_f16x8_kernel, dim3((unsigned)rows, (unsigned)ceil_div(ldk, 2048)),
                       dim3(256), 0, s, reinterpret_cast<const _Float16*>(W), cols, ldw, Wk, ldk);
  else if (w_dtype == GPTQ_DTYPE_F16)
    hipLaunchKernelGGL(convert_kernel<_Float16>, grid, dim3(256), 0, s,
                       reinterpret_cast<const _Float16*>(W), rows, cols, ldw, Wk, ldk);
  else
    hipLaunchKernelGGL(convert_kernel<float>, grid, dim3(256), 0, s,
                       reinterpret_cast<const float*>(W), rows, cols, ldw, Wk, ldk);
  return hipGetLastError();
}

hipError_t launch_sweep_block(float* Wk, int64_t ldk, int64_t rows, int64_t cols, int i1, int p0,
                              const float* Hinv, int bits, int groupsize, uint8_t* codes,
                              float* scales, float* zeros, float* Err, float* lpart,
                              hipStream_t s) {
  dim3 grid((unsigned)ceil_div(rows, kSweepRows));
#define GPTQ_SWEEP(G)                                                                          \
  hipLaunchKernelGGL(sweep_kernel<G>, grid, dim3(256), 0, s, Wk, ldk, rows, cols, i1, p0,     \
                     Hinv, bits, groupsize, codes, scales, zeros, Err, lpart)
  switch (groupsize) {
    case 16: GPTQ_SWEEP(16); break;
    case 32: GPTQ_SWEEP(32); break;
    case 64: GPTQ_SWEEP(64); break;
    case 128: GPTQ_SWEEP(128); break;
    default: GPTQ_SWEEP(0); break;
  }
#undef GPTQ_SWEEP
  return hipGetLastError();
}

hipError_t launch_lazy_update(float* Wk, int64_t ldk, int64_t rows, int64_t cols, int k0, int k1,
                              int c0, int c1, const float* Err, const float* Hinv, hipStream_t s) {
  if (c1 <= c0 || k1 <= k0) return hipSuccess;
  const int64_t ncol = ceil_div(c1 - c0, LT);
  // big updates: 128x128 tiles; small ones: 32x128 tiles so more CUs take
  // part, with all of K (at most 128) and the W tile loaded up front
  if (ncol * ceil_div(rows, 128) >= 512) {
    dim3 grid((unsigned)ncol, (unsigned)ceil_div(rows, 128));
    hipLaunchKernelGGL((lazy_kernel<4, false>), grid, dim3(256), 0, s, Wk, ldk, rows, cols, k0, k1,
                       c0, c1, Err, Hinv);
  } else {
    dim3 grid((unsigned)ncol, (unsigned)ceil_div(rows, 32));
    if (k1 - k0 <= 4 * LK)
      hipLaunchKernelGGL((lazy_kernel<1, true>), grid, dim3(256), 0, s, Wk, ldk, rows, cols, k0,
                         k1, c0, c1, Err, Hinv);
    else
      hipLaunchKernelGGL((lazy_kernel<1, false>), grid, dim3(256), 0, s, Wk, ldk, rows, cols, k0,
                         k1, c0, c1, Err, Hinv);
  }
  return hipGetLastError();
}

hipError_t launch_loss_reduce(const float* lpart, int64_t nparts, int64_t cols, float* losses,
                              hipStream_t s) {
  const int64_t ldk = round_up(cols, kBlock);
  hipLaunchKernelGGL(loss_reduce_kernel, dim3((unsigned)ceil_div(cols, 16)), dim3(256), 0, s,
                     lpart, nparts, ldk, cols, losses);
  return hipGetLastError();
}

}  // namespace gptq
