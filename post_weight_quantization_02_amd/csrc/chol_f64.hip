// Hinv preparation in fp64: damp, Cholesky, triangular inverse and the fp32
// upper factor of the inverse.
//
// Result: "GPTQ, Line by Line: Hessian-Based Weight Quantization", percdamp
// question (add percdamp * mean(diag H) to the diagonal) and Cholesky
// question (the upper Cholesky factor of the damped inverse, which the page
// forms by factoring, inverting through the factor and factoring the
// inverse; the same three calls appear in the gptq_quantize_layer listing of
// "GPTQ-style round-to-nearest with Hessian weighting").
//
// Route: with J the reversal permutation and L the lower Cholesky factor of
// J H_d J, H_d^-1 = J L^-T L^-1 J = M^T M for M = J L^-1 J, which is upper
// triangular with a positive diagonal, so M is that factor.  One
// factorization and one triangular inverse (2/3 d^3 flops) replace two
// factorizations, the inverse and the product L^-T L^-1 (4/3 d^3).  When the
// factorization of J H_d J fails, the three-step route runs in forward order,
// so the failing pivot reported is the one of the factor of H_d (or of its
// inverse).
//
// gfx950 design:
//   * Everything runs in fp64: the sweep's integer decisions are sensitive
//     to the factor's accuracy, and fp32 factorizations of calibration
//     Hessians lose several digits.  fp64 MFMA (v_mfma_f64_16x16x4_f64)
//     carries every O(d^3) product; each 64x64 diagonal block is factored and
//     inverted by one workgroup, in registers (16-column steps on one wave
//     with DPP, readlane and ds_bpermute) and LDS (the 16x16 L blocks).
//   * Blocked right-looking Cholesky with 64-wide panels: one workgroup
//     factors and inverts the panel's diagonal block (diag_factor), one
//     workgroup per 64-row block below solves against it (a product with the
//     inverse), then one MFMA kernel applies the rank-64 update to the lower
//     triangle of the trailing matrix; its workgroup 0 updates the next
//     diagonal block first and factors it while the others finish (lookahead
//     of one panel).  Once the trailing matrix is small, solve and update
//     share one launch (potrf_fused_kernel).  Products with an inverted
//     diagonal block skip the k-steps its triangle makes zero, and the
//     diagonal update forms only the lower blocks.  Large matrices use two
//     levels (see the host code).
//   * The triangular inverse uses recursive doubling: the 64x64 diagonal
//     blocks are inverted during the factorization, then each level combines
//     neighbouring inverted blocks with X21 = -C^-1 (B A^-1), two batched MFMA
//     launches per level.
//   * L^-T L^-1 is one MFMA launch over the lower tiles, each tile with its
//     own K range (the triangle of L^-1 makes the rest zero).
//   * The products run on 64x64 or 128x128 fp64 MFMA tiles, chosen by size;
//     tiles of triangular products are ordered longest first.
//   * Only the lower triangle of A is ever read: the damped copy writes just
//     that half.
//   * A failed pivot (<= 0 or NaN) sets a device flag with atomicMin of its
//     1-based index; the host reads it once at the end.
#include <limits.h>

#include <atomic>
#include <utility>

#include "common.h"

namespace gptq {

namespace {

constexpr int NB = kPanel;  // 64
constexpr int PP = NB + 2;  // LDS pitch (doubles) of the 64x64 panel tiles: conflict-free
                            // MFMA operand reads (rows m = lane%16, columns k = lane/16)

// 1/sqrt(p): hardware estimate (measured 5.2e-8 relative) and one Newton
// step (measured 4.1e-15 relative over 2^20 values from 2^-40 to 2^41; a
// second step gives 2.4e-16).  It sits on the serial pivot chain of every
// 64x64 diagonal factorization; 4e-15 per pivot is far below what the fp32
// Hinv resolves.
__device__ inline double rsqrt_f64(double p) {
  const double r = __builtin_amdgcn_rsq(p);
  return r * __builtin_fma(-0.5 * p * r, r, 1.5);
}

// 1/p: hardware estimate and one Newton step (relative error of order the
// square of the estimate's, as for rsqrt_f64).  The pivot chain of the 16x16
// factorization needs 1/p for its multipliers; taking it here rather than as
// the square of rsqrt_f64 puts two fewer dependent operations on that chain.
__device__ inline double rcp_f64(double p) {
  const double r = __builtin_amdgcn_rcp(p);
  return __builtin_fma(r, __builtin_fma(-p, r, 1.0), r);
}
constexpr int GT = 64;      // GEMM tile edge
constexpr int GK = 16;      // GEMM K chunk

// -------------------------------------------------------------- damping
__global__ __launch_bounds__(256) void damp_lambda_kernel(const float* __restrict__ H, int d,
                                                          double percdamp, double* lam,
                                                          int* flag) {
  __shared__ double part[256];
  double s = 0.0;
  for (int i = threadIdx.x; i < d; i += 256) s += (double)H[(int64_t)i * d + i];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    *lam = percdamp * (part[0] / (double)d);
    *flag = INT_MAX;
  }
}

// A = H + lambda I in fp64, lower triangle only (one workgroup per row; the
// factorizations never read the upper triangle).
__global__ __launch_bounds__(256) void damp_copy_kernel(const float* __restrict__ H, int d,
                                                        const double* lam, double* __restrict__ A) {
  const int64_t i = blockIdx.x;
  const double l = *lam;
  for (int64_t j = threadIdx.x; j <= i; j += 256) {
    double v = (double)H[i * d + j];
    if (j == i) v += l;
    A[i * d + j] = v;
  }
}

// Reversed order: A[i][j] = H[d-1-i][d-1-j] + lambda [i == j] for j <= i,
// read from H's lower triangle as H[d-1-j][d-1-i].  One workgroup per 64x64
// tile of A's lower triangle; the source tile is read along H's rows and
// transposed through LDS, so reads and writes are both coalesced.
__global__ __launch_bounds__(256) void damp_copy_rev_kernel(const float* __restrict__ H, int d,
                                                            const double* lam,
                                                            double* __restrict__ A) {
  __shared__ float t[64][65];
  int bi, bj;
  lower_tile(blockIdx.x, bi, bj);
  const int i0 = bi * 64, j0 = bj * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  // t[r][c] = H[d-1-(j0+r)][d-1-(i0+c)], the entry that lands at A[i0+c][j0+r]
  for (int r = ty; r < 64; r += 4) {
    const int j = j0 + r, i = i0 + tx;
    t[r][tx] = (i < d && j <= i) ? H[(int64_t)(d - 1 - j) * d + (d - 1 - i)] : 0.f;
  }
  __syncthreads();
  const double l = *lam;
  for (int r = ty; r < 64; r += 4) {
    const int i = i0 + r, j = j0 + tx;
    if (i < d && j <= i) {
      double v = (double)t[tx][r];
      if (j == i) v += l;
      A[(int64_t)i * d + j] = v;
    }
  }
}

// Act-order variant: A = P H P^T + lambda I with (P H P^T)[i][j] =
// H[q[i]][q[j]], lower triangle, q[i] = perm[i] (or perm[d-1-i] with `rev`);
// H must hold both triangles.  One workgroup per row i; with `stage` row
// q[i] of H is first copied to LDS (dynamic, d floats) so the gather reads
// LDS.  perm entries are clamped into [0, d).
__global__ __launch_bounds__(256) void damp_copy_perm_kernel(const float* __restrict__ H, int d,
                                                             const int* __restrict__ perm,
                                                             const double* lam,
                                                             double* __restrict__ A, bool stage,
                                                             bool rev) {
  extern __shared__ float hrowbuf[];
  const int64_t i = blockIdx.x;
  const double l = *lam;
  auto q = [&](int64_t k) -> int64_t {
    return min(max(perm[rev ? d - 1 - k : k], 0), d - 1);
  };
  const float* hrow = H + q(i) * d;
  if (stage) {
    for (int64_t j = threadIdx.x; j < d; j += 256) hrowbuf[j] = hrow[j];
    __syncthreads();
    hrow = hrowbuf;
  }
  for (int64_t j = threadIdx.x; j <= i; j += 256) {
    double v = (double)hrow[q(j)];
    if (j == i) v += l;
    A[i * d + j] = v;
  }
}

// Row of the 16x16 fp64 MFMA result held in element i of lane `lane`
// (the fp64 variant interleaves rows: lane/16, lane/16 + 4, ...).
__device__ inline int mfma64_row(int lane, int i) { return (lane >> 4) + 4 * i; }

// -------------------------------------------------------------- panel
// Value of v held by lane J of this lane's row of 16 (DPP row_newbcast; one
// v_mov_b64_dpp; with every row and bank enabled the old value is unused).
template <int J>
__device__ inline double row_bcast(double v) {
  return __builtin_amdgcn_update_dpp(0.0, v, 0x150 + J, 0xF, 0xF, true);
}

// ---- 16x16 blocks in registers ("CS layout")
// Lane (m, g) = (lane % 16, lane / 16) holds B[m][g + 4i] in element i of a
// double[4]: row m of the block, every fourth column.  This is the layout in
// which v_mfma_f64_16x16x4f64 returns a product (its element i at lane
// (n, q) is D[q + 4i][n], i.e. row n of D^T), and element s is also the
// operand of k-step s when K = 16 runs as k = g + 4s.  So, for blocks in this
// layout, MFMA(A = P[s], B = Q[s]) accumulates (Q P^T) into a block held in
// this layout, and every product below stays in it.

// Value of v at lane L of the wave (uniform).
template <int L>
__device__ inline double lane_value(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)u, L);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(u >> 32), L);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Value of v at lane addr / 4 (ds_bpermute: the LDS crossbar, no LDS memory).
__device__ inline double lane_gather(double v, int addr) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_ds_bpermute(addr, (int)(uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_ds_bpermute(addr, (int)(uint32_t)(u >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Step J = 4Q + K of the in-wave 16x16 Cholesky and inverse (see factor16).
// c[k] holds A[m][4Q + k] in every lane of row m; row J of anything held in
// every lane group comes from lane J of the group (DPP row_newbcast).
template <int Q, int K>
__device__ inline void factor16_step(double (&a)[4], double (&y)[4], double (&c)[4], int m) {
  constexpr int J = 4 * Q + K;
  const double p = row_bcast<J>(c[K]);                // pivot A[J][J]
  // multiplier of row J for the rows below it, and exactly 0 for the others
  // (also when A[m][J] is not finite), so no step after a row's own touches
  // its diagonal entry
  const double t = (m > J) ? c[K] * rcp_f64(p) : 0.0;
  // rows below J: the columns past J get the right-looking update with row J
#pragma unroll
  for (int k = K + 1; k < 4; ++k) c[k] = __builtin_fma(-t, row_bcast<J>(c[k]), c[k]);
#pragma unroll
  for (int i = Q + 1; i < 4; ++i) a[i] = __builtin_fma(-t, row_bcast<J>(a[i]), a[i]);
  // forward substitution L Y = I: rows below J lose t times row J of Y
#pragma unroll
  for (int i = 0; i <= Q; ++i) y[i] = __builtin_fma(-t, row_bcast<J>(y[i]), y[i]);
}

// Columns 4Q .. 4Q+3 (element Q of lane groups 0..3): gathered once into
// every lane of each row, stepped there, and handed back to their owners.
template <int Q>
__device__ inline void factor16_quad(double (&a)[4], double (&y)[4], int m, int g,
                                     const int (&gaddr)[4]) {
  double c[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) c[k] = lane_gather(a[Q], gaddr[k]);
  factor16_step<Q, 0>(a, y, c, m);
  factor16_step<Q, 1>(a, y, c, m);
  factor16_step<Q, 2>(a, y, c, m);
  factor16_step<Q, 3>(a, y, c, m);
  double v = c[0];
  v = (g == 1) ? c[1] : v;
  v = (g == 2) ? c[2] : v;
  v = (g == 3) ? c[3] : v;
  a[Q] = v;
}

// Cholesky factor and inverse of one symmetric 16x16 block held by a single
// wave in CS layout, with no barrier and no LDS memory.  Step j reads the
// pivot with a readlane, column j of the block from its lane group
// (ds_bpermute) and row j from lane j of each group (DPP row_newbcast),
// applies the right-looking update a[i][l] -= (a[i][j] / p) a[j][l] to the
// columns past j, and the forward substitution of L Y = I: rows below j lose
// (L[i][j] / L[j][j]) times row j of Y.  Nothing a step does depends on
// 1 / sqrt(p), so the scalings by it wait for the end: a column is final
// once its step has passed (later steps change only columns past theirs, and
// its diagonal entry is its pivot), so column j of L is that column times
// 1 / sqrt(p_j), and row i of L^-1 is row i of Y times 1 / sqrt(p_i).  On
// return a[] holds L (entries above the diagonal are meaningless) and y[]
// holds L^-1 (exact zeros above the diagonal).  The first pivot that is not
// > 0 (or NaN) is reported through atomicMin(flag, info_base + j + 1) when
// `report` is set.
__device__ __attribute__((always_inline)) inline void factor16(double (&a)[4], double (&y)[4],
                                                               int m, int g, int* flag,
                                                               int info_base, bool report) {
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] = (g + 4 * i == m) ? 1.0 : 0.0;
  int gaddr[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) gaddr[q] = (m + 16 * q) * 4;
  factor16_quad<0>(a, y, m, g, gaddr);
  factor16_quad<1>(a, y, m, g, gaddr);
  factor16_quad<2>(a, y, m, g, gaddr);
  factor16_quad<3>(a, y, m, g, gaddr);
  // pivot of row m: the diagonal entry, element m / 4 of lane (m, m % 4)
  const int im = m >> 2;
  double own = a[0];
  own = (im == 1) ? a[1] : own;
  own = (im == 2) ? a[2] : own;
  own = (im == 3) ? a[3] : own;
  const double pm = lane_gather(own, (m + 16 * (m & 3)) * 4);
  const double ysc = rsqrt_f64(pm);
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] *= ysc;
  // pivot of column g + 4i: element i of lane (g + 4i, g)
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] *= rsqrt_f64(lane_gather(a[i], (g + 4 * i + 16 * g) * 4));
  // lanes 0..15 are rows 0..15 of lane group 0
  const uint64_t badm = __builtin_amdgcn_ballot_w64(g == 0 && !(pm > 0.0));
  if (report && badm != 0 && (threadIdx.x & 63) == 0)
    atomicMin(flag, info_base + __builtin_ctzll(badm) + 1);
}

// LDS of the diagonal-block factorization; the trailing update reuses S and
// Xs as its two panel tiles.
struct DiagLds {
  double S[NB][PP];   // the block (lower triangle); blocks L_IJ below the diagonal as they form
  double Xs[NB][PP];  // blocks of L^-1 on and below the diagonal, row-major
};

// Block (I, K) of a row-major LDS tile in CS layout.  With SYM, a diagonal
// block is read from its lower triangle (the tile holds a symmetric matrix).
template <bool SYM>
__device__ inline void load_cs(const double (*S)[PP], int I, int K, int m, int g, double (&v)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = g + 4 * i;
    const bool up = SYM && (I == K) && (c > m);
    v[i] = up ? S[16 * I + c][16 * K + m] : S[16 * I + m][16 * K + c];
  }
}

__device__ inline void store_cs(double (*S)[PP], int I, int K, int m, int g, const double (&v)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) S[16 * I + m][16 * K + g + 4 * i] = v[i];
}

// L_IJ = A_IJ X_JJ^T from X_JJ and A_IJ in CS layout.
__device__ inline void l_block(const double (&x)[4], const double (&aij)[4], double (&l)[4]) {
  f64x4 t = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int s = 0; s < 4; ++s) t = __builtin_amdgcn_mfma_f64_16x16x4f64(x[s], aij[s], t, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) l[i] = t[i];
}

// A_IK -= L_IJ L_KJ^T, all in CS layout.
__device__ inline void rank16_update(double (&aik)[4], const double (&lij)[4],
                                     const double (&lkj)[4]) {
  f64x4 c = {aik[0], aik[1], aik[2], aik[3]};
#pragma unroll
  for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f64_16x16x4f64(-lkj[s], lij[s], c, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) aik[i] = c[i];
}

// T += L_JK X_KJ' with L_JK in CS layout (from S) and X_KJ' as the B operand
// (from Xs); T comes back in MFMA result layout (element i at lane (m, g) is
// T[g + 4i][m]), which is the B operand of the product with X_JJ that follows.
__device__ inline void t_accum(const double (*S)[PP], const double (*Xs)[PP], int J, int K, int Jp,
                               int m, int g, f64x4& t) {
  double l[4];
  load_cs<false>(S, J, K, m, g, l);
#pragma unroll
  for (int s = 0; s < 4; ++s)
    t = __builtin_amdgcn_mfma_f64_16x16x4f64(l[s], Xs[16 * K + g + 4 * s][16 * Jp + m], t, 0, 0, 0);
}

// X_JJ' = -X_JJ T, to Xs.
__device__ inline void x_block(double (*Xs)[PP], int J, int Jp, int m, int g, const f64x4& t) {
  double x[4];
  load_cs<false>(Xs, J, J, m, g, x);
  f64x4 r = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int s = 0; s < 4; ++s) r = __builtin_amdgcn_mfma_f64_16x16x4f64(-x[s], t[s], r, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * J + g + 4 * i, col = 16 * Jp + m;
    Xs[row][col] = r[i];
  }
}

struct DiagCtx {
  double (*S)[PP];
  double (*Xs)[PP];
  int w, m, g;
  int* flag;
  int info_base;  // info_offset + k
};

// Phase J of diag_factor (see there).
template <int J>
__device__ __attribute__((always_inline)) inline void diag_phase(const DiagCtx& cx,
                                                                 double (&row)[4][4], f64x4& tsum) {
  const int w = cx.w, m = cx.m, g = cx.g;
  if (w == J) {
    double y[4];
    factor16(row[J], y, m, g, cx.flag, cx.info_base + 16 * J, true);
    store_cs(cx.Xs, J, J, m, g, y);
    store_cs(cx.S, J, J, m, g, row[J]);
  }
  __syncthreads();  // X_JJ published
  if (w > J) {
    double x[4], l[4];
    load_cs<false>(cx.Xs, J, J, m, g, x);
    l_block(x, row[J], l);
    store_cs(cx.S, w, J, m, g, l);
#pragma unroll
    for (int i = 0; i < 4; ++i) row[J][i] = l[i];
    if constexpr (J + 1 < 4) {
      if (w == J + 1) rank16_update(row[J + 1], l, l);
    }
  } else if (w < J) {
    x_block(cx.Xs, J, w, m, g, tsum);
  }
  if constexpr (J < 3) {
    __syncthreads();  // L_wJ published
    if (w > J + 1) {
      // the rest of this wave's row: A_wK -= L_wJ L_KJ^T, K = J+1..w
#pragma unroll
      for (int K = J + 1; K < 4; ++K) {
        if (K < w) {
          double lk[4];
          load_cs<false>(cx.S, K, J, m, g, lk);
          rank16_update(row[K], row[J], lk);
        } else if (K == w) {
          rank16_update(row[K], row[J], row[J]);
        }
      }
    } else if (w <= J) {
      // sum for X_{J+1, w}: L_{J+1,K} X_{K,w}, K = w..J
      tsum = f64x4{0.0, 0.0, 0.0, 0.0};
      for (int K = w; K <= J; ++K) t_accum(cx.S, cx.Xs, J + 1, K, w, m, g, tsum);
    }
  }
}

// Factor the 64x64 block in sh.S (lower triangle; rows past kb are identity)
// and invert the factor: L goes to the lower triangle of the block at
// A[k.., k..], L^-1 (zeros above its diagonal) to Xd.  A barrier must
// separate the filling of sh.S from the call.
//
// Wave w owns block row w of the tile and keeps its blocks A_w0..A_ww in
// registers (CS layout).  Phase J: wave J factors and inverts A_JJ on its
// own (factor16) and publishes X_JJ; each wave w > J then forms
// L_wJ = A_wJ X_JJ^T and publishes it, and wave J+1 updates A_{J+1,J+1} with
// its own L_{J+1,J} and goes straight on to the next factorization while the
// others apply the remaining rank-16 updates of their rows.  The waves whose
// rows are done build the blocks of L^-1 below the diagonal,
// X_JJ' = -X_JJ sum_{K=J'..J-1} L_JK X_KJ', one block column each: the sum
// before X_JJ is ready, the last product after.  Blocks are published in LDS
// only (L in sh.S, L^-1 in sh.Xs); the whole workgroup copies both tiles to
// global memory at the end, row by row, so no global store sits on the
// serial chain of phases.  All 16x16 products are v_mfma_f64_16x16x4f64.
__device__ __attribute__((always_inline)) inline void diag_factor(DiagLds& sh, double* __restrict__ A, int lda, int k, int kb,
                                   int* flag, int info_offset, double* __restrict__ Xd,
                                   int ldxd) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  DiagCtx cx;
  cx.S = sh.S;
  cx.Xs = sh.Xs;
  cx.w = __builtin_amdgcn_readfirstlane(tid >> 6);
  cx.m = lane & 15;
  cx.g = lane >> 4;
  cx.flag = flag;
  cx.info_base = info_offset + k;

  // this wave's block row A_w0 .. A_ww
  double row[4][4];
#pragma unroll
  for (int K = 0; K < 4; ++K)
    if (K <= cx.w) load_cs<true>(sh.S, cx.w, K, cx.m, cx.g, row[K]);
  __syncthreads();  // every wave has its row before L blocks overwrite S
  f64x4 tsum = {0.0, 0.0, 0.0, 0.0};
  diag_phase<0>(cx, row, tsum);
  diag_phase<1>(cx, row, tsum);
  diag_phase<2>(cx, row, tsum);
  diag_phase<3>(cx, row, tsum);
  __syncthreads();  // every block of L and L^-1 is in LDS
  // rows below kb: L's lower triangle to A, L^-1 to Xd with the blocks above
  // its block diagonal zero (the diagonal blocks hold exact zeros above the
  // diagonal); each store instruction writes 64 consecutive elements of a row
  double* __restrict__ Ak = A + (int64_t)k * lda + k;
  const int c = tid & 63, r0 = tid >> 6;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int r = r0 + 4 * q;
    if (r < kb && c < kb) {
      if (c <= r) Ak[(int64_t)r * lda + c] = sh.S[r][c];
      Xd[(int64_t)r * ldxd + c] = ((c >> 4) <= (r >> 4)) ? sh.Xs[r][c] : 0.0;
    }
  }
}

// One workgroup factors the 64x64 diagonal block of the panel at column k and
// inverts the factor (diag_factor); the block is read from the lower
// triangle of A.  Used for the first panel; later diagonal blocks are
// factored inside the previous panel's trailing update.
__global__ __launch_bounds__(256) void potrf_diag_kernel(double* __restrict__ A, int lda, int d,
                                                         int k, int* flag, int info_offset,
                                                         double* __restrict__ Xd, int ldxd) {
  __shared__ DiagLds sh;
  const int tid = threadIdx.x;
  const int kb = min(NB, d - k);
  double v[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int e = tid + 256 * q;
    const int i = e >> 6, l = e & 63;
    double x = (i == l) ? 1.0 : 0.0;
    if (i < kb && l <= i) x = A[(int64_t)(k + i) * lda + k + l];
    v[q] = x;
  }
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int e = tid + 256 * q;
    sh.S[e >> 6][e & 63] = v[q];
  }
  __syncthreads();
  diag_factor(sh, A, lda, k, kb, flag, info_offset, Xd, ldxd);
}

// 64x64x64 fp64 MFMA product on LDS tiles: acc += P (64 x K) * Q^T, with
// P[m][kk] and Q[n][kk] stored row-major at pitch PP.  Wave w owns the
// 32x32 quadrant (w/2, w%2) as 2x2 tiles of 16x16.
__device__ inline void mma64_f64(const double (*P)[PP], const double (*Q)[PP], int K,
                                 f64x4 (&acc)[2][2], int lane, int wm, int wn) {
  for (int ks = 0; ks < K; ks += 4) {
    const int kr = ks + (lane >> 4);
    double af[2], bf[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) af[a] = P[32 * wm + 16 * a + (lane & 15)][kr];
#pragma unroll
    for (int b = 0; b < 2; ++b) bf[b] = Q[32 * wn + 16 * b + (lane & 15)][kr];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(af[a], bf[b], acc[a][b], 0, 0, 0);
  }
}


// Row block w (rows 16w..16w+15, all 64 columns) of P X^T, with P and X
// row-major 64x64 LDS tiles and X lower triangular (an inverted diagonal
// block): column c of the product only takes k <= c, so column block cb runs
// the first 16(cb + 1) k-steps.  Each wave issues 40 MFMAs instead of the 64
// of a full product, and the k-steps left out would only add exact zeros, so
// every element is the same as the full product's.  o[cb] holds block
// (w, cb) in the 16x16 fp64 result layout.
__device__ inline void panel_times_xt(const double (*P)[PP], const double (*X)[PP], f64x4 (&o)[4],
                                      int lane, int w) {
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) o[cb] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int ks = 0; ks < NB; ks += 4) {
    const int kr = ks + (lane >> 4);
    const double a = P[16 * w + (lane & 15)][kr];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
      if (ks < 16 * (cb + 1))
        o[cb] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, X[16 * cb + (lane & 15)][kr], o[cb], 0, 0,
                                                     0);
  }
}

// Element i of o[cb] from panel_times_xt: its row and column in the 64x64 tile.
__device__ inline int strip_row(int w, int lane, int i) { return 16 * w + mfma64_row(lane, i); }
__device__ inline int strip_col(int cb, int lane) { return 16 * cb + (lane & 15); }

// The lower 16x16 blocks (ra >= cb) of the symmetric 64x64 product P P^T,
// which is all a diagonal tile's factorization reads: ten blocks, three or
// two per wave (48 MFMAs at most instead of 64).  Wave w forms block
// (kSymRa[w][s], kSymCb[w][s]) for s < kSymCnt[w].
constexpr int kSymCnt[4] = {3, 3, 2, 2};
constexpr int kSymRa[4][3] = {{3, 3, 3}, {3, 2, 2}, {2, 1, 1}, {1, 0, 0}};
constexpr int kSymCb[4][3] = {{3, 2, 1}, {0, 2, 1}, {0, 1, 1}, {0, 0, 0}};

template <int W>
__device__ inline void sym_lower_product_w(const double (*P)[PP], f64x4 (&acc)[3], int lane) {
#pragma unroll
  for (int s = 0; s < 3; ++s) acc[s] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int ks = 0; ks < NB; ks += 4) {
    const int kr = ks + (lane >> 4);
#pragma unroll
    for (int s = 0; s < kSymCnt[W]; ++s)
      acc[s] = __builtin_amdgcn_mfma_f64_16x16x4f64(P[16 * kSymRa[W][s] + (lane & 15)][kr],
                                                    P[16 * kSymCb[W][s] + (lane & 15)][kr], acc[s],
                                                    0, 0, 0);
  }
}

// w must be the same in every lane of the wave.  Each wave's blocks are fixed
// at compile time, so its operand reads carry no branches and are issued
// ahead of the products.
__device__ inline void sym_lower_product(const double (*P)[PP], f64x4 (&acc)[3], int lane, int w) {
  switch (w) {
    case 0: sym_lower_product_w<0>(P, acc, lane); break;
    case 1: sym_lower_product_w<1>(P, acc, lane); break;
    case 2: sym_lower_product_w<2>(P, acc, lane); break;
    default: sym_lower_product_w<3>(P, acc, lane); break;
  }
}

// L_ik = A_ik X_kk^T for the 64-row blocks below the diagonal block
// (one workgroup per block; X_kk = L_kk^-1 from the diagonal kernel).
__global__ __launch_bounds__(256) void potrf_trsm_kernel(double* __restrict__ A, int lda, int d,
                                                         int k, const double* __restrict__ Xd,
                                                         int ldxd) {
  __shared__ double Bs[NB][PP];
  __shared__ double Xs[NB][PP];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int kb = min(NB, d - k);
  const int row0 = k + NB * (blockIdx.x + 1);
  const int rb = min(NB, d - row0);
  const int j = tid & 63, i0 = tid >> 6;
  double bv[16], xv[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int i = i0 + 4 * q;
    bv[q] = (i < rb && j < kb) ? A[(int64_t)(row0 + i) * lda + k + j] : 0.0;
    xv[q] = (i < kb && j < kb) ? Xd[(int64_t)i * ldxd + j] : 0.0;
  }
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    Bs[i0 + 4 * q][j] = bv[q];
    Xs[i0 + 4 * q][j] = xv[q];
  }
  __syncthreads();
  f64x4 o[4];
  panel_times_xt(Bs, Xs, o, lane, wave);
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = strip_row(wave, lane, i), c = strip_col(cb, lane);
      if (r < rb && c < kb) A[(int64_t)(row0 + r) * lda + k + c] = o[cb][i];
    }
}

// Lower tile p of the trailing matrix A[t0:, t0:] numbered column by column
// (column tj holds nt - tj tiles): its top-left corner, and whether it is a
// diagonal tile.
__device__ inline bool tile_coords(int p, int nt, int t0, int& r0, int& c0) {
  int ti = p, tj = 0;
  while (ti >= nt - tj) {
    ti -= nt - tj;
    ++tj;
  }
  ti += tj;
  r0 = t0 + NB * ti;
  c0 = t0 + NB * tj;
  return ti == tj;
}

// Workgroup 0 of a panel step (lookahead): the next diagonal block
// A(t0, t0), t0 = k + 64, takes the rank-64 update with L(t0, k), the panel
// block below the diagonal, and is then factored and inverted in place
// (diag_factor).  Only the lower 16x16 blocks of the update are formed.
// FUSED: L(t0, k) is formed here from the raw block A(t0, k) and X_kk (the
// inverted diagonal block at Xk) and also written to Lout (row pitch ldo);
// otherwise it is read from A, where the panel solve left it.
template <bool FUSED>
__device__ __attribute__((always_inline)) inline void lookahead_diag(
    DiagLds& sh, double* __restrict__ A, int lda, int d, int k, const double* __restrict__ Xk,
    double* __restrict__ Lout, int ldo, int* flag, int info_offset, double* __restrict__ Xn,
    int ldxn) {
  const int t0 = k + NB;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = tid & 63, i0 = tid >> 6;
  const int kb = min(NB, d - t0);
  const int cnt = kSymCnt[wave];
  // every load up front: the panel block (rows clamped; rows past the matrix
  // reach only masked elements), X_kk, and this wave's C blocks
  double pv[16], xv[16], cs[3][4];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int i = i0 + 4 * q;
    pv[q] = A[(int64_t)min(t0 + i, d - 1) * lda + k + j];
    if (FUSED) xv[q] = Xk[(int64_t)i * ldo + j];
  }
#pragma unroll
  for (int s = 0; s < 3; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * kSymRa[wave][s] + mfma64_row(lane, i);
      const int c = 16 * kSymCb[wave][s] + (lane & 15);
      cs[s][i] = (s < cnt) ? A[(int64_t)min(t0 + r, d - 1) * lda + min(t0 + c, d - 1)] : 0.0;
    }
  if (FUSED) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      sh.S[i0 + 4 * q][j] = pv[q];
      sh.Xs[i0 + 4 * q][j] = xv[q];
    }
    __syncthreads();
    f64x4 o[4];
    panel_times_xt(sh.S, sh.Xs, o, lane, wave);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = strip_row(wave, lane, i), c = strip_col(cb, lane);
        if (r < kb) Lout[(int64_t)r * ldo + c] = o[cb][i];
      }
    __syncthreads();  // every wave is done with the raw block and X_kk
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) sh.Xs[strip_row(wave, lane, i)][strip_col(cb, lane)] = o[cb][i];
  } else {
#pragma unroll
    for (int q = 0; q < 16; ++q) sh.Xs[i0 + 4 * q][j] = pv[q];
  }
  __syncthreads();
  f64x4 acc[3];
  sym_lower_product(sh.Xs, acc, lane, wave);
  // the updated block goes to sh.S (rows past the matrix become identity);
  // diag_factor reads only its lower blocks and the lower triangle of the
  // diagonal ones
#pragma unroll
  for (int s = 0; s < 3; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * kSymRa[wave][s] + mfma64_row(lane, i);
      const int c = 16 * kSymCb[wave][s] + (lane & 15);
      if (s < cnt) sh.S[r][c] = (r < kb && c < kb) ? cs[s][i] - acc[s][i] : ((r == c) ? 1.0 : 0.0);
    }
  __syncthreads();
  diag_factor(sh, A, lda, t0, kb, flag, info_offset, Xn, ldxn);
}

// Update after panel k inside an outer panel: A_ij -= L_ik L_jk^T for the
// 64x64 tiles i >= j of A[t0:, t0:], t0 = k + 64, whose column block j lies
// in the first `ncol` blocks (`ntiles` tiles, numbered column by column),
// both panel blocks in LDS.  Workgroup 0 takes tile (0, 0), the next panel's
// diagonal block, keeps the updated block in LDS and goes on to factor and
// invert it (diag_factor): the next panel's serial step runs while the other
// workgroups are still updating, instead of after them (lookahead of one
// panel).  The grid may be smaller than the tile count: workgroup b > 0 then
// takes tiles b, b + G - 1, b + 2(G - 1), ... (G = gridDim.x) and loads the
// next tile's panel blocks and C tile into registers before the current
// tile's MFMAs, so a large early update is not a sequence of rounds that each
// wait for their loads.
__global__ __launch_bounds__(256, 2) void potrf_update_kernel(double* __restrict__ A, int lda, int d,
                                                           int k, int nt, int ntiles, int* flag,
                                                           int info_offset, double* __restrict__ Xn,
                                                           int ldxn) {
  __shared__ DiagLds sh;
  if (blockIdx.x == 0) {
    lookahead_diag<false>(sh, A, lda, d, k, nullptr, nullptr, 0, flag, info_offset, Xn, ldxn);
    return;
  }
  double (*Ps)[PP] = sh.S;
  double (*Qs)[PP] = sh.Xs;
  const int t0 = k + NB;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int j = tid & 63, i0 = tid >> 6;
  auto coords = [&](int p, int& r0, int& c0) { return tile_coords(p, nt, t0, r0, c0); };
  // Every load is issued, with its row and column clamped into the matrix,
  // so the compiler can count outstanding loads exactly and waits only for
  // the registers each use needs.  Clamped values are not masked: output
  // element (r, c) reads only P row r, Q row c and C(r, c), so they reach
  // only elements with r >= d or c >= d, which are never stored (the
  // diagonal block of workgroup 0 is masked when it goes to LDS).  A diagonal
  // tile's Q rows are its P rows; its multiply reads P twice.  Part q of a
  // tile's loads (q = 0..15): panel rows i0 + 4q of P and Q, and one of this
  // lane's sixteen C elements.
  auto load_part = [&](int q, int r0, int c0, double (&pv)[16], double (&qv)[16],
                       f64x4 (&cv)[2][2]) {
    const int i = i0 + 4 * q;
    pv[q] = A[(int64_t)min(r0 + i, d - 1) * lda + k + j];
    qv[q] = A[(int64_t)min(c0 + i, d - 1) * lda + k + j];
    const int a = q >> 3, b = (q >> 2) & 1, e = q & 3;
    const int r = r0 + 32 * wm + 16 * a + mfma64_row(lane, e);
    const int c = c0 + 32 * wn + 16 * b + (lane & 15);
    cv[a][b][e] = A[(int64_t)min(r, d - 1) * lda + min(c, d - 1)];
  };
  auto load = [&](int r0, int c0, double (&pv)[16], double (&qv)[16], f64x4 (&cv)[2][2]) {
#pragma unroll
    for (int q = 0; q < 16; ++q) load_part(q, r0, c0, pv, qv, cv);
  };
  auto stage = [&](const double (&pv)[16], const double (&qv)[16]) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      Ps[i0 + 4 * q][j] = pv[q];
      Qs[i0 + 4 * q][j] = qv[q];
    }
  };
  double pv[16], qv[16];
  f64x4 cv[2][2], acc[2][2];
  int r0, c0;
  bool diag = coords(blockIdx.x, r0, c0);
  load(r0, c0, pv, qv, cv);
  stage(pv, qv);
  __syncthreads();
  {
    const int stride = (int)gridDim.x - 1;
    // One tile: multiply from LDS while issuing the next tile's loads (its C
    // tile into cvn), three per k-step, so the products run while the memory
    // system takes the loads (issued up front, the loads stalled the wave
    // until the previous tile's traffic drained, and the products waited
    // behind them); then write this tile and stage the next panel blocks.
    // The next k-step's operands are read from LDS while this one's products
    // run.  The two C register sets alternate (loop unrolled by two), so no
    // wait covers the stores just issued.
    f64x4 cv2[2][2];
    int p = blockIdx.x;
    auto step = [&](const f64x4 (&cvc)[2][2], f64x4 (&cvn)[2][2]) {
      const int pn = p + stride;
      const bool more = pn < ntiles;
      // the last step re-reads its own tile, so every step issues the same
      // loads and the outstanding-load count stays exact
      int r0n, c0n;
      const bool diagn = coords(more ? pn : p, r0n, c0n);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};
      const double (*Qt)[PP] = diag ? Ps : Qs;
      double af[2], bf[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) af[a] = Ps[32 * wm + 16 * a + (lane & 15)][lane >> 4];
#pragma unroll
      for (int b = 0; b < 2; ++b) bf[b] = Qt[32 * wn + 16 * b + (lane & 15)][lane >> 4];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        load_part(q, r0n, c0n, pv, qv, cvn);
        const int kn = 4 * ((q + 1) & 15) + (lane >> 4);
        double afn[2], bfn[2];
#pragma unroll
        for (int a = 0; a < 2; ++a) afn[a] = Ps[32 * wm + 16 * a + (lane & 15)][kn];
#pragma unroll
        for (int b = 0; b < 2; ++b) bfn[b] = Qt[32 * wn + 16 * b + (lane & 15)][kn];
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(af[a], bf[b], acc[a][b], 0, 0, 0);
        // keep this order: three global loads, four LDS reads, four products
        __builtin_amdgcn_sched_group_barrier(0x0020, 3, 0);
        __builtin_amdgcn_sched_group_barrier(0x0100, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x0008, 4, 0);
#pragma unroll
        for (int a = 0; a < 2; ++a) af[a] = afn[a];
#pragma unroll
        for (int b = 0; b < 2; ++b) bf[b] = bfn[b];
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = r0 + 32 * wm + 16 * a + mfma64_row(lane, i);
            const int c = c0 + 32 * wn + 16 * b + (lane & 15);
            if (r < d && c < d) A[(int64_t)r * lda + c] = cvc[a][b][i] - acc[a][b][i];
          }
      if (!more) return false;
      __syncthreads();  // every wave is done reading the panel tiles
      stage(pv, qv);
      __syncthreads();
      r0 = r0n;
      c0 = c0n;
      diag = diagn;
      p = pn;
      return true;
    };
    while (step(cv, cv2) && step(cv2, cv)) {
    }
  }
}

// One whole panel step for a small trailing matrix: the panel solve and the
// rank-64 update in one launch, one lower 64x64 tile of A[t0:, t0:] per
// workgroup (t0 = k + 64, nt block rows).  Each workgroup forms the two
// panel blocks it needs, L(i, k) = A(i, k) X_kk^T and L(j, k), from the raw
// panel and X_kk itself (the triangular product of panel_times_xt, the same
// values the separate solve stores), then applies A_ij -= L(i, k) L(j, k)^T.
// The raw panel stays in place while other workgroups read it, so L(i, k) is
// written to the free block Lp(i, k) of the inverted-diagonal workspace (by
// the workgroup of tile (i, t0)) and copied into A after the factorization.
// Workgroup 0 does the lookahead of potrf_update_kernel.  With the solve
// launch gone, each late step of the serial panel chain is one launch.
__global__ __launch_bounds__(256, 2) void potrf_fused_kernel(double* __restrict__ A, int lda, int d,
                                                          int k, int nt, double* __restrict__ Xi,
                                                          int ldxi, int* flag, int info_offset) {
  __shared__ DiagLds sh;
  const int t0 = k + NB;
  const double* Xk = Xi + (int64_t)k * ldxi + k;
  double* Lp = Xi + k;  // Lp(i, k) at row i of column block k of the workspace
  if (blockIdx.x == 0) {
    lookahead_diag<true>(sh, A, lda, d, k, Xk, Lp + (int64_t)t0 * ldxi, ldxi, flag, info_offset,
                         Xi + (int64_t)t0 * ldxi + t0, ldxi);
    return;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int j = tid & 63, i0 = tid >> 6;
  int r0, c0;
  const bool diag = tile_coords(blockIdx.x, nt, t0, r0, c0);
  // every load up front; rows past the matrix are clamped and reach only
  // elements that are never stored
  double pa[16], qa[16], xv[16];
  f64x4 cv[2][2];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int i = i0 + 4 * q;
    pa[q] = A[(int64_t)min(r0 + i, d - 1) * lda + k + j];
    qa[q] = A[(int64_t)min(c0 + i, d - 1) * lda + k + j];
    xv[q] = Xk[(int64_t)i * ldxi + j];
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + 32 * wm + 16 * a + mfma64_row(lane, i);
        const int c = c0 + 32 * wn + 16 * b + (lane & 15);
        cv[a][b][i] = A[(int64_t)min(r, d - 1) * lda + min(c, d - 1)];
      }
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    sh.S[i0 + 4 * q][j] = pa[q];
    sh.Xs[i0 + 4 * q][j] = xv[q];
  }
  __syncthreads();
  f64x4 oP[4], oQ[4];
  panel_times_xt(sh.S, sh.Xs, oP, lane, wave);
  if (!diag) {
    __syncthreads();  // every wave is done with the raw row block
#pragma unroll
    for (int q = 0; q < 16; ++q) sh.S[i0 + 4 * q][j] = qa[q];
    __syncthreads();
    panel_times_xt(sh.S, sh.Xs, oQ, lane, wave);
  }
  if (c0 == t0) {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = strip_row(wave, lane, i), c = strip_col(cb, lane);
        if (r0 + r < d) Lp[(int64_t)(r0 + r) * ldxi + c] = oP[cb][i];
      }
  }
  __syncthreads();  // every wave is done with the raw blocks and X_kk
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = strip_row(wave, lane, i), c = strip_col(cb, lane);
      sh.S[r][c] = oP[cb][i];
      if (!diag) sh.Xs[r][c] = oQ[cb][i];
    }
  __syncthreads();
  f64x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};
  mma64_f64(sh.S, diag ? sh.S : sh.Xs, NB, acc, lane, wm, wn);
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + 32 * wm + 16 * a + mfma64_row(lane, i);
        const int c = c0 + 32 * wn + 16 * b + (lane & 15);
        if (r < d && c < d) A[(int64_t)r * lda + c] = cv[a][b][i] - acc[a][b][i];
      }
}

// Panels k0, k0 + 64, ... that went through potrf_fused_kernel: their blocks
// below the diagonal move from the workspace into A.  Workgroup (x, y) copies
// block row k + 64 (x + 1) of panel k = k0 + 64 y.
__global__ __launch_bounds__(256) void copy_panels_kernel(double* __restrict__ A, int lda, int d,
                                                          int k0, const double* __restrict__ Xi,
                                                          int ldxi) {
  const int k = k0 + NB * (int)blockIdx.y;
  const int r0 = k + NB * ((int)blockIdx.x + 1);
  if (r0 >= d) return;
  const int rb = min(NB, d - r0);
  const int j = threadIdx.x & 63, i0 = threadIdx.x >> 6;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int i = i0 + 4 * q;
    if (i < rb) A[(int64_t)(r0 + i) * lda + k + j] = Xi[(int64_t)(r0 + i) * ldxi + k + j];
  }
}

// -------------------------------------------------------------- MFMA GEMM
// C = beta*C + alpha * sum_{k in range(tile)} opA(m,k) opB(k,n) on 64x64 tiles.
struct GemmDesc {
  const double* A;
  const double* B;
  double* C;
  int64_t lda, ldb, ldc;
  int M, N, K;
  double alpha, beta;
  int tri;    // 1: only tiles with tm >= tn (square C)
  int kmode;  // K range of a tile: 0 all; 1 k >= n0; 2 k < m0 + tile; 3 k >= m0
  int trA;    // 1: opA(m,k) = 0 for k > m; 2: opA(m,k) = 0 for k < m
  int trB;    // 1: opB(k,n) = 0 for k < n; 2: opB(k,n) = 0 for k > n
  int64_t bsa, bsb, bsc;  // per-batch (blockIdx.y) element offsets
};

// v where c holds, else +0.0, as a select on the bits (no branch).
__device__ inline double keep_if(bool c, double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  return __builtin_bit_cast(double, c ? u : (uint64_t)0);
}

// Zero an operand element outside its triangle (the K-range of a tile is
// only tile-aligned, so a triangular operand's other half may be read):
// tr 1 keeps row >= col, tr 2 keeps row <= col.
__device__ inline double tri_mask(double v, int tr, int row, int col) {
  const bool zero = (tr == 1 && col > row) || (tr == 2 && col < row);
  return keep_if(!zero, v);
}

// Tile of a GEMM launch for workgroup `p`.  When the K range depends on the
// tile (triangular operands), tiles are taken longest first, snaking over
// groups of 256 workgroups (one per CU), so the tiles a CU holds at the
// same time have mixed lengths.
__device__ inline void gemm_tile(int p, int ntiles, int ntm, int ntn, int tri, int kmode, int& tm,
                                 int& tn) {
  int r = p;
  if (kmode != 0) {
    const int g = p >> 8, i = p & 255;
    const int gsize = min(256, ntiles - (g << 8));
    r = (g << 8) + ((g & 1) ? gsize - 1 - i : i);
  }
  if (tri) {
    lower_tile(r, tm, tn);  // tm ascending: longest first for kmode 3
  } else if (kmode == 1) {  // length K - n0: columns first
    tn = r / ntm;
    tm = r % ntm;
  } else if (kmode == 2) {  // length m0 + tile: last rows first
    tm = ntm - 1 - r / ntn;
    tn = r % ntn;
  } else {
    tm = r / ntn;
    tn = r % ntn;
  }
}

// AK: A element (m,k) at A[m*lda+k] (else A[k*lda+m]).
// BN: B element (k,n) at B[k*ldb+n] (else B[n*ldb+k]).
// CN: C element (m,n) at C[m*ldc+n] (else C[n*ldc+m]).
// K is streamed in chunks of GK through double-buffered LDS tiles; the next
// chunk's global loads are issued before the current chunk's MFMAs.
template <bool AK, bool BN, bool CN>
__global__ __launch_bounds__(256) void gemm64_f64_kernel(GemmDesc g) {
  // LDS layout per operand follows its contiguous global dimension, so the
  // stores are conflict-free: k-contiguous operands are kept row-major
  // ([m][k], pitch GK + 1), m-contiguous ones k-major ([k][m], pitch 80).
  constexpr int PK = GT + 16;
  constexpr int PR = GK + 1;
  constexpr int SA = AK ? GT * PR : GK * PK;
  constexpr int SB = BN ? GK * PK : GT * PR;
  __shared__ double As[2][SA];
  __shared__ double Bs[2][SB];
  auto a_at = [&](int buf, int m, int k) -> double& {
    return AK ? As[buf][m * PR + k] : As[buf][k * PK + m];
  };
  auto b_at = [&](int buf, int k, int n) -> double& {
    return BN ? Bs[buf][k * PK + n] : Bs[buf][n * PR + k];
  };
  int tm, tn;
  const int ntm = (int)ceil_div(g.M, GT), ntn = (int)ceil_div(g.N, GT);
  gemm_tile(blockIdx.x, gridDim.x, ntm, ntn, g.tri, g.kmode, tm, tn);
  const double* Ap = g.A + (int64_t)blockIdx.y * g.bsa;
  const double* Bp = g.B + (int64_t)blockIdx.y * g.bsb;
  double* Cp = g.C + (int64_t)blockIdx.y * g.bsc;
  const int m0 = tm * GT, n0 = tn * GT;
  int k0 = 0, k1 = g.K;
  if (g.kmode == 1) k0 = n0;
  else if (g.kmode == 2) k1 = min(g.K, m0 + GT);
  else if (g.kmode == 3) k0 = m0;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  f64x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};

  // Loads: a uniform base per chunk plus a 32-bit per-thread byte offset
  // (global_load with a scalar base).  The offsets are computed once, with the
  // row clamped into the operand; only the last chunk clamps k to its valid
  // range, so every address is inside the operand (the bounds and triangle
  // masks are applied at the LDS store, and skipped for chunks that need
  // none), and the MFMAs of the current chunk never wait for these loads.
  // Offsets stay below 2^31 for leading dimensions up to 65536.
  constexpr int NLD = GT * GK / 256;
  double av[NLD], bv[NLD];
  uint32_t aoff[NLD], boff[NLD];
  const uint32_t lda8 = (uint32_t)g.lda * 8u, ldb8 = (uint32_t)g.ldb * 8u;
  const uint32_t ska = AK ? 8u : lda8, skb = BN ? ldb8 : 8u;  // byte stride of one k
#pragma unroll
  for (int q = 0; q < NLD; ++q) {
    const int e = tid + 256 * q;
    const int kk = AK ? (e % GK) : (e / GT);
    const int mm = min(AK ? (e / GK) : (e % GT), g.M - 1 - m0);
    aoff[q] = (AK ? (uint32_t)mm * lda8 : (uint32_t)mm * 8u) + (uint32_t)kk * ska;
    const int kb = BN ? (e / GT) : (e % GK);
    const int nn = min(BN ? (e % GT) : (e / GK), g.N - 1 - n0);
    boff[q] = (BN ? (uint32_t)nn * 8u : (uint32_t)nn * ldb8) + (uint32_t)kb * skb;
  }
  auto gload = [&](int kc) {
    const char* abase = reinterpret_cast<const char*>(
        Ap + (AK ? (int64_t)m0 * g.lda + kc : (int64_t)kc * g.lda + m0));
    const char* bbase = reinterpret_cast<const char*>(
        Bp + (BN ? (int64_t)kc * g.ldb + n0 : (int64_t)n0 * g.ldb + kc));
    if (kc + GK <= k1) {  // whole chunk: the fixed offsets
#pragma unroll
      for (int q = 0; q < NLD; ++q) {
        av[q] = *reinterpret_cast<const double*>(abase + aoff[q]);
        bv[q] = *reinterpret_cast<const double*>(bbase + boff[q]);
      }
      return;
    }
    const int lim = k1 - 1 - kc;  // last chunk: k clamped to lim
#pragma unroll
    for (int q = 0; q < NLD; ++q) {
      const int e = tid + 256 * q;
      const int kk = AK ? (e % GK) : (e / GT);
      const int kb = BN ? (e / GT) : (e % GK);
      const uint32_t oa = aoff[q] - (uint32_t)(kk - min(kk, lim)) * ska;
      const uint32_t ob = boff[q] - (uint32_t)(kb - min(kb, lim)) * skb;
      av[q] = *reinterpret_cast<const double*>(abase + oa);
      bv[q] = *reinterpret_cast<const double*>(bbase + ob);
    }
  };
  auto lstore = [&](int buf, int kc) {
    // uniform: every element of the chunk in bounds and inside both triangles
    const bool in_k = kc + GK <= k1;
    const bool full_a = in_k && m0 + GT <= g.M &&
                        (g.trA == 0 || (g.trA == 1 && m0 >= kc + GK - 1) ||
                         (g.trA == 2 && m0 + GT - 1 <= kc));
    const bool full_b = in_k && n0 + GT <= g.N &&
                        (g.trB == 0 || (g.trB == 1 && kc >= n0 + GT - 1) ||
                         (g.trB == 2 && kc + GK - 1 <= n0));
    if (full_a && full_b) {
#pragma unroll
      for (int q = 0; q < NLD; ++q) {
        const int e = tid + 256 * q;
        a_at(buf, AK ? (e / GK) : (e % GT), AK ? (e % GK) : (e / GT)) = av[q];
        b_at(buf, BN ? (e / GT) : (e % GK), BN ? (e % GT) : (e / GK)) = bv[q];
      }
      return;
    }
#pragma unroll
    for (int q = 0; q < NLD; ++q) {
      const int e = tid + 256 * q;
      const int kk = AK ? (e % GK) : (e / GT);
      const int mm = AK ? (e / GK) : (e % GT);
      const int gm = m0 + mm, gk = kc + kk;
      const bool va = gm < g.M && gk < k1;
      a_at(buf, mm, kk) = keep_if(va, tri_mask(av[q], g.trA, gm, gk));
      const int kb = BN ? (e / GT) : (e % GK);
      const int nn = BN ? (e % GT) : (e / GK);
      const int gn = n0 + nn, gk2 = kc + kb;
      const bool vb = gn < g.N && gk2 < k1;
      b_at(buf, kb, nn) = keep_if(vb, tri_mask(bv[q], g.trB, gk2, gn));
    }
  };
  if (k0 < k1) {
    gload(k0);
    lstore(0, k0);
    __syncthreads();
  }
  int buf = 0;
  for (int kc = k0; kc < k1; kc += GK) {
    const bool more = kc + GK < k1;
    if (more) gload(kc + GK);
    // every k-step's operands of the chunk first, then the products (held in
    // that order by scheduling barriers), so only the first k-step waits for
    // its LDS reads; read per k-step, each k-step waited for its own
    constexpr int NS = GK / 4;
    double af[NS][2], bf[NS][2];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int kr = 4 * s + (lane >> 4);
#pragma unroll
      for (int a = 0; a < 2; ++a) af[s][a] = a_at(buf, 32 * wm + 16 * a + (lane & 15), kr);
#pragma unroll
      for (int b = 0; b < 2; ++b) bf[s][b] = b_at(buf, kr, 32 * wn + 16 * b + (lane & 15));
    }
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(af[s][a], bf[s][b], acc[a][b], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x0100, 4 * NS, 0);
    __builtin_amdgcn_sched_group_barrier(0x0008, 4 * NS, 0);
    if (more) lstore(buf ^ 1, kc + GK);
    __syncthreads();
    buf ^= 1;
  }
  // epilogue: all C loads before the stores
  double cold[2][2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = min(m0 + 32 * wm + 16 * a + mfma64_row(lane, i), g.M - 1);
        const int n = min(n0 + 32 * wn + 16 * b + (lane & 15), g.N - 1);
        cold[a][b][i] = (g.beta == 0.0) ? 0.0
                        : (CN ? Cp[(int64_t)m * g.ldc + n] : Cp[(int64_t)n * g.ldc + m]);
      }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + 32 * wm + 16 * a + mfma64_row(lane, i);
        const int n = n0 + 32 * wn + 16 * b + (lane & 15);
        if (m < g.M && n < g.N) {
          double* c = CN ? Cp + (int64_t)m * g.ldc + n : Cp + (int64_t)n * g.ldc + m;
          const double v = g.alpha * acc[a][b][i];
          *c = (g.beta == 0.0) ? v : __builtin_fma(g.beta, cold[a][b][i], v);
        }
      }
}

template <bool AK, bool BN, bool CN>
hipError_t gemm64(const GemmDesc& g, int batches, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || batches <= 0) return hipSuccess;
  const int64_t tm = ceil_div(g.M, GT), tn = ceil_div(g.N, GT);
  const int64_t tiles = g.tri ? tm * (tm + 1) / 2 : tm * tn;
  hipLaunchKernelGGL((gemm64_f64_kernel<AK, BN, CN>), dim3((unsigned)tiles, batches), dim3(256), 0,
                     s, g);
  return hipGetLastError();
}


// The same product on 128x128 tiles: each wave owns a 64x64 quadrant (4x4
// MFMA tiles), twice the arithmetic per loaded element of the 64x64 kernel,
// which keeps large products on fp64 MFMA rather than on L2 bandwidth.
constexpr int GT2 = 128;
template <bool AK, bool BN, bool CN>
__global__ __launch_bounds__(256, 2) void gemm128_f64_kernel(GemmDesc g) {
  // LDS layout per operand follows its contiguous global dimension, so the
  // stores are conflict-free: k-contiguous operands are kept row-major
  // ([m][k], pitch GK + 1), m-contiguous ones k-major ([k][m], pitch 144).
  constexpr int PK = GT2 + 16;
  constexpr int PR = GK + 1;
  constexpr int SA = AK ? GT2 * PR : GK * PK;  // doubles per buffer
  constexpr int SB = BN ? GK * PK : GT2 * PR;
  __shared__ double As[2][SA];
  __shared__ double Bs[2][SB];
  auto a_at = [&](int buf, int m, int k) -> double& {
    return AK ? As[buf][m * PR + k] : As[buf][k * PK + m];
  };
  auto b_at = [&](int buf, int k, int n) -> double& {
    return BN ? Bs[buf][k * PK + n] : Bs[buf][n * PR + k];
  };
  int tm, tn;
  const int ntm = (int)ceil_div(g.M, GT2), ntn = (int)ceil_div(g.N, GT2);
  gemm_tile(blockIdx.x, gridDim.x, ntm, ntn, g.tri, g.kmode, tm, tn);
  const double* Ap = g.A + (int64_t)blockIdx.y * g.bsa;
  const double* Bp = g.B + (int64_t)blockIdx.y * g.bsb;
  double* Cp = g.C + (int64_t)blockIdx.y * g.bsc;
  const int m0 = tm * GT2, n0 = tn * GT2;
  int k0 = 0, k1 = g.K;
  if (g.kmode == 1) k0 = n0;
  else if (g.kmode == 2) k1 = min(g.K, m0 + GT2);
  else if (g.kmode == 3) k0 = m0;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  f64x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};

  // Loads: a uniform base per chunk plus a 32-bit per-thread byte offset
  // (global_load with a scalar base).  The offsets are computed once, with the
  // row clamped into the operand; only the last chunk clamps k to its valid
  // range, so every address is inside the operand (the bounds and triangle
  // masks are applied at the LDS store, and skipped for chunks that need
  // none), and the MFMAs of the current chunk never wait for these loads.
  // Offsets stay below 2^31 for leading dimensions up to 65536.
  constexpr int NLD = GT2 * GK / 256;
  double av[NLD], bv[NLD];
  uint32_t aoff[NLD], boff[NLD];
  const uint32_t lda8 = (uint32_t)g.lda * 8u, ldb8 = (uint32_t)g.ldb * 8u;
  const uint32_t ska = AK ? 8u : lda8, skb = BN ? ldb8 : 8u;  // byte stride of one k
#pragma unroll
  for (int q = 0; q < NLD; ++q) {
    const int e = tid + 256 * q;
    const int kk = AK ? (e % GK) : (e / GT2);
    const int mm = min(AK ? (e / GK) : (e % GT2), g.M - 1 - m0);
    aoff[q] = (AK ? (uint32_t)mm * lda8 : (uint32_t)mm * 8u) + (uint32_t)kk * ska;
    const int kb = BN ? (e / GT2) : (e % GK);
    const int nn = min(BN ? (e % GT2) : (e / GK), g.N - 1 - n0);
    boff[q] = (BN ? (uint32_t)nn * 8u : (uint32_t)nn * ldb8) + (uint32_t)kb * skb;
  }
  auto gload = [&](int kc) {
    const char* abase = reinterpret_cast<const char*>(
        Ap + (AK ? (int64_t)m0 * g.lda + kc : (int64_t)kc * g.lda + m0));
    const char* bbase = reinterpret_cast<const char*>(
        Bp + (BN ? (int64_t)kc * g.ldb + n0 : (int64_t)n0 * g.ldb + kc));
    if (kc + GK <= k1) {  // whole chunk: the fixed offsets
#pragma unroll
      for (int q = 0; q < NLD; ++q) {
        av[q] = *reinterpret_cast<const double*>(abase + aoff[q]);
        bv[q] = *reinterpret_cast<const double*>(bbase + boff[q]);
      }
      return;
    }
    const int lim = k1 - 1 - kc;  // last chunk: k clamped to lim
#pragma unroll
    for (int q = 0; q < NLD; ++q) {
      const int e = tid + 256 * q;
      const int kk = AK ? (e % GK) : (e / GT2);
      const int kb = BN ? (e / GT2) : (e % GK);
      const uint32_t oa = aoff[q] - (uint32_t)(kk - min(kk, lim)) * ska;
      const uint32_t ob = boff[q] - (uint32_t)(kb - min(kb, lim)) * skb;
      av[q] = *reinterpret_cast<const double*>(abase + oa);
      bv[q] = *reinterpret_cast<const double*>(bbase + ob);
    }
  };
  auto lstore = [&](int buf, int kc) {
    // uniform: every element of the chunk in bounds and inside both triangles
    const bool in_k = kc + GK <= k1;
    const bool full_a = in_k && m0 + GT2 <= g.M &&
                        (g.trA == 0 || (g.trA == 1 && m0 >= kc + GK - 1) ||
                         (g.trA == 2 && m0 + GT2 - 1 <= kc));
    const bool full_b = in_k && n0 + GT2 <= g.N &&
                        (g.trB == 0 || (g.trB == 1 && kc >= n0 + GT2 - 1) ||
                         (g.trB == 2 && kc + GK - 1 <= n0));
    if (full_a && full_b) {
#pragma unroll
      for (int q = 0; q < NLD; ++q) {
        const int e = tid + 256 * q;
        a_at(buf, AK ? (e / GK) : (e % GT2), AK ? (e % GK) : (e / GT2)) = av[q];
        b_at(buf, BN ? (e / GT2) : (e % GK), BN ? (e % GT2) : (e / GK)) = bv[q];
      }
      return;
    }
#pragma unroll
    for (int q = 0; q < NLD; ++q) {
      const int e = tid + 256 * q;
      const int kk = AK ? (e % GK) : (e / GT2);
      const int mm = AK ? (e / GK) : (e % GT2);
      const int gm = m0 + mm, gk = kc + kk;
      const bool va = gm < g.M && gk < k1;
      a_at(buf, mm, kk) = keep_if(va, tri_mask(av[q], g.trA, gm, gk));
      const int kb = BN ? (e / GT2) : (e % GK);
      const int nn = BN ? (e % GT2) : (e / GK);
      const int gn = n0 + nn, gk2 = kc + kb;
      const bool vb = gn < g.N && gk2 < k1;
      b_at(buf, kb, nn) = keep_if(vb, tri_mask(bv[q], g.trB, gk2, gn));
    }
  };
  if (k0 < k1) {
    gload(k0);
    lstore(0, k0);
    __syncthreads();
  }
  int buf = 0;
  for (int kc = k0; kc < k1; kc += GK) {
    const bool more = kc + GK < k1;
    if (more) gload(kc + GK);
#pragma unroll
    for (int ks = 0; ks < GK; ks += 4) {
      const int kr = ks + (lane >> 4);
      double af[4], bf[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) af[a] = a_at(buf, 64 * wm + 16 * a + (lane & 15), kr);
#pragma unroll
      for (int b = 0; b < 4; ++b) bf[b] = b_at(buf, kr, 64 * wn + 16 * b + (lane & 15));
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(af[a], bf[b], acc[a][b], 0, 0, 0);
    }
    if (more) lstore(buf ^ 1, kc + GK);
    __syncthreads();
    buf ^= 1;
  }
  // epilogue: per row block, all C loads go out before any store
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    double cold[4][4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = min(m0 + 64 * wm + 16 * a + mfma64_row(lane, i), g.M - 1);
        const int n = min(n0 + 64 * wn + 16 * b + (lane & 15), g.N - 1);
        cold[b][i] = (g.beta == 0.0) ? 0.0
                     : (CN ? Cp[(int64_t)m * g.ldc + n] : Cp[(int64_t)n * g.ldc + m]);
      }
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + 64 * wm + 16 * a + mfma64_row(lane, i);
        const int n = n0 + 64 * wn + 16 * b + (lane & 15);
        if (m < g.M && n < g.N) {
          double* c = CN ? Cp + (int64_t)m * g.ldc + n : Cp + (int64_t)n * g.ldc + m;
          const double v = g.alpha * acc[a][b][i];
          *c = (g.beta == 0.0) ? v : __builtin_fma(g.beta, cold[b][i], v);
        }
      }
  }
}

// Products take the 64x64 kernel unless they have a very large number of
// 128x128 tiles: with conflict-free LDS both kernels reach about 51 TF/s on
// a dense 4096^3 product, and the finer tiles balance triangular K ranges
// and small updates better.
template <bool AK, bool BN, bool CN>
hipError_t gemm_f64(const GemmDesc& g, int batches, hipStream_t s, int64_t min_big_tiles = 4096) {
  if (g.M <= 0 || g.N <= 0 || batches <= 0) return hipSuccess;
  const int64_t tm = ceil_div(g.M, GT2), tn = ceil_div(g.N, GT2);
  const int64_t tiles = (g.tri ? tm * (tm + 1) / 2 : tm * tn) * batches;
  const bool big = g.M > GT && g.N > GT && tiles >= min_big_tiles;
  if (!big) return gemm64<AK, BN, CN>(g, batches, s);
  hipLaunchKernelGGL((gemm128_f64_kernel<AK, BN, CN>), dim3((unsigned)(tiles / batches), batches),
                     dim3(256), 0, s, g);
  return hipGetLastError();
}

// -------------------------------------------------------------- fp32 output
// Hinv[i][j] = L2[j][i] for j >= i, 0 below the diagonal.
__global__ __launch_bounds__(256) void store_upper_kernel(const double* __restrict__ L2, int ld2,
                                                          float* __restrict__ Hinv, int d) {
  __shared__ double t[64][65];
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;  // output tile rows i0.., cols j0..
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  if (j0 + 63 < i0) {  // tile strictly below the diagonal
    for (int r = ty; r < 64; r += 4)
      if (i0 + r < d && j0 + tx < d) Hinv[(int64_t)(i0 + r) * d + j0 + tx] = 0.f;
    return;
  }
  // load L2[j0 + r][i0 + tx] (rows of L2 = columns of Hinv)
  for (int r = ty; r < 64; r += 4) {
    const int jr = j0 + r, ic = i0 + tx;
    t[r][tx] = (jr < d && ic < d && ic <= jr) ? L2[(int64_t)jr * ld2 + ic] : 0.0;
  }
  __syncthreads();
  for (int r = ty; r < 64; r += 4) {
    const int i = i0 + r, j = j0 + tx;
    if (i < d && j < d) Hinv[(int64_t)i * d + j] = (j >= i) ? (float)t[tx][r] : 0.f;
  }
}

// Hinv[i][j] = X[d-1-i][d-1-j] for j >= i (row d-1-i of the lower
// triangular X, read backwards), 0 below the diagonal.  One workgroup per row.
__global__ __launch_bounds__(256) void store_reversed_kernel(const double* __restrict__ X, int ldx,
                                                             float* __restrict__ Hinv, int d) {
  const int i = blockIdx.x;
  const double* xrow = X + (int64_t)(d - 1 - i) * ldx + (d - 1);
  float* hrow = Hinv + (int64_t)i * d;
  for (int j = threadIdx.x; j < d; j += 256) hrow[j] = (j >= i) ? (float)xrow[-j] : 0.f;
}

// Compute units of the current device (cached per device id; concurrent
// callers may both query and store the same value).
int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace

hipError_t launch_damp_to_f64(const float* H, int d, double percdamp, const int* perm, bool reverse,
                              double* A, int* flag, hipStream_t s) {
  double* lam = reinterpret_cast<double*>(reinterpret_cast<char*>(flag) + 8);
  hipLaunchKernelGGL(damp_lambda_kernel, dim3(1), dim3(256), 0, s, H, d, percdamp, lam, flag);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (perm != nullptr) {
    const bool stage = (int64_t)d * 4 <= kStageBytes;
    hipLaunchKernelGGL(damp_copy_perm_kernel, dim3((unsigned)d), dim3(256),
                       stage ? (unsigned)d * 4u : 0u, s, H, d, perm, (const double*)lam, A,
                       stage, reverse);
  } else if (reverse) {
    const int64_t nt = ceil_div(d, 64);
    hipLaunchKernelGGL(damp_copy_rev_kernel, dim3((unsigned)(nt * (nt + 1) / 2)), dim3(256), 0, s,
                       H, d, (const double*)lam, A);
  } else
    hipLaunchKernelGGL(damp_copy_kernel, dim3((unsigned)d), dim3(256), 0, s, H, d,
                       (const double*)lam, A);
  return hipGetLastError();
}

hipError_t launch_potrf_diag(double* A, int lda, int d, int k, int* flag, int info_offset,
                             double* Xi, int ldxi, hipStream_t s) {
  double* Xd = Xi + (int64_t)k * ldxi + k;
  hipLaunchKernelGGL(potrf_diag_kernel, dim3(1), dim3(256), 0, s, A, lda, d, k, flag, info_offset,
                     Xd, ldxi);
  return hipGetLastError();
}

hipError_t launch_potrf_trsm(double* A, int lda, int d, int k, const double* Xi, int ldxi,
                             hipStream_t s) {
  const int nbelow = (int)ceil_div(d - k, NB) - 1;
  if (nbelow <= 0) return hipSuccess;
  hipLaunchKernelGGL(potrf_trsm_kernel, dim3(nbelow), dim3(256), 0, s, A, lda, d, k,
                     Xi + (int64_t)k * ldxi + k, ldxi);
  return hipGetLastError();
}

hipError_t launch_potrf_update(double* A, int lda, int d, int k, int ncol, int* flag,
                               int info_offset, double* Xi, int ldxi, hipStream_t s) {
  const int64_t nt = ceil_div(d - k - NB, NB);
  if (nt <= 0 || ncol <= 0) return hipSuccess;
  const int64_t nc = ncol < nt ? ncol : nt;
  const int64_t tiles = nc * nt - nc * (nc - 1) / 2;
  // two resident workgroups per CU (the LDS of the diagonal factorization)
  const int64_t cap = 2 * (int64_t)device_cus();
  const int64_t grid = tiles < cap ? tiles : cap;
  const int kn = k + NB;
  hipLaunchKernelGGL(potrf_update_kernel, dim3((unsigned)grid), dim3(256), 0, s, A, lda, d, k,
                     (int)nt, (int)tiles, flag, info_offset, Xi + (int64_t)kn * ldxi + kn, ldxi);
  return hipGetLastError();
}

hipError_t launch_potrf_fused(double* A, int lda, int d, int k, int* flag, int info_offset,
                              double* Xi, int ldxi, hipStream_t s) {
  const int64_t nt = ceil_div(d - k - NB, NB);
  if (nt <= 0) return hipSuccess;
  const int64_t tiles = nt * (nt + 1) / 2;
  hipLaunchKernelGGL(potrf_fused_kernel, dim3((unsigned)tiles), dim3(256), 0, s, A, lda, d, k,
                     (int)nt, Xi, ldxi, flag, info_offset);
  return hipGetLastError();
}

hipError_t launch_copy_panels(double* A, int lda, int d, int k0, const double* Xi, int ldxi,
                              hipStream_t s) {
  const int64_t below = ceil_div(d - k0, NB) - 1;  // block rows below panel k0 = panels to copy
  if (below <= 0) return hipSuccess;
  hipLaunchKernelGGL(copy_panels_kernel, dim3((unsigned)below, (unsigned)below), dim3(256), 0, s, A,
                     lda, d, k0, Xi, ldxi);
  return hipGetLastError();
}

// A[k1:, k1:] -= P P^T on the lower 128x128 tiles, P = A[k1:, k0:k1] (the
// panels of the finished outer block): one rank-(k1 - k0) update.
hipError_t launch_potrf_outer_update(double* A, int lda, int d, int k0, int k1, hipStream_t s) {
  if (k1 >= d || k1 <= k0) return hipSuccess;
  GemmDesc g{};
  g.A = A + (int64_t)k1 * lda + k0;
  g.B = A + (int64_t)k1 * lda + k0;  // element (k, n) = P[n][k]
  g.C = A + (int64_t)k1 * lda + k1;
  g.lda = lda; g.ldb = lda; g.ldc = lda;
  g.M = g.N = d - k1;
  g.K = k1 - k0;
  g.alpha = -1.0; g.beta = 1.0; g.tri = 1; g.kmode = 0;
  return gemm_f64<true, false, true>(g, 1, s);
}

// Combine pairs of inverted blocks of size `half`:
//   pair p: a0 = 2*half*p (inverted A), c0 = a0 + half (inverted C), B = L[c, a]
//   T  = B A^-1   stored transposed in the free upper block X[a, c]
//   X[c, a] = -C^-1 T
hipError_t launch_trtri_level(const double* L, int ldl, double* X, int ldx, int d, int half,
                              hipStream_t s) {
  const int full = d / (2 * half);               // pairs with a full C block
  const int rem_c = d - full * 2 * half - half;  // C size of a trailing partial pair
  for (int part = 0; part < 2; ++part) {
    const int batches = part == 0 ? full : (rem_c > 0 ? 1 : 0);
    if (batches == 0) continue;
    const int a0 = part == 0 ? 0 : full * 2 * half;
    const int c0 = a0 + half;
    const int sc = part == 0 ? half : rem_c;
    const int64_t bs = (int64_t)2 * half * (ldx + 1);
    GemmDesc g1{};
    g1.A = L + (int64_t)c0 * ldl + a0;  // B block, row-major
    g1.B = X + (int64_t)a0 * ldx + a0;  // A^-1, lower
    g1.C = X + (int64_t)a0 * ldx + c0;  // T^T location
    g1.lda = ldl; g1.ldb = ldx; g1.ldc = ldx;
    g1.M = sc; g1.N = half; g1.K = half;
    g1.alpha = 1.0; g1.beta = 0.0; g1.tri = 0; g1.kmode = 1;
    g1.trA = 0; g1.trB = 1;
    g1.bsa = (int64_t)2 * half * (ldl + 1); g1.bsb = bs; g1.bsc = bs;
    hipError_t e = gemm_f64<true, true, false>(g1, batches, s);
    if (e != hipSuccess) return e;
    GemmDesc g2{};
    g2.A = X + (int64_t)c0 * ldx + c0;  // C^-1, lower
    g2.B = X + (int64_t)a0 * ldx + c0;  // T (element (k=c, n=a) at T^T[a][c])
    g2.C = X + (int64_t)c0 * ldx + a0;
    g2.lda = ldx; g2.ldb = ldx; g2.ldc = ldx;
    g2.M = sc; g2.N = half; g2.K = sc;
    g2.alpha = -1.0; g2.beta = 0.0; g2.tri = 0; g2.kmode = 2;
    g2.trA = 1; g2.trB = 0;
    g2.bsa = bs; g2.bsb = bs; g2.bsc = bs;
    e = gemm_f64<true, false, true>(g2, batches, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_lauum(const double* X, int ldx, double* S, int lds, int d, hipStream_t s) {
  GemmDesc g{};
  g.A = X;  // element (m=i, k) = X[k][i]
  g.B = X;  // element (k, n=j) = X[k][j]
  g.C = S;
  g.lda = ldx; g.ldb = ldx; g.ldc = lds;
  g.M = g.N = g.K = d;
  g.alpha = 1.0; g.beta = 0.0; g.tri = 1; g.kmode = 3;
  g.trA = 2; g.trB = 1;
  // one large triangular product: from about d = 8192 on (2048 tiles of
  // 128x128) the coarser tiles win
  return gemm_f64<false, true, true>(g, 1, s, 2048);
}

hipError_t launch_store_upper_f32(const double* L2, int ld2, float* Hinv, int d, hipStream_t s) {
  const int nt = (int)ceil_div(d, 64);
  hipLaunchKernelGGL(store_upper_kernel, dim3(nt, nt), dim3(256), 0, s, L2, ld2, Hinv, d);
  return hipGetLastError();
}

hipError_t launch_store_reversed_f32(const double* X, int ldx, float* Hinv, int d, hipStream_t s) {
  hipLaunchKernelGGL(store_reversed_kernel, dim3((unsigned)d), dim3(256), 0, s, X, ldx, Hinv, d);
  return hipGetLastError();
}

}  // namespace gptq
