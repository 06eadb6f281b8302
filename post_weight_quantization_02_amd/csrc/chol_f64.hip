// Hinv preparation in fp64: damp, Cholesky, triangular inverse, L^-T L^-1,
// Cholesky again, and the fp32 upper factor.
//
// Route: "GPTQ, Line by Line: Hessian-Based Weight Quantization", percdamp
// question (add percdamp * mean(diag H) to the diagonal) and Cholesky
// question (factor, form the inverse through the factor, take the upper
// Cholesky factor of the inverse); the same three calls appear in the
// gptq_quantize_layer listing of "GPTQ-style round-to-nearest with Hessian
// weighting".
//
// gfx950 design:
//   * Everything runs in fp64: the sweep's integer decisions are sensitive
//     to the factor's accuracy, and fp32 factorizations of calibration
//     Hessians lose several digits.  fp64 MFMA (v_mfma_f64_16x16x4_f64)
//     carries every O(d^3) product; the O(nb^3) panel work runs in LDS.
//   * Blocked right-looking Cholesky with 64-wide panels: one workgroup
//     factors the panel's diagonal block in LDS, one workgroup per 64-row
//     block below solves against it, then one MFMA kernel applies the rank-64
//     update to the lower triangle of the trailing matrix.
//   * The triangular inverse uses recursive doubling: invert the 64x64
//     diagonal blocks, then at each level combine neighbouring inverted
//     blocks with X21 = -C^-1 (B A^-1), two batched MFMA launches per level.
//   * L^-T L^-1 is one MFMA launch over the lower tiles, each tile with its
//     own K range (the triangle of L^-1 makes the rest zero).
//   * A failed pivot (<= 0 or NaN) sets a device flag with atomicMin of its
//     1-based index; the host reads it once at the end.
#include <limits.h>

#include "common.h"

namespace gptq {

namespace {

constexpr int NB = kPanel;  // 64
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

// A = H + lambda I in fp64, both triangles taken from the lower triangle of H.
__global__ __launch_bounds__(256) void damp_copy_kernel(const float* __restrict__ H, int d,
                                                        const double* lam, double* __restrict__ A) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)d * d) return;
  const int i = (int)(e / d), j = (int)(e % d);
  const int r = i >= j ? i : j, c = i >= j ? j : i;
  double v = (double)H[(int64_t)r * d + c];
  if (i == j) v += *lam;
  A[e] = v;
}

// -------------------------------------------------------------- panel
// Factor the 64x64 diagonal block of the panel at column k in LDS and write
// L_kk over it (one workgroup).  Right-looking and unscaled: step j subtracts
// D[i][j] D[l][j] / D[j][j] from the trailing lower triangle; the column is
// scaled by 1/sqrt(D[j][j]) at the end.  One barrier per step.
__global__ __launch_bounds__(256) void potrf_diag_kernel(double* __restrict__ A, int lda, int d,
                                                         int k, int* flag, int info_offset) {
  __shared__ double D[NB][NB + 1];
  __shared__ double rinv[NB];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int kb = min(NB, d - k);
  for (int e = tid; e < NB * NB; e += 256) {
    const int i = e / NB, j = e % NB;
    double v = (i == j) ? 1.0 : 0.0;
    if (i < kb && j < kb && j <= i) v = A[(int64_t)(k + i) * lda + k + j];
    D[i][j] = v;
  }
  __syncthreads();
  for (int j = 0; j < kb; ++j) {
    const double djj = D[j][j];
    if (tid == 0 && !(djj > 0.0)) atomicMin(flag, info_offset + k + j + 1);
    const double inv = 1.0 / djj;
    for (int i = j + 1 + ty; i < kb; i += 16) {
      const double dij = D[i][j] * inv;
      for (int l = j + 1 + tx; l <= i; l += 16) D[i][l] -= dij * D[l][j];
    }
    __syncthreads();
  }
  if (tid < NB) rinv[tid] = (tid < kb) ? 1.0 / sqrt(D[tid][tid]) : 1.0;
  __syncthreads();
  for (int e = tid; e < NB * NB; e += 256) {
    const int i = e / NB, j = e % NB;
    if (i < kb && j <= i) A[(int64_t)(k + i) * lda + k + j] = D[i][j] * rinv[j];
  }
}

// Solve X L_kk^T = A[k+64(r+1).., k..k+63] for the row blocks below the
// diagonal block (one workgroup per 64-row block), right-looking over
// columns: B[:, m] -= (B[:, j] / L[j][j]) L[m][j].
__global__ __launch_bounds__(256) void potrf_trsm_kernel(double* __restrict__ A, int lda, int d,
                                                         int k) {
  __shared__ double Lk[NB][NB + 1];
  __shared__ double Bk[NB][NB + 1];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int kb = min(NB, d - k);
  const int row0 = k + NB * (blockIdx.x + 1);
  const int rb = min(NB, d - row0);
  for (int e = tid; e < NB * NB; e += 256) {
    const int i = e / NB, j = e % NB;
    double v = (i == j) ? 1.0 : 0.0;
    if (i < kb && j <= i) v = A[(int64_t)(k + i) * lda + k + j];
    Lk[i][j] = v;
    Bk[i][j] = (i < rb && j < kb) ? A[(int64_t)(row0 + i) * lda + k + j] : 0.0;
  }
  __syncthreads();
  for (int j = 0; j < kb; ++j) {
    const double ljj = 1.0 / Lk[j][j];
    for (int i = ty; i < rb; i += 16) {
      const double xij = Bk[i][j] * ljj;
      for (int m = j + 1 + tx; m < kb; m += 16) Bk[i][m] -= xij * Lk[m][j];
    }
    __syncthreads();
  }
  for (int e = tid; e < NB * NB; e += 256) {
    const int i = e / NB, j = e % NB;
    if (i < rb && j < kb) A[(int64_t)(row0 + i) * lda + k + j] = Bk[i][j] / Lk[j][j];
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
  int kmode;  // 0 all K; 1 k >= tn*GT; 2 k < (tm+1)*GT; 3 k >= tm*GT
  int64_t bsa, bsb, bsc;  // per-batch (blockIdx.y) element offsets
};

// AK: A element (m,k) at A[m*lda+k] (else A[k*lda+m]).
// BN: B element (k,n) at B[k*ldb+n] (else B[n*ldb+k]).
// CN: C element (m,n) at C[m*ldc+n] (else C[n*ldc+m]).
template <bool AK, bool BN, bool CN>
__global__ __launch_bounds__(256) void gemm64_f64_kernel(GemmDesc g) {
  __shared__ double As[GK][GT + 1];
  __shared__ double Bs[GK][GT + 1];
  int tm, tn;
  const int ntn = (int)ceil_div(g.N, GT);
  if (g.tri) {
    lower_tile(blockIdx.x, tm, tn);
  } else {
    tm = blockIdx.x / ntn;
    tn = blockIdx.x % ntn;
  }
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

  for (int kc = k0; kc < k1; kc += GK) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + 256 * q;
      int kk, mm;
      if (AK) { kk = e % GK; mm = e / GK; } else { mm = e % GT; kk = e / GT; }
      const int gm = m0 + mm, gk = kc + kk;
      double v = 0.0;
      if (gm < g.M && gk < k1) v = AK ? Ap[(int64_t)gm * g.lda + gk] : Ap[(int64_t)gk * g.lda + gm];
      As[kk][mm] = v;
      int nn;
      if (BN) { nn = e % GT; kk = e / GT; } else { kk = e % GK; nn = e / GK; }
      const int gn = n0 + nn;
      const int gk2 = kc + kk;
      double u = 0.0;
      if (gn < g.N && gk2 < k1) u = BN ? Bp[(int64_t)gk2 * g.ldb + gn] : Bp[(int64_t)gn * g.ldb + gk2];
      Bs[kk][nn] = u;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < GK; ks += 4) {
      const int kr = ks + (lane >> 4);
      double af[2], bf[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) af[a] = As[kr][32 * wm + 16 * a + (lane & 15)];
#pragma unroll
      for (int b = 0; b < 2; ++b) bf[b] = Bs[kr][32 * wn + 16 * b + (lane & 15)];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(af[a], bf[b], acc[a][b], 0, 0, 0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // v_mfma_f64_16x16x4_f64 returns rows lane/16, lane/16 + 4, ... in
        // its four doubles (row-interleaved, unlike the fp32 variant)
        const int m = m0 + 32 * wm + 16 * a + (lane >> 4) + 4 * i;
        const int n = n0 + 32 * wn + 16 * b + (lane & 15);
        if (m < g.M && n < g.N) {
          double* c = CN ? Cp + (int64_t)m * g.ldc + n : Cp + (int64_t)n * g.ldc + m;
          const double v = g.alpha * acc[a][b][i];
          *c = (g.beta == 0.0) ? v : g.beta * (*c) + v;
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

// -------------------------------------------------------------- trtri diag
// X_bb = inverse of the lower-triangular 64x64 diagonal block L_bb.
__global__ __launch_bounds__(256) void trtri_diag_kernel(const double* __restrict__ L, int ldl,
                                                         double* __restrict__ X, int ldx, int d) {
  __shared__ double Ls[NB][NB + 1];
  __shared__ double Xs[NB][NB + 1];
  const int b0 = blockIdx.x * NB;
  const int nb = min(NB, d - b0);
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  for (int e = tid; e < NB * NB; e += 256) {
    const int i = e / NB, j = e % NB;
    double v = (i == j) ? 1.0 : 0.0;
    if (i < nb && j <= i) v = L[(int64_t)(b0 + i) * ldl + b0 + j];
    Ls[i][j] = v;
    Xs[i][j] = (i == j) ? 1.0 : 0.0;  // right-hand side I, overwritten by X
  }
  __syncthreads();
  // rows top-down: x_m = xs_m / L_mm is final at step m; then xs_i -= L_im x_m for i > m
  for (int m = 0; m < nb; ++m) {
    const double inv = 1.0 / Ls[m][m];
    for (int i = m + 1 + ty; i < nb; i += 16) {
      const double lim = Ls[i][m] * inv;
      for (int j = tx; j <= m; j += 16) Xs[i][j] -= lim * Xs[m][j];
    }
    __syncthreads();
  }
  for (int e = tid; e < NB * NB; e += 256) {
    const int i = e / NB, j = e % NB;
    if (i < nb && j < nb) X[(int64_t)(b0 + i) * ldx + b0 + j] = (j <= i) ? Xs[i][j] / Ls[i][i] : 0.0;
  }
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

}  // namespace

hipError_t launch_damp_to_f64(const float* H, int d, double percdamp, double* A, int* flag,
                              hipStream_t s) {
  double* lam = reinterpret_cast<double*>(reinterpret_cast<char*>(flag) + 8);
  hipLaunchKernelGGL(damp_lambda_kernel, dim3(1), dim3(256), 0, s, H, d, percdamp, lam, flag);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)d * d;
  hipLaunchKernelGGL(damp_copy_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, H, d,
                     (const double*)lam, A);
  return hipGetLastError();
}

hipError_t launch_potrf_panel(double* A, int lda, int d, int k, int* flag, int info_offset,
                              hipStream_t s) {
  hipLaunchKernelGGL(potrf_diag_kernel, dim3(1), dim3(256), 0, s, A, lda, d, k, flag, info_offset);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nbelow = (int)ceil_div(d - k, NB) - 1;
  if (nbelow > 0) {
    hipLaunchKernelGGL(potrf_trsm_kernel, dim3(nbelow), dim3(256), 0, s, A, lda, d, k);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_potrf_update(double* A, int lda, int d, int k, hipStream_t s) {
  const int t0 = k + NB;
  GemmDesc g{};
  g.A = A + (int64_t)t0 * lda + k;
  g.B = A + (int64_t)t0 * lda + k;
  g.C = A + (int64_t)t0 * lda + t0;
  g.lda = g.ldb = g.ldc = lda;
  g.M = g.N = d - t0;
  g.K = NB;
  g.alpha = -1.0;
  g.beta = 1.0;
  g.tri = 1;
  g.kmode = 0;
  return gemm64<true, false, true>(g, 1, s);
}

hipError_t launch_trtri_diag(const double* L, int ldl, double* X, int ldx, int d, hipStream_t s) {
  hipLaunchKernelGGL(trtri_diag_kernel, dim3((unsigned)ceil_div(d, NB)), dim3(256), 0, s, L, ldl,
                     X, ldx, d);
  return hipGetLastError();
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
    g1.bsa = (int64_t)2 * half * (ldl + 1); g1.bsb = bs; g1.bsc = bs;
    hipError_t e = gemm64<true, true, false>(g1, batches, s);
    if (e != hipSuccess) return e;
    GemmDesc g2{};
    g2.A = X + (int64_t)c0 * ldx + c0;  // C^-1, lower
    g2.B = X + (int64_t)a0 * ldx + c0;  // T (element (k=c, n=a) at T^T[a][c])
    g2.C = X + (int64_t)c0 * ldx + a0;
    g2.lda = ldx; g2.ldb = ldx; g2.ldc = ldx;
    g2.M = sc; g2.N = half; g2.K = sc;
    g2.alpha = -1.0; g2.beta = 0.0; g2.tri = 0; g2.kmode = 2;
    g2.bsa = bs; g2.bsb = bs; g2.bsc = bs;
    e = gemm64<true, false, true>(g2, batches, s);
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
  return gemm64<false, true, true>(g, 1, s);
}

hipError_t launch_store_upper_f32(const double* L2, int ld2, float* Hinv, int d, hipStream_t s) {
  const int nt = (int)ceil_div(d, 64);
  hipLaunchKernelGGL(store_upper_kernel, dim3(nt, nt), dim3(256), 0, s, L2, ld2, Hinv, d);
  return hipGetLastError();
}

}  // namespace gptq
