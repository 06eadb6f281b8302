// Internal helpers shared by the gfx950 kernels and the host entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gptq.h"

namespace gptq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// Index of a lower-triangle tile (bi >= bj) in row-major order of the lower
// triangle: t = bi*(bi+1)/2 + bj.
__host__ __device__ inline void lower_tile(int64_t t, int& bi, int& bj) {
  int64_t i = (int64_t)((__builtin_sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
  while (i * (i + 1) / 2 > t) --i;
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  bi = (int)i;
  bj = (int)(t - i * (i + 1) / 2);
}

// ---------------------------------------------------------------- launches
// Each launcher returns hipSuccess or the launch error.
hipError_t launch_syrk_partial(const _Float16* X, int64_t ldx, int d, int64_t n, int splits,
                               int64_t kper, float* partials, hipStream_t s);
hipError_t launch_syrk_reduce(const float* partials, int d, int splits, float alpha, float* H,
                              hipStream_t s);

int syrk_splits(int64_t d, int64_t n);
int64_t syrk_kper(int64_t n, int splits);
constexpr int kSyrkTile = 256;

// fp64 Cholesky route
// perm == nullptr: A = H + lambda I; else A = P H P^T + lambda I (act-order).
// reverse: rows and columns in reversed order, A = J (...) J with J the
// reversal permutation.
hipError_t launch_damp_to_f64(const float* H, int d, double percdamp, const int* perm, bool reverse,
                              double* A, int* flag, hipStream_t s);
// Cholesky of panel k's 64x64 diagonal block, with its inverse stored in Xi
hipError_t launch_potrf_diag(double* A, int lda, int d, int k, int* flag, int info_offset,
                             double* Xi, int ldxi, hipStream_t s);
// L_ik = A_ik L_kk^-T below panel k's diagonal block
hipError_t launch_potrf_trsm(double* A, int lda, int d, int k, const double* Xi, int ldxi,
                             hipStream_t s);
// update after panel k of the first ncol 64-column blocks to its right, fused
// with the diagonal block of panel k+1
hipError_t launch_potrf_update(double* A, int lda, int d, int k, int ncol, int* flag,
                               int info_offset, double* Xi, int ldxi, hipStream_t s);
// one whole panel step (solve, update, next diagonal block) for a small
// trailing matrix
hipError_t launch_potrf_fused(double* A, int lda, int d, int k, int* flag, int info_offset,
                              double* Xi, int ldxi, hipStream_t s);
hipError_t launch_copy_panels(double* A, int lda, int d, int k0, const double* Xi, int ldxi,
                              hipStream_t s);
// rank-(k1-k0) update of A[k1:, k1:] by the finished outer block [k0, k1)
hipError_t launch_potrf_outer_update(double* A, int lda, int d, int k0, int k1, hipStream_t s);
hipError_t launch_trtri_level(const double* L, int ldl, double* X, int ldx, int d, int half,
                              hipStream_t s);
hipError_t launch_lauum(const double* X, int ldx, double* S, int lds, int d, hipStream_t s);
hipError_t launch_store_upper_f32(const double* L2, int ld2, float* Hinv, int d, hipStream_t s);
// Hinv[i][j] = X[d-1-i][d-1-j] on and above the diagonal, 0 below (fp32)
hipError_t launch_store_reversed_f32(const double* X, int ldx, float* Hinv, int d, hipStream_t s);
constexpr int kPanel = 64;
constexpr int kOuterPanel = 1024;  // columns per outer block of the two-level Cholesky

// sweep
// perm != nullptr gathers W's columns into processing order (act-order)
hipError_t launch_convert_w(const void* W, int w_dtype, int64_t rows, int64_t cols, int64_t ldw,
                            const int* perm, float* Wk, int64_t ldk, hipStream_t s);
// sweep of the block at column i1; with p0 < i1 (groups inside blocks), the
// pending errors of blocks [p0, i1) are applied to the block first
hipError_t launch_sweep_block(float* Wk, int64_t ldk, int64_t rows, int64_t cols, int i1, int p0,
                              const float* Hinv, int bits, int groupsize, uint8_t* codes,
                              float* scales, float* zeros, float* Err, float* loss_part,
                              hipStream_t s);
hipError_t launch_lazy_update(float* Wk, int64_t ldk, int64_t rows, int64_t cols, int k0, int k1,
                              int c0, int c1, const float* Err, const float* Hinv, hipStream_t s);
hipError_t launch_loss_reduce(const float* loss_part, int64_t nparts, int64_t cols,
                              float* losses, hipStream_t s);
// act-order
constexpr int64_t kStageBytes = 48 * 1024;  // largest row a gather kernel stages in LDS
hipError_t launch_act_order(const float* H, int64_t d, int* perm, hipStream_t s);
// *bad = 0 if perm is a permutation of [0, n), else 1 (inv: n ints of scratch)
hipError_t launch_perm_check(const int* perm, int64_t n, int* inv, int* bad, hipStream_t s);
hipError_t launch_perm_inverse(const int* perm, int64_t n, int* inv, hipStream_t s);
hipError_t launch_unpermute_outputs(const uint8_t* cp, int64_t rows, int64_t cols, const int* inv,
                                    uint8_t* codes, const float* lp, float* losses, int g,
                                    int* g_idx, hipStream_t s);
hipError_t launch_group_index(int64_t cols, int g, int* g_idx, hipStream_t s);
// inference with the packed codes
int64_t packed_words(int64_t cols, int bits);
hipError_t launch_pack_codes(const uint8_t* codes, int64_t rows, int64_t cols, int bits,
                             uint32_t* packed, hipStream_t s);
hipError_t launch_dequant_gemv(const _Float16* x, int64_t ldx, int64_t m, const uint32_t* packed,
                               int bits, int64_t rows, int64_t cols, const float* scales,
                               const float* zeros, int groupsize, const int* g_idx, float* y,
                               int64_t ldy, hipStream_t s);
// the forward product of a 4- or 8-bit layer for many tokens (MFMA), fp16 out
bool linear_forward_supported(int bits, int64_t m, int64_t rows, int64_t cols, int groupsize,
                              const void* x, int64_t ldx, const void* packed);
hipError_t launch_linear_forward(int bits, const _Float16* x, int64_t ldx, int64_t m,
                                 const uint32_t* packed, int64_t rows, int64_t cols,
                                 const float* scales, const float* zeros, int groupsize, bool relu,
                                 _Float16* y, int64_t ldy, hipStream_t s);
constexpr int kSweepRows = 16;  // rows per sweep workgroup
constexpr int kBlock = 128;     // columns per block
constexpr int kSuperBlock = 512;  // columns per superblock of the two-level lazy update

}  // namespace gptq
