// Host side of the C ABI declared in include/gptq.h: argument validation,
// workspace carving and the launch order of the gfx950 kernels.
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include "common.h"

using namespace gptq;

namespace {

constexpr size_t kAlign = 256;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Upper bound on dimensions: indices are int inside the kernels.
constexpr int64_t kMaxDim = 1 << 20;
constexpr int64_t kMaxElems = (int64_t)1 << 40;

size_t acc_bytes(int64_t d, int64_t n) {
  if (d < 1 || d > kMaxDim || n < 0) return 0;
  if (n == 0) return 0;
  const int64_t nb = ceil_div(d, kSyrkTile);
  const int64_t tiles = nb * (nb + 1) / 2;
  const int splits = syrk_splits(d, n);
  return align_up((size_t)splits * tiles * kSyrkTile * kSyrkTile * sizeof(float));
}

size_t prep_bytes(int64_t d) {
  if (d < 1 || d > kMaxDim) return 0;
  return 2 * align_up((size_t)d * d * sizeof(double)) + kAlign;
}

struct QuantLayout {
  int64_t ldk;        // row stride of the fp32 working copy and of Err
  size_t wk_off, err_off, loss_off, total;
  int64_t nparts;     // loss partial rows
  // act-order: codes and losses in processing order, and the inverse order
  size_t cp_off, lp_off, inv_off, total_perm;
};

QuantLayout quant_layout(int64_t rows, int64_t cols) {
  QuantLayout L{};
  L.ldk = round_up(cols, kBlock);
  L.nparts = ceil_div(rows, kSweepRows);
  L.wk_off = 0;
  L.err_off = L.wk_off + align_up((size_t)rows * L.ldk * sizeof(float));
  L.loss_off = L.err_off + align_up((size_t)rows * L.ldk * sizeof(float));
  L.total = L.loss_off + align_up((size_t)L.nparts * L.ldk * sizeof(float));
  L.cp_off = L.total;
  L.lp_off = L.cp_off + align_up((size_t)rows * cols);
  L.inv_off = L.lp_off + align_up((size_t)cols * sizeof(float));
  L.total_perm = L.inv_off + align_up((size_t)cols * sizeof(int));
  return L;
}

size_t quant_bytes(int64_t rows, int64_t cols, bool perm) {
  if (rows < 1 || cols < 1 || rows > kMaxDim || cols > kMaxDim) return 0;
  const QuantLayout L = quant_layout(rows, cols);
  return perm ? L.total_perm : L.total;
}

bool group_ok(int g) {
  if (g == 16 || g == 32 || g == 64) return true;
  return g >= kBlock && g % kBlock == 0;
}

// Blocked Cholesky of the lower triangle of A (d x d), in place; the
// inverted 64x64 diagonal blocks of L land at the diagonal of Xi.
//
// While more than kSingleLevelTail columns remain after an outer block, the
// factorization is two-level: the outer block of kOuterPanel columns is
// factored panel by panel with updates confined to it (the serial chain of
// 64x64 diagonal blocks with small updates beside it), then the trailing
// matrix takes one rank-kOuterPanel update (a GEMM, MFMA-bound).  Rank-64
// updates of a large trailing matrix are bound by moving it (HBM, or the
// Infinity Cache while it fits), so this moves it once per outer block
// instead of once per panel.  The last kSingleLevelTail (or fewer) columns
// are right-looking with 64-column panels, each trailing update (rank 64)
// also factoring the next diagonal block; once the trailing matrix is small
// the steps are bound by the serial chain (panel solve, diagonal update,
// diagonal factorization), so the solve and the update share one launch and
// the panels of those steps are copied into A at the end.
constexpr int kSingleLevelTail = 3072;
constexpr int64_t kFusedStepTiles = 512;  // trailing 64x64 tiles below which a step is one launch
hipError_t potrf(double* A, int d, int* flag, int info_offset, double* Xi, hipStream_t s) {
  hipError_t e = launch_potrf_diag(A, d, d, 0, flag, info_offset, Xi, d, s);
  int K = 0;
  while (e == hipSuccess && d - K - kOuterPanel > kSingleLevelTail) {
    const int Kend = K + kOuterPanel;
    for (int k = K; k < Kend && e == hipSuccess; k += kPanel) {
      e = launch_potrf_trsm(A, d, d, k, Xi, d, s);
      if (e == hipSuccess && k + kPanel < Kend)
        e = launch_potrf_update(A, d, d, k, (int)ceil_div(Kend - k - kPanel, kPanel), flag,
                                info_offset, Xi, d, s);
    }
    if (e == hipSuccess) e = launch_potrf_outer_update(A, d, d, K, Kend, s);
    if (e == hipSuccess) e = launch_potrf_diag(A, d, d, Kend, flag, info_offset, Xi, d, s);
    K = Kend;
  }
  int fused_from = d;
  for (int k = K; k < d && e == hipSuccess; k += kPanel) {
    const int64_t nt = ceil_div(d - k - kPanel, kPanel);
    if (nt > 0 && nt * (nt + 1) / 2 <= kFusedStepTiles) {
      e = launch_potrf_fused(A, d, d, k, flag, info_offset, Xi, d, s);
      if (fused_from == d) fused_from = k;
      continue;
    }
    e = launch_potrf_trsm(A, d, d, k, Xi, d, s);
    if (e == hipSuccess && k + kPanel < d)
      e = launch_potrf_update(A, d, d, k, d, flag, info_offset, Xi, d, s);
  }
  if (e == hipSuccess && fused_from < d) e = launch_copy_panels(A, d, d, fused_from, Xi, d, s);
  return e;
}

}  // namespace

extern "C" {

int gptq_version(void) { return 100; }

const char* gptq_status_string(int status) {
  switch (status) {
    case GPTQ_OK: return "GPTQ_OK";
    case GPTQ_ERR_INVALID_ARG: return "GPTQ_ERR_INVALID_ARG";
    case GPTQ_ERR_WORKSPACE: return "GPTQ_ERR_WORKSPACE";
    case GPTQ_ERR_NOT_PD: return "GPTQ_ERR_NOT_PD";
    case GPTQ_ERR_HIP: return "GPTQ_ERR_HIP";
    case GPTQ_ERR_UNSUPPORTED: return "GPTQ_ERR_UNSUPPORTED";
    default: return "GPTQ_ERR_UNKNOWN";
  }
}

size_t gptq_workspace_bytes(int op, int64_t rows, int64_t cols, int64_t n) {
  switch (op) {
    case GPTQ_OP_ACCUMULATE: return acc_bytes(cols, n);
    case GPTQ_OP_PREPARE: return prep_bytes(cols);
    case GPTQ_OP_QUANTIZE: return quant_bytes(rows, cols, false);
    case GPTQ_OP_QUANTIZE_PERM: return quant_bytes(rows, cols, true);
    default: return 0;
  }
}

gptq_status gptq_hessian_accumulate(float* H, int64_t d, const void* X, int64_t n, int64_t ldx,
                                    float alpha, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  if (d < 1 || d > kMaxDim || n < 0 || ldx < d) return GPTQ_ERR_INVALID_ARG;
  if (H == nullptr || (n > 0 && X == nullptr)) return GPTQ_ERR_INVALID_ARG;
  if (n > 0 && (n > kMaxElems / ldx)) return GPTQ_ERR_INVALID_ARG;
  if (!aligned(H, 4) || !aligned(X, 2)) return GPTQ_ERR_INVALID_ARG;
  if (n == 0) return GPTQ_OK;
  const size_t need = acc_bytes(d, n);
  if (workspace_bytes < need || (need > 0 && workspace == nullptr)) return GPTQ_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return GPTQ_ERR_INVALID_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int splits = syrk_splits(d, n);
  const int64_t kper = syrk_kper(n, splits);
  float* P = reinterpret_cast<float*>(workspace);
  if (launch_syrk_partial(reinterpret_cast<const _Float16*>(X), ldx, (int)d, n, splits, kper, P,
                          s) != hipSuccess)
    return GPTQ_ERR_HIP;
  if (launch_syrk_reduce(P, (int)d, splits, alpha, H, s) != hipSuccess) return GPTQ_ERR_HIP;
  return GPTQ_OK;
}

}  // extern "C"

namespace {

// The preparation with an optional act-order permutation (perm == nullptr:
// the identity).  Validation of the scalar arguments is done by the callers.
gptq_status prepare_impl(const float* H, int64_t d, const int* perm, double percdamp, float* Hinv,
                         void* workspace, size_t workspace_bytes, int64_t* info, void* stream,
                         bool three_step = false) {
  if (info) *info = 0;
  if (d < 1 || d > 65536 || H == nullptr || Hinv == nullptr) return GPTQ_ERR_INVALID_ARG;
  if (!(percdamp >= 0.0) || percdamp > 1e6) return GPTQ_ERR_INVALID_ARG;
  if (!aligned(H, 4) || !aligned(Hinv, 4) || !aligned(perm, 4)) return GPTQ_ERR_INVALID_ARG;
  const size_t need = prep_bytes(d);
  if (workspace == nullptr || workspace_bytes < need) return GPTQ_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return GPTQ_ERR_INVALID_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int di = (int)d;
  const size_t mat = align_up((size_t)d * d * sizeof(double));
  double* A = reinterpret_cast<double*>(workspace);
  double* Xi = reinterpret_cast<double*>(reinterpret_cast<char*>(workspace) + mat);
  // flag words: [0] pivot flag (int), [8] lambda (double), [16] perm check (int)
  int* flag = reinterpret_cast<int*>(reinterpret_cast<char*>(workspace) + 2 * mat);
  int* permbad = reinterpret_cast<int*>(reinterpret_cast<char*>(flag) + 16);

#define GPTQ_TRY(call) \
  do {                 \
    if ((call) != hipSuccess) return GPTQ_ERR_HIP; \
  } while (0)

  // act-order: check that perm is a permutation (Xi is free scratch until the
  // first factorization writes its block inverses)
  if (perm != nullptr) GPTQ_TRY(launch_perm_check(perm, d, reinterpret_cast<int*>(Xi), permbad, s));
  int hflag[5] = {0, 0, 0, 0, 0};
  if (!three_step) {
    // A = J H_d J (H_d = H + lambda I, or P H P^T + lambda I; J the reversal),
    // fp64, lower triangle; resets the pivot flag.
    GPTQ_TRY(launch_damp_to_f64(H, di, percdamp, perm, true, A, flag, s));
    // L = chol(A), in place; the inverted 64x64 diagonal blocks of L land in Xi.
    GPTQ_TRY(potrf(A, di, flag, 0, Xi, s));
    // Xi = L^{-1}: combine the inverted diagonal blocks level by level
    for (int half = kPanel; half < di; half *= 2)
      GPTQ_TRY(launch_trtri_level(A, di, Xi, di, di, half, s));
    // Hinv = J L^{-1} J, the upper Cholesky factor of H_d^{-1}, fp32
    GPTQ_TRY(launch_store_reversed_f32(Xi, di, Hinv, di, s));
    GPTQ_TRY(hipMemcpyAsync(hflag, flag, sizeof(hflag), hipMemcpyDeviceToHost, s));
    GPTQ_TRY(hipStreamSynchronize(s));
    if (perm != nullptr && hflag[4] != 0) return GPTQ_ERR_INVALID_ARG;
    if (hflag[0] == 0x7fffffff) return GPTQ_OK;
  }

  // The pages' three steps in forward order: on request, or when H_d is
  // not numerically positive definite in reversed order, to find the first
  // failing pivot of chol(H_d), or of chol(H_d^{-1}) (reported from d + 1 on).
  GPTQ_TRY(launch_damp_to_f64(H, di, percdamp, perm, false, A, flag, s));
  GPTQ_TRY(potrf(A, di, flag, 0, Xi, s));
  for (int half = kPanel; half < di; half *= 2) GPTQ_TRY(launch_trtri_level(A, di, Xi, di, di, half, s));
  // A = Xi^T Xi = H_d^{-1} (lower triangle)
  GPTQ_TRY(launch_lauum(Xi, di, A, di, di, s));
  // L2 = chol(H_d^{-1}), in place (Xi is free again and takes the block inverses)
  GPTQ_TRY(potrf(A, di, flag, di, Xi, s));
  // Hinv = L2^T (upper), fp32
  GPTQ_TRY(launch_store_upper_f32(A, di, Hinv, di, s));
  GPTQ_TRY(hipMemcpyAsync(hflag, flag, sizeof(hflag), hipMemcpyDeviceToHost, s));
  GPTQ_TRY(hipStreamSynchronize(s));
#undef GPTQ_TRY
  if (perm != nullptr && hflag[4] != 0) return GPTQ_ERR_INVALID_ARG;
  if (hflag[0] != 0x7fffffff) {
    if (info) *info = hflag[0];
    return GPTQ_ERR_NOT_PD;
  }
  return GPTQ_OK;
}

// The sweep with an optional act-order permutation.  With perm, W's columns
// are gathered into processing order, the sweep's codes and losses go to the
// workspace, and one kernel writes them back in the original column order
// together with g_idx.
gptq_status quantize_impl(const void* W, int w_dtype, int64_t rows, int64_t cols, int64_t ldw,
                          const int* perm, const float* Hinv, int bits, int groupsize,
                          int blocksize, uint8_t* codes, float* scales, float* zeros,
                          float* losses, int* g_idx, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (rows < 1 || cols < 1 || rows > kMaxDim || cols > kMaxDim || ldw < cols)
    return GPTQ_ERR_INVALID_ARG;
  if (W == nullptr || Hinv == nullptr || codes == nullptr || scales == nullptr ||
      zeros == nullptr || losses == nullptr)
    return GPTQ_ERR_INVALID_ARG;
  if (w_dtype != GPTQ_DTYPE_F16 && w_dtype != GPTQ_DTYPE_F32) return GPTQ_ERR_INVALID_ARG;
  if (bits < 2 || bits > 8) return GPTQ_ERR_INVALID_ARG;
  if (groupsize < 1 || blocksize < 1) return GPTQ_ERR_INVALID_ARG;
  // groupsize >= cols: one group per row (per-channel), statistics at
  // column 0 only, before any update
  const bool per_channel = groupsize >= cols;
  // group statistics taken at a group start must see every pending update:
  // either groups lie inside blocks or blocks inside groups
  if (!per_channel && groupsize % blocksize != 0 && blocksize % groupsize != 0)
    return GPTQ_ERR_INVALID_ARG;
  if (rows > kMaxElems / ldw) return GPTQ_ERR_INVALID_ARG;
  if (!aligned(W, w_dtype == GPTQ_DTYPE_F16 ? 2 : 4) || !aligned(Hinv, 4) ||
      !aligned(scales, 4) || !aligned(zeros, 4) || !aligned(losses, 4) || !aligned(perm, 4) ||
      !aligned(g_idx, 4))
    return GPTQ_ERR_INVALID_ARG;
  if (blocksize != kBlock || (!per_channel && !group_ok(groupsize))) return GPTQ_ERR_UNSUPPORTED;
  const QuantLayout L = quant_layout(rows, cols);
  const size_t need = perm != nullptr ? L.total_perm : L.total;
  if (workspace == nullptr || workspace_bytes < need) return GPTQ_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return GPTQ_ERR_INVALID_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  float* Wk = reinterpret_cast<float*>(ws + L.wk_off);
  float* Err = reinterpret_cast<float*>(ws + L.err_off);
  float* lpart = reinterpret_cast<float*>(ws + L.loss_off);
  // with act-order the sweep writes processing-order codes and losses here
  uint8_t* sweep_codes = perm != nullptr ? reinterpret_cast<uint8_t*>(ws + L.cp_off) : codes;
  float* sweep_losses = perm != nullptr ? reinterpret_cast<float*>(ws + L.lp_off) : losses;

  if (launch_convert_w(W, w_dtype, rows, cols, ldw, perm, Wk, L.ldk, s) != hipSuccess)
    return GPTQ_ERR_HIP;
  // Two-level lazy batching.  Inside a superblock of SB columns each block's
  // errors reach the rest of the superblock before those columns are swept;
  // the columns after the superblock receive all of its errors in one GEMM
  // with K = SB.  Every column still gets every update before its block is
  // swept (and before its group's statistics are taken: when groups span
  // blocks SB is a multiple of the group size, so every group lies inside
  // one superblock and its later columns receive each block's errors right
  // away), so the result equals per-block lazy updates in exact arithmetic.  When groups lie
  // inside blocks, the sweep kernel applies a block's pending errors from the
  // earlier blocks of its superblock itself (to its own rows, just before
  // sweeping them); when groups span blocks, a group's statistics read
  // columns of later blocks, so those get each block's errors right away in a
  // separate lazy update.
  // (A single per-channel group takes its statistics before any update, so
  // it puts no constraint on the superblock.)
  const int64_t SB = (groupsize > kBlock && !per_channel)
                         ? groupsize * ceil_div(kSuperBlock, groupsize)
                         : kSuperBlock;
  const bool fused_near = groupsize <= kBlock;
  for (int64_t s0 = 0; s0 < cols; s0 += SB) {
    const int64_t s1 = (s0 + SB < cols) ? s0 + SB : cols;
    for (int64_t i1 = s0; i1 < s1; i1 += kBlock) {
      const int64_t i2 = (i1 + kBlock < s1) ? i1 + kBlock : s1;
      if (launch_sweep_block(Wk, L.ldk, rows, cols, (int)i1, (int)(fused_near ? s0 : i1), Hinv,
                             bits, groupsize, sweep_codes, scales, zeros, Err, lpart, s) !=
          hipSuccess)
        return GPTQ_ERR_HIP;
      if (!fused_near &&
          launch_lazy_update(Wk, L.ldk, rows, cols, (int)i1, (int)i2, (int)i2, (int)s1, Err, Hinv,
                             s) != hipSuccess)
        return GPTQ_ERR_HIP;
    }
    if (launch_lazy_update(Wk, L.ldk, rows, cols, (int)s0, (int)s1, (int)s1, (int)cols, Err, Hinv,
                           s) != hipSuccess)
      return GPTQ_ERR_HIP;
  }
  if (launch_loss_reduce(lpart, L.nparts, cols, sweep_losses, s) != hipSuccess) return GPTQ_ERR_HIP;
  if (perm != nullptr) {
    int* inv = reinterpret_cast<int*>(ws + L.inv_off);
    if (launch_perm_inverse(perm, cols, inv, s) != hipSuccess) return GPTQ_ERR_HIP;
    if (launch_unpermute_outputs(sweep_codes, rows, cols, inv, codes, sweep_losses, losses,
                                 groupsize, g_idx, s) != hipSuccess)
      return GPTQ_ERR_HIP;
  } else if (g_idx != nullptr) {
    if (launch_group_index(cols, groupsize, g_idx, s) != hipSuccess) return GPTQ_ERR_HIP;
  }
  return GPTQ_OK;
}

}  // namespace

extern "C" {

gptq_status gptq_prepare_hinv(const float* H, int64_t d, double percdamp, float* Hinv,
                              void* workspace, size_t workspace_bytes, int64_t* info,
                              void* stream) {
  return prepare_impl(H, d, nullptr, percdamp, Hinv, workspace, workspace_bytes, info, stream);
}

gptq_status gptq_prepare_hinv_three_step(const float* H, int64_t d, double percdamp, float* Hinv,
                                         void* workspace, size_t workspace_bytes, int64_t* info,
                                         void* stream) {
  return prepare_impl(H, d, nullptr, percdamp, Hinv, workspace, workspace_bytes, info, stream,
                      true);
}

gptq_status gptq_quantize_layer(const void* W, int w_dtype, int64_t rows, int64_t cols,
                                int64_t ldw, const float* Hinv, int bits, int groupsize,
                                int blocksize, uint8_t* codes, float* scales, float* zeros,
                                float* losses, void* workspace, size_t workspace_bytes,
                                void* stream) {
  return quantize_impl(W, w_dtype, rows, cols, ldw, nullptr, Hinv, bits, groupsize, blocksize,
                       codes, scales, zeros, losses, nullptr, workspace, workspace_bytes, stream);
}

gptq_status gptq_act_order(const float* H, int64_t d, int32_t* perm, void* stream) {
  if (d < 1 || d > kMaxDim || H == nullptr || perm == nullptr) return GPTQ_ERR_INVALID_ARG;
  if (!aligned(H, 4) || !aligned(perm, 4)) return GPTQ_ERR_INVALID_ARG;
  if (launch_act_order(H, d, perm, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return GPTQ_ERR_HIP;
  return GPTQ_OK;
}

gptq_status gptq_prepare_hinv_perm(const float* H, int64_t d, const int32_t* perm,
                                   double percdamp, float* Hinv, void* workspace,
                                   size_t workspace_bytes, int64_t* info, void* stream) {
  return prepare_impl(H, d, perm, percdamp, Hinv, workspace, workspace_bytes, info, stream);
}

gptq_status gptq_quantize_layer_perm(const void* W, int w_dtype, int64_t rows, int64_t cols,
                                     int64_t ldw, const int32_t* perm, const float* Hinv,
                                     int bits, int groupsize, int blocksize, uint8_t* codes,
                                     float* scales, float* zeros, float* losses, int32_t* g_idx,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  return quantize_impl(W, w_dtype, rows, cols, ldw, perm, Hinv, bits, groupsize, blocksize,
                       codes, scales, zeros, losses, g_idx, workspace, workspace_bytes, stream);
}

int64_t gptq_packed_words(int64_t cols, int bits) {
  if (cols < 1 || cols > kMaxDim || bits < 2 || bits > 8) return 0;
  return packed_words(cols, bits);
}

gptq_status gptq_pack_codes(const uint8_t* codes, int64_t rows, int64_t cols, int bits,
                            uint32_t* packed, void* stream) {
  if (rows < 1 || cols < 1 || rows > kMaxDim || cols > kMaxDim || bits < 2 || bits > 8)
    return GPTQ_ERR_INVALID_ARG;
  if (codes == nullptr || packed == nullptr || !aligned(packed, 4)) return GPTQ_ERR_INVALID_ARG;
  if (launch_pack_codes(codes, rows, cols, bits, packed, reinterpret_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return GPTQ_ERR_HIP;
  return GPTQ_OK;
}

gptq_status gptq_dequant_gemm(const void* x, int64_t m, int64_t cols, int64_t ldx,
                              const uint32_t* packed, int bits, int64_t rows, const float* scales,
                              const float* zeros, int groupsize, const int32_t* g_idx, float* y,
                              int64_t ldy, void* stream) {
  if (m < 0 || rows < 1 || cols < 1 || rows > kMaxDim || cols > kMaxDim) return GPTQ_ERR_INVALID_ARG;
  if (bits < 2 || bits > 8 || groupsize < 1 || ldy < rows || (m > 0 && ldx < cols))
    return GPTQ_ERR_INVALID_ARG;
  if (m > kMaxElems / (ldx > ldy ? ldx : ldy)) return GPTQ_ERR_INVALID_ARG;
  if (packed == nullptr || scales == nullptr || zeros == nullptr) return GPTQ_ERR_INVALID_ARG;
  if (m > 0 && (x == nullptr || y == nullptr)) return GPTQ_ERR_INVALID_ARG;  // m = 0: never read
  if (!aligned(x, 2) || !aligned(packed, 4) || !aligned(scales, 4) || !aligned(zeros, 4) ||
      !aligned(g_idx, 4) || !aligned(y, 4))
    return GPTQ_ERR_INVALID_ARG;
  if (m == 0) return GPTQ_OK;
  if (launch_dequant_gemv(reinterpret_cast<const _Float16*>(x), ldx, m, packed, bits, rows, cols,
                          scales, zeros, groupsize, g_idx, y, ldy,
                          reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return GPTQ_ERR_HIP;
  return GPTQ_OK;
}

gptq_status gptq_linear_forward(const void* x, int64_t m, int64_t cols, int64_t ldx,
                                const uint32_t* packed, int bits, int64_t rows,
                                const float* scales, const float* zeros, int groupsize, int relu,
                                void* y, int64_t ldy, void* stream) {
  if (m < 0 || rows < 1 || cols < 1 || rows > kMaxDim || cols > kMaxDim) return GPTQ_ERR_INVALID_ARG;
  if (bits < 2 || bits > 8 || groupsize < 1 || ldy < rows || (m > 0 && ldx < cols) ||
      (relu != 0 && relu != 1))
    return GPTQ_ERR_INVALID_ARG;
  if (m > kMaxElems / (ldx > ldy ? ldx : ldy)) return GPTQ_ERR_INVALID_ARG;
  if (packed == nullptr || scales == nullptr || zeros == nullptr) return GPTQ_ERR_INVALID_ARG;
  if (m > 0 && (x == nullptr || y == nullptr)) return GPTQ_ERR_INVALID_ARG;  // m = 0: never read
  if (!aligned(x, 2) || !aligned(packed, 4) || !aligned(scales, 4) || !aligned(zeros, 4) ||
      !aligned(y, 2))
    return GPTQ_ERR_INVALID_ARG;
  if (!linear_forward_supported(bits, m, rows, cols, groupsize, x, m > 0 ? ldx : 8, packed))
    return GPTQ_ERR_UNSUPPORTED;
  if (m == 0) return GPTQ_OK;
  if (launch_linear_forward(bits, reinterpret_cast<const _Float16*>(x), ldx, m, packed, rows, cols,
                            scales, zeros, groupsize, relu == 1, reinterpret_cast<_Float16*>(y),
                            ldy, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return GPTQ_ERR_HIP;
  return GPTQ_OK;
}

}  // extern "C"
