// Act-order (desc_act): the columns of a layer are processed in decreasing
// order of the Hessian diagonal H_qq, so the inputs with the largest
// activations are quantized first, while many columns remain to absorb their
// error ("GPTQ: fixing errors as you go", "The tricks that make it fast";
// "GPTQ > The GPTQ Algorithm", the note on quantization order).
//
// perm[k] is the original column processed k-th.  Ties keep the original
// column order, so the order is a function of the diagonal alone.  The other
// stages gather through perm (the damped H copy, the W working copy) and the
// outputs are scattered back to the original column order here.
//
// Every kernel that reads a perm entry clamps it into [0, n): a caller's
// array that is not a permutation gives undefined numbers, never an access
// outside the buffers.
#include <limits.h>

#include "common.h"

namespace gptq {
namespace {

// Sort key of a diagonal entry: IEEE total order mapped onto unsigned
// integers (a larger key is a larger value), with -0 taken as +0.  Every
// float, NaN included, gets a key, so the ranks below always form a
// permutation.
__device__ inline uint32_t order_key(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kRankChunk = 2048;
constexpr int kRankCols = 16;  // columns per workgroup, 16 lanes each

// rank(c) = #{c' : key(c') > key(c), or key(c') == key(c) and c' < c};
// perm[rank(c)] = c.  A workgroup ranks 16 columns; lane s of a column's 16
// compares the keys s, s + 16, ... of each chunk of the diagonal staged in
// LDS (in a wave, lanes of one slice read the same word and the 16 slices
// read 16 consecutive words), and the 16 partial counts are summed with lane
// shuffles.
__global__ __launch_bounds__(256) void act_order_rank_kernel(const float* __restrict__ H,
                                                             int64_t d, int* __restrict__ perm) {
  __shared__ uint32_t keys[kRankChunk];
  const int tid = threadIdx.x;
  const int sl = tid & (kRankCols - 1);
  const int64_t c = (int64_t)blockIdx.x * kRankCols + (tid >> 4);
  const bool valid = c < d;
  const uint32_t kc = valid ? order_key(H[c * d + c]) : 0u;
  int rank = 0;
  for (int64_t base = 0; base < d; base += kRankChunk) {
    const int n = (int)((d - base < kRankChunk) ? d - base : kRankChunk);
    __syncthreads();
    for (int t = tid; t < n; t += 256) keys[t] = order_key(H[(base + t) * d + base + t]);
    __syncthreads();
    // columns of this chunk before c (all of them when the chunk ends at or
    // before c) win ties
    const int64_t before = c - base;
    for (int t = sl; t < n; t += kRankCols) {
      const uint32_t k = keys[t];
      rank += (k > kc) | ((k == kc) & (t < before));
    }
  }
#pragma unroll
  for (int m = kRankCols / 2; m > 0; m >>= 1) rank += __shfl_xor(rank, m, kRankCols);
  if (valid && sl == 0) perm[rank] = (int)c;
}

// ---- checks of a caller's perm (values in range, each index exactly once)
__global__ __launch_bounds__(256) void perm_init_kernel(int* __restrict__ inv, int64_t n,
                                                        int* __restrict__ bad) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) inv[i] = -1;
  if (i == 0) *bad = 0;
}

// inv[perm[j]] = j; a value outside [0, n) marks the perm bad
__global__ __launch_bounds__(256) void perm_scatter_kernel(const int* __restrict__ perm, int64_t n,
                                                           int* __restrict__ inv,
                                                           int* __restrict__ bad) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= n) return;
  const int p = perm[j];
  if (p < 0 || (int64_t)p >= n) {
    *bad = 1;
    return;
  }
  inv[p] = (int)j;
}

// every index must have been hit, by an entry that still holds it (a
// duplicate leaves some index unhit)
__global__ __launch_bounds__(256) void perm_verify_kernel(const int* __restrict__ perm, int64_t n,
                                                          const int* __restrict__ inv,
                                                          int* __restrict__ bad) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= n) return;
  const int j = inv[c];
  if (j < 0 || (int64_t)j >= n || perm[j] != (int)c) *bad = 1;
}

// inv[perm[j]] = j with perm clamped (no checks: used after a checked call)
__global__ __launch_bounds__(256) void perm_inverse_kernel(const int* __restrict__ perm, int64_t n,
                                                           int* __restrict__ inv) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= n) return;
  const int p = min(max(perm[j], 0), (int)(n - 1));
  inv[p] = (int)j;
}

// Outputs back to the original column order: codes[r][c] = cp[r][inv[c]]
// (cp: codes in processing order); workgroup 0 also writes
// losses[c] = lp[inv[c]] and g_idx[c] = inv[c] / g.  One workgroup per row:
// with `stage` the row of cp is first copied to LDS (dynamic, cols bytes) so
// the gather reads LDS; four columns per thread, written as one 32-bit word
// when vec4 (cols % 4 == 0 and codes 4-byte aligned).
__global__ __launch_bounds__(256) void unpermute_outputs_kernel(
    const uint8_t* __restrict__ cp, int64_t rows, int64_t cols, const int* __restrict__ inv,
    uint8_t* __restrict__ codes, const float* __restrict__ lp, float* __restrict__ losses,
    int g, int* __restrict__ g_idx, bool vec4, bool stage) {
  extern __shared__ uint8_t rowbuf[];
  const int64_t r = blockIdx.x;
  const uint8_t* src = cp + r * cols;
  if (stage) {
    for (int64_t c = threadIdx.x; c < cols; c += 256) rowbuf[c] = src[c];
    __syncthreads();
    src = rowbuf;
  }
  const int cmax = (int)(cols - 1);
  for (int64_t c0 = (int64_t)threadIdx.x * 4; c0 < cols; c0 += 1024) {
    int k[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) k[u] = (c0 + u < cols) ? min(max(inv[c0 + u], 0), cmax) : 0;
    uint8_t* dst = codes + r * cols + c0;
    if (vec4 && c0 + 4 <= cols) {
      const uint32_t w = (uint32_t)src[k[0]] | ((uint32_t)src[k[1]] << 8) |
                         ((uint32_t)src[k[2]] << 16) | ((uint32_t)src[k[3]] << 24);
      *reinterpret_cast<uint32_t*>(dst) = w;
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (c0 + u < cols) dst[u] = src[k[u]];
    }
    if (r == 0) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (c0 + u >= cols) break;
        losses[c0 + u] = lp[k[u]];
        if (g_idx != nullptr) g_idx[c0 + u] = k[u] / g;
      }
    }
  }
}

// g_idx[c] = c / g (the identity order)
__global__ __launch_bounds__(256) void group_index_kernel(int64_t cols, int g,
                                                          int* __restrict__ g_idx) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c < cols) g_idx[c] = (int)(c / g);
}

}  // namespace

hipError_t launch_act_order(const float* H, int64_t d, int* perm, hipStream_t s) {
  hipLaunchKernelGGL(act_order_rank_kernel, dim3((unsigned)ceil_div(d, kRankCols)), dim3(256), 0,
                     s, H, d, perm);
  return hipGetLastError();
}

hipError_t launch_perm_check(const int* perm, int64_t n, int* inv, int* bad, hipStream_t s) {
  const dim3 grid((unsigned)ceil_div(n, 256));
  hipLaunchKernelGGL(perm_init_kernel, grid, dim3(256), 0, s, inv, n, bad);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(perm_scatter_kernel, grid, dim3(256), 0, s, perm, n, inv, bad);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(perm_verify_kernel, grid, dim3(256), 0, s, perm, n, (const int*)inv, bad);
  return hipGetLastError();
}

hipError_t launch_perm_inverse(const int* perm, int64_t n, int* inv, hipStream_t s) {
  hipLaunchKernelGGL(perm_inverse_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, perm,
                     n, inv);
  return hipGetLastError();
}

hipError_t launch_unpermute_outputs(const uint8_t* cp, int64_t rows, int64_t cols, const int* inv,
                                    uint8_t* codes, const float* lp, float* losses, int g,
                                    int* g_idx, hipStream_t s) {
  const bool vec4 = (cols % 4 == 0) && ((reinterpret_cast<uintptr_t>(codes) & 3) == 0);
  const bool stage = cols <= kStageBytes;
  hipLaunchKernelGGL(unpermute_outputs_kernel, dim3((unsigned)rows), dim3(256),
                     stage ? (unsigned)cols : 0u, s, cp, rows, cols, inv, codes, lp, losses, g,
                     g_idx, vec4, stage);
  return hipGetLastError();
}

hipError_t launch_group_index(int64_t cols, int g, int* g_idx, hipStream_t s) {
  hipLaunchKernelGGL(group_index_kernel, dim3((unsigned)ceil_div(cols, 256)), dim3(256), 0, s,
                     cols, g, g_idx);
  return hipGetLastError();
}

}  // namespace gptq
