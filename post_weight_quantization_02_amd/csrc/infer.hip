// Inference with the stored quantized weights: the low-bit codes packed into
// 32-bit words and the product y = x W_hat^T with W_hat dequantized on the
// fly ("GPTQ: fixing errors as you go": the file holds the low-bit integers
// and one scale per 128 weights, and decode, which is memory-bound, gets
// faster; "GPTQ, Line by Line", the AutoGPTQ example).
//
// Packed layout: row r of the codes is stored along the input dimension in
// words of K = floor(32 / bits) codes, the code of column c at bits
// [bits * (c % K), bits * (c % K) + bits) of word c / K; unused high bits are
// zero.  W_hat[r][c] = (code - zero[r][g]) * scale[r][g] with the fp32
// scales and zeros of the quantizer, g = g_idx[c] (act-order) or
// c / groupsize.
//
// The product is written for decode: a few tokens x (fp16, m x cols) against
// a weight matrix streamed once from HBM per pass of up to 4 tokens.  Each
// wave owns 4 output rows; its lanes take the packed words of those rows in
// lane order (each load instruction reads consecutive words), dequantize in
// fp32 and accumulate x * W_hat with fp32 FMAs; the 64 lane sums of every
// output are added by lane shuffles.
#include "common.h"

namespace gptq {
namespace {

// One thread per output word: packed[r][w] = sum_j (codes[r][w*K + j] & mask)
// << (bits * j).
__global__ __launch_bounds__(256) void pack_codes_kernel(const uint8_t* __restrict__ codes,
                                                         int64_t rows, int64_t cols, int bits,
                                                         int64_t nw, uint32_t* __restrict__ out) {
  const int64_t r = blockIdx.y;
  const int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (w >= nw) return;
  const int k = 32 / bits;
  const uint32_t mask = (1u << bits) - 1u;
  const uint8_t* src = codes + r * cols;
  uint32_t v = 0;
  for (int j = 0; j < k; ++j) {
    const int64_t c = w * k + j;
    if (c < cols) v |= ((uint32_t)src[c] & mask) << (bits * j);
  }
  out[r * nw + w] = v;
}

constexpr int kGemvRows = 4;   // output rows per wave
constexpr int kGemvUnroll = 4; // words per lane in flight per row

// y[t][r] = sum_c x[t][c] * W_hat[r][c] for t < m <= MT.
template <int BITS, int MT>
__global__ __launch_bounds__(256) void dequant_gemv_kernel(
    const _Float16* __restrict__ x, int64_t ldx, int m, const uint32_t* __restrict__ packed,
    int64_t nw, int64_t rows, int64_t cols, const float* __restrict__ scales,
    const float* __restrict__ zeros, int64_t ngroups, int groupsize, const int* __restrict__ g_idx,
    float* __restrict__ y, int64_t ldy) {
  constexpr int K = 32 / BITS;
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  constexpr int R = kGemvRows;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r0 = ((int64_t)blockIdx.x * 4 + wave) * R;
  if (r0 >= rows) return;  // whole wave idle (no barrier below)
  // rows past the matrix read row rows - 1 and are not stored
  int64_t rr[R];
#pragma unroll
  for (int i = 0; i < R; ++i) rr[i] = (r0 + i < rows) ? r0 + i : rows - 1;
  // one (scale, zero) per word when no word straddles a group
  const bool word_groups = (g_idx == nullptr) && (groupsize % K == 0);
  float acc[R][MT];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[i][t] = 0.f;

  for (int64_t wb = 0; wb < nw; wb += 64 * kGemvUnroll) {
    uint32_t q[kGemvUnroll][R];
#pragma unroll
    for (int u = 0; u < kGemvUnroll; ++u) {
      const int64_t w = wb + 64 * u + lane;
      const int64_t wc = (w < nw) ? w : nw - 1;
#pragma unroll
      for (int i = 0; i < R; ++i) q[u][i] = packed[rr[i] * nw + wc];
    }
#pragma unroll
    for (int u = 0; u < kGemvUnroll; ++u) {
      const int64_t w = wb + 64 * u + lane;
      if (w >= nw) break;
      const int64_t c0 = w * K;
      // x of the word's columns (0 past the last column)
      float xv[MT][K];
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int j = 0; j < K; ++j)
          xv[t][j] = (t < m && c0 + j < cols) ? (float)x[(int64_t)t * ldx + c0 + j] : 0.f;
      if (word_groups) {
        const int64_t g = c0 / groupsize;
#pragma unroll
        for (int i = 0; i < R; ++i) {
          const float s = scales[rr[i] * ngroups + g];
          const float z = zeros[rr[i] * ngroups + g];
#pragma unroll
          for (int j = 0; j < K; ++j) {
            const float wv = ((float)((q[u][i] >> (BITS * j)) & MASK) - z) * s;
#pragma unroll
            for (int t = 0; t < MT; ++t) acc[i][t] = __builtin_fmaf(xv[t][j], wv, acc[i][t]);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < K; ++j) {
          const int64_t c = (c0 + j < cols) ? c0 + j : cols - 1;
          const int64_t g = (g_idx != nullptr) ? (int64_t)g_idx[c] : c / groupsize;
          const int64_t gc = (g < 0) ? 0 : ((g >= ngroups) ? ngroups - 1 : g);
#pragma unroll
          for (int i = 0; i < R; ++i) {
            const float wv =
                ((float)((q[u][i] >> (BITS * j)) & MASK) - zeros[rr[i] * ngroups + gc]) *
                scales[rr[i] * ngroups + gc];
#pragma unroll
            for (int t = 0; t < MT; ++t) acc[i][t] = __builtin_fmaf(xv[t][j], wv, acc[i][t]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      float v = acc[i][t];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
      acc[i][t] = v;
    }
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int t = 0; t < MT; ++t)
        if (t < m && r0 + i < rows) y[(int64_t)t * ldy + r0 + i] = acc[i][t];
  }
}

template <int BITS>
hipError_t launch_gemv_bits(const _Float16* x, int64_t ldx, int64_t m, const uint32_t* packed,
                            int64_t nw, int64_t rows, int64_t cols, const float* scales,
                            const float* zeros, int64_t ngroups, int groupsize, const int* g_idx,
                            float* y, int64_t ldy, hipStream_t s) {
  const dim3 grid((unsigned)ceil_div(rows, 4 * kGemvRows));
  for (int64_t t0 = 0; t0 < m; t0 += 4) {
    const int mt = (int)((m - t0 < 4) ? m - t0 : 4);
    const _Float16* xt = x + t0 * ldx;
    float* yt = y + t0 * ldy;
    if (mt == 1)
      hipLaunchKernelGGL((dequant_gemv_kernel<BITS, 1>), grid, dim3(256), 0, s, xt, ldx, mt,
                         packed, nw, rows, cols, scales, zeros, ngroups, groupsize, g_idx, yt, ldy);
    else if (mt == 2)
      hipLaunchKernelGGL((dequant_gemv_kernel<BITS, 2>), grid, dim3(256), 0, s, xt, ldx, mt,
                         packed, nw, rows, cols, scales, zeros, ngroups, groupsize, g_idx, yt, ldy);
    else
      hipLaunchKernelGGL((dequant_gemv_kernel<BITS, 4>), grid, dim3(256), 0, s, xt, ldx, mt,
                         packed, nw, rows, cols, scales, zeros, ngroups, groupsize, g_idx, yt, ldy);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

int64_t packed_words(int64_t cols, int bits) { return ceil_div(cols, 32 / bits); }

hipError_t launch_pack_codes(const uint8_t* codes, int64_t rows, int64_t cols, int bits,
                             uint32_t* packed, hipStream_t s) {
  const int64_t nw = packed_words(cols, bits);
  hipLaunchKernelGGL(pack_codes_kernel, dim3((unsigned)ceil_div(nw, 256), (unsigned)rows),
                     dim3(256), 0, s, codes, rows, cols, bits, nw, packed);
  return hipGetLastError();
}

hipError_t launch_dequant_gemv(const _Float16* x, int64_t ldx, int64_t m, const uint32_t* packed,
                               int bits, int64_t rows, int64_t cols, const float* scales,
                               const float* zeros, int groupsize, const int* g_idx, float* y,
                               int64_t ldy, hipStream_t s) {
  const int64_t nw = packed_words(cols, bits);
  const int64_t ngroups = ceil_div(cols, groupsize);
  switch (bits) {
#define GPTQ_GEMV(B) \
  case B:            \
    return launch_gemv_bits<B>(x, ldx, m, packed, nw, rows, cols, scales, zeros, ngroups, \
                               groupsize, g_idx, y, ldy, s);
    GPTQ_GEMV(2)
    GPTQ_GEMV(3)
    GPTQ_GEMV(4)
    GPTQ_GEMV(5)
    GPTQ_GEMV(6)
    GPTQ_GEMV(7)
    GPTQ_GEMV(8)
#undef GPTQ_GEMV
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gptq
