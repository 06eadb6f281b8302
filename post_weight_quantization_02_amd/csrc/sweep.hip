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
//     columns it holds.  Hinv's 128x128 diagonal block is in LDS, permuted so
//     a lane's 8 coefficients for step j are contiguous; entries left of the
//     diagonal are zero, which makes the update of finished columns a no-op.
//   * Group min/max is a per-lane reduction followed by a 4-step xor shuffle
//     across the 16 lanes of the row.
//   * Per-column loss partials are reduced inside the workgroup and written
//     per workgroup; a final kernel adds them in a fixed order.
//
// The lazy update W[:, i2:] -= Err[:, i1:i2] Hinv[i1:i2, i2:] is an fp32
// MFMA GEMM (v_mfma_f32_16x16x4_f32), 128x128 output tiles, K = 128 streamed
// through LDS in chunks of 16.
#include "common.h"

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

// G: group size when it divides the block (16, 32, 64, 128); G == 0 means the
// group spans several blocks (groupsize a multiple of 128).
template <int G>
__global__ __launch_bounds__(256) void sweep_kernel(float* __restrict__ Wk, int64_t ldk,
                                                    int64_t rows, int64_t cols, int i1,
                                                    const float* __restrict__ Hinv, int bits,
                                                    int groupsize, uint8_t* __restrict__ codes,
                                                    float* __restrict__ scales,
                                                    float* __restrict__ zeros,
                                                    float* __restrict__ Err,
                                                    float* __restrict__ lpart) {
  __shared__ __attribute__((aligned(16))) float Up[BC * RL * CPL];  // [j][l][k]
  __shared__ float rdiag[BC];
  __shared__ float lsum[4][BC];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l = lane & 15;
  const int rg = lane >> 4;
  const int64_t row = (int64_t)blockIdx.x * kSweepRows + wave * 4 + rg;
  const bool rv = row < rows;
  const int nbc = (int)((cols - i1) < BC ? (cols - i1) : BC);
  const int64_t ngroups = ceil_div(cols, groupsize);

  for (int e = tid; e < BC * BC; e += 256) {
    const int j = e >> 7, c = e & (BC - 1);
    float v = 0.f;
    if (c >= j && c < nbc) v = Hinv[(int64_t)(i1 + j) * cols + i1 + c];
    Up[(j * RL + (c & 15)) * CPL + (c >> 4)] = v;
  }
  for (int j = tid; j < BC; j += 256)
    rdiag[j] = (j < nbc) ? 1.f / Hinv[(int64_t)(i1 + j) * cols + i1 + j] : 0.f;

  float w[CPL];
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    const int c = l + RL * k;
    w[k] = (rv && c < nbc) ? Wk[row * ldk + i1 + c] : 0.f;
  }
  __syncthreads();

  const float qm = (float)((1 << bits) - 1);
  float s = 1.f, z = 0.f;
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
      row_minmax(mn, mx);
      grid_params(mn, mx, qm, s, z);
      if (rv && l == 0) {
        scales[row * ngroups + gi] = s;
        zeros[row * ngroups + gi] = z;
      }
    } else if (rv) {
      s = scales[row * ngroups + gi];
      z = zeros[row * ngroups + gi];
    }
  }

  float qc[CPL], ev[CPL];
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    qc[k] = 0.f;
    ev[k] = 0.f;
  }

#pragma unroll
  for (int j = 0; j < BC; ++j) {
    if (j < nbc) {
      const int kj = j >> 4, lj = j & 15;
      if (G != 0 && j % (G > 0 ? G : 1) == 0) {
        float mn = INFINITY, mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
          const int c = l + RL * k;
          if (c >= j && c < j + G && c < nbc) {
            mn = fminf(mn, w[k]);
            mx = fmaxf(mx, w[k]);
          }
        }
        row_minmax(mn, mx);
        grid_params(mn, mx, qm, s, z);
        if (rv && l == 0) {
          const int64_t gi = (i1 + j) / groupsize;
          scales[row * ngroups + gi] = s;
          zeros[row * ngroups + gi] = z;
        }
      }
      const float x = w[kj];
      const float t = x / s + z;
      const float q = fminf(fmaxf(rintf(t), 0.f), qm);
      const float err = x - (q - z) * s;
      const float e = err * rdiag[j];
      const float eb = __shfl(e, lj, RL);
      if (l == lj) {
        qc[kj] = q;
        ev[kj] = eb;
      }
      const float* u = Up + (j * RL + l) * CPL;
#pragma unroll
      for (int k = kj; k < CPL; ++k) w[k] -= eb * u[k];
    }
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
constexpr int LT = 128;  // output tile edge
constexpr int LK = 16;   // K chunk
constexpr int LP = LT + 4;

__global__ __launch_bounds__(256) void lazy_kernel(float* __restrict__ Wk, int64_t ldk,
                                                   int64_t rows, int64_t cols, int i1, int i2,
                                                   const float* __restrict__ Err,
                                                   const float* __restrict__ Hinv) {
  __shared__ float As[LK][LP];  // [k][m]
  __shared__ float Bs[LK][LP];  // [k][n]
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t r0 = (int64_t)blockIdx.y * LT;
  const int64_t n0 = (int64_t)i2 + (int64_t)blockIdx.x * LT;
  const int K = i2 - i1;

  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int kc = 0; kc < K; kc += LK) {
#pragma unroll
    for (int q = 0; q < (LT * LK) / 256; ++q) {
      const int e = tid + 256 * q;
      // A: Err rows, 16 consecutive k per row
      const int kk = e & (LK - 1), mm = e >> 4;
      const int64_t gr = r0 + mm;
      As[kk][mm] = (gr < rows && kc + kk < K) ? Err[gr * ldk + i1 + kc + kk] : 0.f;
      // B: Hinv rows i1+kc+kk, 128 consecutive columns
      const int nn = e & (LT - 1), kb = e >> 7;
      const int64_t gc = n0 + nn;
      Bs[kb][nn] = (gc < cols && kc + kb < K) ? Hinv[(int64_t)(i1 + kc + kb) * cols + gc] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < LK; ks += 4) {
      const int kr = ks + (lane >> 4);
      float af[4], bf[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) af[a] = As[kr][64 * wm + 16 * a + (lane & 15)];
#pragma unroll
      for (int b = 0; b < 4; ++b) bf[b] = Bs[kr][64 * wn + 16 * b + (lane & 15)];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[a], bf[b], acc[a][b], 0, 0, 0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = r0 + 64 * wm + 16 * a + 4 * (lane >> 4) + i;
        const int64_t c = n0 + 64 * wn + 16 * b + (lane & 15);
        if (r < rows && c < cols) Wk[r * ldk + c] -= acc[a][b][i];
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

__global__ __launch_bounds__(256) void loss_reduce_kernel(const float* __restrict__ lpart,
                                                          int64_t nparts, int64_t ldk,
                                                          int64_t cols, float* __restrict__ out) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= cols) return;
  float s = 0.f;
  for (int64_t p = 0; p < nparts; ++p) s += lpart[p * ldk + c];
  out[c] = s;
}

}  // namespace

hipError_t launch_convert_w(const void* W, int w_dtype, int64_t rows, int64_t cols, int64_t ldw,
                            float* Wk, int64_t ldk, hipStream_t s) {
  dim3 grid((unsigned)rows, (unsigned)((ceil_div(ldk, 256) < 16) ? ceil_div(ldk, 256) : 16));
  if (w_dtype == GPTQ_DTYPE_F16)
    hipLaunchKernelGGL(convert_kernel<_Float16>, grid, dim3(256), 0, s,
                       reinterpret_cast<const _Float16*>(W), rows, cols, ldw, Wk, ldk);
  else
    hipLaunchKernelGGL(convert_kernel<float>, grid, dim3(256), 0, s,
                       reinterpret_cast<const float*>(W), rows, cols, ldw, Wk, ldk);
  return hipGetLastError();
}

hipError_t launch_sweep_block(float* Wk, int64_t ldk, int64_t rows, int64_t cols, int i1,
                              const float* Hinv, int bits, int groupsize, uint8_t* codes,
                              float* scales, float* zeros, float* Err, float* lpart,
                              hipStream_t s) {
  dim3 grid((unsigned)ceil_div(rows, kSweepRows));
#define GPTQ_SWEEP(G)                                                                          \
  hipLaunchKernelGGL(sweep_kernel<G>, grid, dim3(256), 0, s, Wk, ldk, rows, cols, i1, Hinv,   \
                     bits, groupsize, codes, scales, zeros, Err, lpart)
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

hipError_t launch_lazy_update(float* Wk, int64_t ldk, int64_t rows, int64_t cols, int i1, int i2,
                              const float* Err, const float* Hinv, hipStream_t s) {
  dim3 grid((unsigned)ceil_div(cols - i2, LT), (unsigned)ceil_div(rows, LT));
  hipLaunchKernelGGL(lazy_kernel, grid, dim3(256), 0, s, Wk, ldk, rows, cols, i1, i2, Err, Hinv);
  return hipGetLastError();
}

hipError_t launch_loss_reduce(const float* lpart, int64_t nparts, int64_t cols, float* losses,
                              hipStream_t s) {
  const int64_t ldk = round_up(cols, kBlock);
  hipLaunchKernelGGL(loss_reduce_kernel, dim3((unsigned)ceil_div(cols, 256)), dim3(256), 0, s,
                     lpart, nparts, ldk, cols, losses);
  return hipGetLastError();
}

}  // namespace gptq
