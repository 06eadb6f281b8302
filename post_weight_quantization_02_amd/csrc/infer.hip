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
// a weight matrix streamed once from HBM per pass of up to 4 tokens.  The
// general kernel (any bit width, g_idx) gives each wave 4 output rows whose
// packed words its lanes take in lane order, dequantizes in fp32 and
// accumulates x * W_hat with fp32 FMAs.  The fast kernel (2, 4, 8 bits, runs
// of 4 words inside a group) stages x in LDS, reads 4 words per lane and row
// with one 16-byte load (prefetched a batch ahead with the groups' scales and
// zeros), sums x * code per run -- for 4 bits two codes per v_dot2_f32_f16 --
// and applies scale and zero once per run.  The 64 lane sums of every output
// are added by lane shuffles.  For 2 to 32 tokens with 4-bit codes in groups
// of a multiple of 128 columns, the MFMA kernel reads each packed word once
// for all of the pass's tokens (see dequant_gemm_mfma_kernel).
#include "common.h"

namespace gptq {
namespace {

// One thread per output word: packed[r][w] = sum_j (codes[r][w*K + j] & mask)
// << (bits * j).
__global__ __launch_bounds__(256) void pack_codes_kernel(const uint8_t* __restrict__ codes,
                                                         int64_t rows, int64_t cols, int bits,
                                                         int64_t nw, uint32_t* __restrict__ out) {
  const int64_t r = blockIdx.x;
  const int64_t w = (int64_t)blockIdx.y * 256 + threadIdx.x;
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

// Code j of a word as a float, for 2, 4 and 8 bits: the codes are spread
// into bytes by masking (K / 4 byte lanes per mask) and each byte converted
// with v_cvt_f32_ubyteN.
template <int BITS>
__device__ inline void unpack_word(uint32_t w, float (&q)[32 / BITS]) {
  if (BITS == 8) {
#pragma unroll
    for (int b = 0; b < 4; ++b) q[b] = (float)((w >> (8 * b)) & 0xFFu);
  } else {
    constexpr int P = 8 / BITS;  // codes per byte
    constexpr uint32_t M = (BITS == 4) ? 0x0F0F0F0Fu : 0x03030303u;
#pragma unroll
    for (int k = 0; k < P; ++k) {
      const uint32_t v = (w >> (BITS * k)) & M;  // byte n holds code P*n + k
#pragma unroll
      for (int n = 0; n < 4; ++n) q[P * n + k] = (float)((v >> (8 * n)) & 0xFFu);
    }
  }
}

// Fast path for 2, 4 and 8 bits when every 4-word run of a row (4K columns)
// lies in one group and no g_idx is given.  x (MT tokens) is staged in LDS as
// fp16.  A lane reads 4 words of each of its R rows with one 16-byte load
// and, per run, sums x * code and x over the run's columns; the group's scale
// and zero then enter once per run: y += s * (sum x q - z * sum x), which
// equals sum x (q - z) s.  Rounding: the products x * q are exact in fp32,
// so each output's error is at most
// (4K + ceil(runs / 64) + 8) * 2^-24 * sum_c |x_c| (|q_c| + |z_g|) s_g.
template <int BITS, int MT, int R, bool XD>
__global__ __launch_bounds__(256) void dequant_gemv_fast_kernel(
    const _Float16* __restrict__ x, int64_t ldx, int m, const uint32_t* __restrict__ packed,
    int64_t nw, int64_t rows, int64_t cols, const float* __restrict__ scales,
    const float* __restrict__ zeros, int64_t ngroups, int groupsize, float* __restrict__ y,
    int64_t ldy, bool xvec) {
  constexpr int K = 32 / BITS;
  constexpr int CW = 4 * K;  // columns per 4-word run
  // R: output rows per wave.  XD (4 bits, one token, cols a multiple of 32,
  // x rows 16-byte aligned): each lane loads its runs' x directly with the
  // packed words instead of the workgroup staging x in LDS (no barrier).
  static_assert(!XD || (BITS == 4 && MT == 1), "direct x: 4 bits, one token");

  extern __shared__ __attribute__((aligned(16))) _Float16 xs[];
  const int64_t ldxs = nw * K;  // a multiple of CW (nw % 4 == 0)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r0 = ((int64_t)blockIdx.x * 4 + wave) * R;
  // rows past the matrix read row rows - 1 and are not stored
  int64_t rr[R];
#pragma unroll
  for (int i = 0; i < R; ++i) rr[i] = (r0 + i < rows) ? r0 + i : rows - 1;
  const int64_t nv = nw / 4;  // 4-word runs per row
  // a batch is 2 runs per lane and row; the next batch is loaded while the
  // current one is used, and the first before x is staged
  // The group's scale and zero of each run travel with its words, so no
  // run waits for them after its products.
  uint4 qv[2][R], qn[2][R];
  float sv[2][R], zv[2][R], sn[2][R], zn[2][R];
  uint4 xb[2][XD ? 4 : 1], xn[2][XD ? 4 : 1];
  auto load_batch = [&](int64_t vb, uint4 (&dst)[2][R], float (&ds)[2][R], float (&dz)[2][R],
                        uint4 (&dx)[2][XD ? 4 : 1]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t v = vb + 64 * u + lane;
      const int64_t vc = (v < nv) ? v : nv - 1;
      const int64_t g = vc * CW / groupsize;
#pragma unroll
      for (int i = 0; i < R; ++i) {
        dst[u][i] = reinterpret_cast<const uint4*>(packed + rr[i] * nw)[vc];
        ds[u][i] = scales[rr[i] * ngroups + g];
        dz[u][i] = zeros[rr[i] * ngroups + g];
      }
      if constexpr (XD) {
#pragma unroll
        for (int wd = 0; wd < 4; ++wd)
          dx[u][wd] = *reinterpret_cast<const uint4*>(x + vc * CW + 8 * wd);
      }
    }
  };
  load_batch(0, qv, sv, zv, xb);
  // staging: 8 halves per 16-byte load where the row allows it (ldxs is a
  // multiple of 8; x rows 16-byte aligned when xvec)
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  if constexpr (!XD) {
#pragma unroll
  for (int t = 0; t < MT; ++t)
    for (int64_t c = (int64_t)threadIdx.x * 8; c < ldxs; c += 256 * 8) {
      h8 v;
      if (xvec && t < m && c + 8 <= cols) {
        v = *reinterpret_cast<const h8*>(x + t * ldx + c);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          v[j] = (t < m && c + j < cols) ? x[t * ldx + c + j] : (_Float16)0.f;
      }
      *reinterpret_cast<h8*>(xs + t * ldxs + c) = v;
    }
  __syncthreads();
  }
  if (r0 >= rows) return;  // no barrier below
  float acc[R][MT];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[i][t] = 0.f;
  for (int64_t vb = 0; vb < nv; vb += 128) {
    const bool more = vb + 128 < nv;
    if (more) load_batch(vb + 128, qn, sn, zn, xn);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t v = vb + 64 * u + lane;
      if (v >= nv) break;
      const int64_t c0 = v * CW;
      float sx[MT], sq[R][MT], so[R][MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        sx[t] = 0.f;
#pragma unroll
        for (int i = 0; i < R; ++i) sq[i][t] = so[i][t] = 0.f;
      }
      if constexpr (BITS == 4) {
        // Two codes per packed-fp16 operation: (w >> 4k) & 0x000F000F puts
        // codes k and k + 4 of a word in the low bits of the two halves; OR
        // 0x6400 makes each the fp16 number 1024 + q, and subtracting 1024
        // leaves q exactly.  v_dot2_f32_f16 then adds x_k q_k + x_{k+4}
        // q_{k+4} (exact products) to an fp32 sum; x is paired to match once
        // per word for all rows.
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        typedef _Float16 h8v __attribute__((ext_vector_type(8)));
        const h2 ones = {(_Float16)1.f, (_Float16)1.f};
        const h2 k1024 = {(_Float16)1024.f, (_Float16)1024.f};
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
          h2 xp[MT][4];
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            h8v xw;
            if constexpr (XD)
              xw = __builtin_bit_cast(h8v, xb[u][wd]);
            else
              xw = *reinterpret_cast<const h8v*>(xs + t * ldxs + c0 + wd * 8);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              xp[t][k] = h2{xw[k], xw[k + 4]};
              sx[t] = __builtin_amdgcn_fdot2(xp[t][k], ones, sx[t], false);
            }
          }
#pragma unroll
          for (int i = 0; i < R; ++i) {
            const uint32_t w = (wd == 0) ? qv[u][i].x : (wd == 1) ? qv[u][i].y
                             : (wd == 2) ? qv[u][i].z : qv[u][i].w;
            // codes 2j, 2j+4 from (w >> 8j) & 0x000F000F; codes 2j+1, 2j+5
            // in place from (w >> 8j) & 0x00F000F0 as 16 q (exact in fp16),
            // summed apart and scaled by 1/16 (exact) when the run is applied
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const uint32_t wj = w >> (8 * j);
              const h2 qe = __builtin_bit_cast(h2, (wj & 0x000F000Fu) | 0x64006400u) - k1024;
              const h2 qo = __builtin_bit_cast(h2, (wj & 0x00F000F0u) | 0x64006400u) - k1024;
#pragma unroll
              for (int t = 0; t < MT; ++t) {
                sq[i][t] = __builtin_amdgcn_fdot2(xp[t][2 * j], qe, sq[i][t], false);
                so[i][t] = __builtin_amdgcn_fdot2(xp[t][2 * j + 1], qo, so[i][t], false);
              }
            }
          }
        }
      } else {
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        float xv[MT][K];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          // K halves at an offset that is a multiple of K (>= 4): 8-byte
          // aligned reads of 4 halves
          const _Float16* xp = xs + t * ldxs + c0 + wd * K;
#pragma unroll
          for (int j0 = 0; j0 < K; j0 += 4) {
            typedef _Float16 h4 __attribute__((ext_vector_type(4)));
            const h4 hv = *reinterpret_cast<const h4*>(xp + j0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              xv[t][j0 + j] = (float)hv[j];
              sx[t] += xv[t][j0 + j];
            }
          }
        }
#pragma unroll
        for (int i = 0; i < R; ++i) {
          const uint32_t w = (wd == 0) ? qv[u][i].x : (wd == 1) ? qv[u][i].y
                           : (wd == 2) ? qv[u][i].z : qv[u][i].w;
          float q[K];
          unpack_word<BITS>(w, q);
#pragma unroll
          for (int j = 0; j < K; ++j)
#pragma unroll
            for (int t = 0; t < MT; ++t) sq[i][t] = __builtin_fmaf(xv[t][j], q[j], sq[i][t]);
        }
      }
      }
#pragma unroll
      for (int i = 0; i < R; ++i)
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const float q = __builtin_fmaf(so[i][t], 0.0625f, sq[i][t]);  // so is 0 below 4 bits
          acc[i][t] = __builtin_fmaf(sv[u][i], __builtin_fmaf(-zv[u][i], sx[t], q), acc[i][t]);
        }
    }
    if (more) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < R; ++i) {
          qv[u][i] = qn[u][i];
          sv[u][i] = sn[u][i];
          zv[u][i] = zn[u][i];
        }
      if constexpr (XD) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int wd = 0; wd < 4; ++wd) xb[u][wd] = xn[u][wd];
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

// ---------------------------------------------------------------- a few tokens on MFMA
// y = x W_hat^T for 2..32 tokens in one pass over the weights: 4-bit codes,
// groups of a multiple of 128 columns (or one group per row), cols % 128 ==
// 0, x rows and the packed rows 16-byte aligned.
//
// A workgroup owns 16 output rows; its four waves split the row's 128-column
// chunks into quarters and their partial tiles are added in a fixed order at
// the end.  Per chunk a wave runs v_mfma_f32_16x16x32_f16 with A = x (16
// tokens) and B = the codes as exact fp16 integers (16 rows): over a chunk,
// lane group k (lanes 16k..16k+15) takes columns 32k..32k+31, so a lane's B
// operands are the four words of one 16-byte load and its A operands four
// 16-byte pieces of an x row.  A second MFMA against all-ones gives sum x over
// the chunk in the same layout, and the chunk enters the running sums as
// s * (sum x q - z * sum x), which equals sum x (q - z) s for any fp32 zero.
// The products are exact in fp32, so the error is the fp32 summation error:
// at most (128 + ceil(cols / 512) + 8) * 2^-24 * sum_c |x_c| (|q_c| + |z|) s
// when each MFMA adds its 32 products and the accumulator no less accurately
// than sequential fp32 additions.  Loads run four chunks ahead.
constexpr int kMK = 128;   // columns per chunk
constexpr int kMPf = 4;    // chunks in flight per wave

typedef _Float16 mh2 __attribute__((ext_vector_type(2)));

// The 8 codes of one 4-bit word as exact fp16 integers, in column order:
// v_perm_b32 puts byte p in both halves (0x00bb00bb), an AND-OR makes the low
// half 0x6400 | q_lo = 1024 + q_lo and the high half 0x6400 | 16 q_hi = 1024 +
// 16 q_hi, and one packed fp16 FMA with (1, 1/16) and (-1024, -64) leaves
// (q_lo, q_hi).
__device__ inline half8 codes4_f16(uint32_t w) {
  const mh2 mul = {(_Float16)1.f, (_Float16)0.0625f};
  const mh2 off = {(_Float16)-1024.f, (_Float16)-64.f};
  half8 r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t b = __builtin_amdgcn_perm(w, w, (12u << 24) | ((uint32_t)p << 16) | (12u << 8) | p);
    const uint32_t m = (b & 0x00F0000Fu) | 0x64006400u;
    const mh2 h = __builtin_bit_cast(mh2, m) * mul + off;
    r[2 * p] = h[0];
    r[2 * p + 1] = h[1];
  }
  return r;
}

template <int TT>  // token tiles of 16 per pass
__global__ __launch_bounds__(256) void dequant_gemm_mfma_kernel(
    const _Float16* __restrict__ x, int64_t ldx, int m, const uint32_t* __restrict__ packed,
    int64_t nw, int64_t rows, int64_t cols, const float* __restrict__ scales,
    const float* __restrict__ zeros, int64_t ngroups, int groupsize, float* __restrict__ y,
    int64_t ldy) {
  __shared__ float part[4][TT * 16][17];  // per-wave partial tiles [wave][token][row]
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, kg = lane >> 4;
  const int64_t r0 = (int64_t)blockIdx.x * 16;
  const int64_t rr = (r0 + n < rows) ? r0 + n : rows - 1;  // this lane's weight row (clamped)
  const int nch = (int)(cols / kMK);
  const int cb = (nch * wave) / 4, ce = (nch * (wave + 1)) / 4;  // this wave's chunks
  const uint32_t* wrow = packed + rr * nw + 4 * kg;
  const float* srow = scales + rr * ngroups;
  const float* zrow = zeros + rr * ngroups;
  const _Float16* xrow[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) xrow[t] = x + (int64_t)min(16 * t + n, m - 1) * ldx + 32 * kg;

  // ring of kMPf chunks in flight: loads are unconditional, from chunk
  // indices clamped into this wave's range (or the row, for an empty range)
  uint4 wv[kMPf];
  half8 xv[kMPf][TT][4];
  float sv[kMPf], zv[kMPf];
  auto fetch = [&](int slot, int c) {
    const int cc = (c < ce) ? c : (ce > cb ? ce - 1 : (cb < nch ? cb : nch - 1));
    wv[slot] = *reinterpret_cast<const uint4*>(wrow + 16 * cc);
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        xv[slot][t][q] = *reinterpret_cast<const half8*>(xrow[t] + (int64_t)kMK * cc + 8 * q);
    const int64_t g = ((int64_t)kMK * cc) / groupsize;
    sv[slot] = srow[g];
    zv[slot] = zrow[g];
  };
#pragma unroll
  for (int i = 0; i < kMPf; ++i) fetch(i, cb + i);

  const half8 ones = {(_Float16)1.f, (_Float16)1.f, (_Float16)1.f, (_Float16)1.f,
                      (_Float16)1.f, (_Float16)1.f, (_Float16)1.f, (_Float16)1.f};
  f32x4 acc[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c0 = cb; c0 < ce; c0 += kMPf) {
#pragma unroll
    for (int i = 0; i < kMPf; ++i) {
      const int c = c0 + i;
      if (c < ce) {
        const uint32_t wd[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
        f32x4 d[TT], dx[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          d[t] = f32x4{0.f, 0.f, 0.f, 0.f};
          dx[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const half8 b = codes4_f16(wd[q]);
#pragma unroll
          for (int t = 0; t < TT; ++t) {
            d[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv[i][t][q], b, d[t], 0, 0, 0);
            dx[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv[i][t][q], ones, dx[t], 0, 0, 0);
          }
        }
        const float sc = sv[i], zc = zv[i];
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[t][e] = __builtin_fmaf(sc, __builtin_fmaf(-zc, dx[t][e], d[t][e]), acc[t][e]);
      }
      fetch(i, c + kMPf);
    }
  }
  // element e of acc[t] at lane (n, kg) is token 16 t + 4 kg + e, row r0 + n
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) part[wave][16 * t + 4 * kg + e][n] = acc[t][e];
  __syncthreads();
  for (int o = tid; o < TT * 256; o += 256) {
    const int tok = o >> 4, rw = o & 15;
    const float v = (part[0][tok][rw] + part[1][tok][rw]) + (part[2][tok][rw] + part[3][tok][rw]);
    if (tok < m && r0 + rw < rows) y[(int64_t)tok * ldy + r0 + rw] = v;
  }
}

bool dequant_mfma_ok(const _Float16* x, int64_t ldx, int64_t m, const uint32_t* packed, int bits,
                     int64_t cols, int groupsize, const int* g_idx) {
  return bits == 4 && m >= 2 && g_idx == nullptr && cols % kMK == 0 &&
         (groupsize % kMK == 0 || groupsize >= cols) && ldx % 8 == 0 &&
         (reinterpret_cast<uintptr_t>(x) & 15) == 0 &&
         (reinterpret_cast<uintptr_t>(packed) & 15) == 0;
}

hipError_t launch_dequant_mfma(const _Float16* x, int64_t ldx, int64_t m, const uint32_t* packed,
                               int64_t rows, int64_t cols, const float* scales,
                               const float* zeros, int groupsize, float* y, int64_t ldy,
                               hipStream_t s) {
  const int64_t nw = packed_words(cols, 4);
  const int64_t ngroups = ceil_div(cols, groupsize);
  const dim3 grid((unsigned)ceil_div(rows, 16));
  for (int64_t t0 = 0; t0 < m; t0 += 32) {
    const int mt = (int)((m - t0 < 32) ? m - t0 : 32);
    if (mt > 16)
      hipLaunchKernelGGL(dequant_gemm_mfma_kernel<2>, grid, dim3(256), 0, s, x + t0 * ldx, ldx, mt,
                         packed, nw, rows, cols, scales, zeros, ngroups, groupsize, y + t0 * ldy,
                         ldy);
    else
      hipLaunchKernelGGL(dequant_gemm_mfma_kernel<1>, grid, dim3(256), 0, s, x + t0 * ldx, ldx, mt,
                         packed, nw, rows, cols, scales, zeros, ngroups, groupsize, y + t0 * ldy,
                         ldy);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

constexpr int64_t kGemvLds = 64 * 1024;  // x staging limit of the fast path

template <int BITS, int R>
hipError_t launch_gemv_fast_direct(const _Float16* x, int64_t ldx, int64_t m,
                                   const uint32_t* packed, int64_t nw, int64_t rows, int64_t cols,
                                   const float* scales, const float* zeros, int64_t ngroups,
                                   int groupsize, float* y, int64_t ldy, hipStream_t s) {
  const dim3 grid((unsigned)ceil_div(rows, 4 * R));
  for (int64_t t0 = 0; t0 < m; ++t0) {
    hipLaunchKernelGGL((dequant_gemv_fast_kernel<BITS, 1, R, true>), grid, dim3(256), 0, s,
                       x + t0 * ldx, ldx, 1, packed, nw, rows, cols, scales, zeros, ngroups,
                       groupsize, y + t0 * ldy, ldy, true);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int BITS, int R>
hipError_t launch_gemv_fast(const _Float16* x, int64_t ldx, int64_t m, const uint32_t* packed,
                            int64_t nw, int64_t rows, int64_t cols, const float* scales,
                            const float* zeros, int64_t ngroups, int groupsize, float* y,
                            int64_t ldy, int maxmt, hipStream_t s) {
  const dim3 grid((unsigned)ceil_div(rows, 4 * R));
  const int64_t row_bytes = nw * (32 / BITS) * 2;
  const bool xvec = (ldx % 8 == 0) && ((reinterpret_cast<uintptr_t>(x) & 15) == 0);
  for (int64_t t0 = 0; t0 < m; t0 += maxmt) {
    const int mt = (int)((m - t0 < maxmt) ? m - t0 : maxmt);
    const _Float16* xt = x + t0 * ldx;
    float* yt = y + t0 * ldy;
    if (mt == 1)
      hipLaunchKernelGGL((dequant_gemv_fast_kernel<BITS, 1, R, false>), grid, dim3(256),
                         (unsigned)row_bytes, s, xt, ldx, mt, packed, nw, rows, cols, scales,
                         zeros, ngroups, groupsize, yt, ldy, xvec);
    else if (mt == 2)
      hipLaunchKernelGGL((dequant_gemv_fast_kernel<BITS, 2, R, false>), grid, dim3(256),
                         (unsigned)(2 * row_bytes), s, xt, ldx, mt, packed, nw, rows, cols,
                         scales, zeros, ngroups, groupsize, yt, ldy, xvec);
    else
      hipLaunchKernelGGL((dequant_gemv_fast_kernel<BITS, 4, R, false>), grid, dim3(256),
                         (unsigned)(4 * row_bytes), s, xt, ldx, mt, packed, nw, rows, cols,
                         scales, zeros, ngroups, groupsize, yt, ldy, xvec);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
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
  // rows in x (up to 2^31 workgroups), words in y (at most 2^20 / 4 / 256)
  hipLaunchKernelGGL(pack_codes_kernel, dim3((unsigned)rows, (unsigned)ceil_div(nw, 256)),
                     dim3(256), 0, s, codes, rows, cols, bits, nw, packed);
  return hipGetLastError();
}

hipError_t launch_dequant_gemv(const _Float16* x, int64_t ldx, int64_t m, const uint32_t* packed,
                               int bits, int64_t rows, int64_t cols, const float* scales,
                               const float* zeros, int groupsize, const int* g_idx, float* y,
                               int64_t ldy, hipStream_t s) {
  const int64_t nw = packed_words(cols, bits);
  const int64_t ngroups = ceil_div(cols, groupsize);
  // two tokens or more, 4 bits, whole 128-column chunks inside groups: MFMA,
  // the weights read once per 32 tokens
  if (dequant_mfma_ok(x, ldx, m, packed, bits, cols, groupsize, g_idx))
    return launch_dequant_mfma(x, ldx, m, packed, rows, cols, scales, zeros, groupsize, y, ldy, s);
  // fast path: 2, 4 or 8 bits, whole 4-word runs inside groups, no g_idx,
  // 16-byte aligned rows, x of at least one token fits the LDS staging
  if ((bits == 2 || bits == 4 || bits == 8) && g_idx == nullptr && nw % 4 == 0 &&
      groupsize % (4 * (32 / bits)) == 0 && (reinterpret_cast<uintptr_t>(packed) & 15) == 0) {
    const int64_t row_bytes = nw * (32 / bits) * 2;
    const int maxmt = (int)((kGemvLds / row_bytes >= 4) ? 4 : (kGemvLds / row_bytes >= 2) ? 2
                                                                                          : 1);
    if (row_bytes <= kGemvLds) {
      // two rows per wave (measured against one and four: 1.78 ms per
      // decode step against 1.86 and 1.81 at one token)
      if (bits == 2)
        return launch_gemv_fast<2, 2>(x, ldx, m, packed, nw, rows, cols, scales, zeros, ngroups,
                                      groupsize, y, ldy, maxmt, s);
      // one token, whole 32-column runs, aligned x rows: x loaded directly
      if (bits == 4 && m == 1 && cols % 32 == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0)
        return launch_gemv_fast_direct<4, 2>(x, ldx, m, packed, nw, rows, cols, scales, zeros,
                                             ngroups, groupsize, y, ldy, s);
      if (bits == 4)
        return launch_gemv_fast<4, 2>(x, ldx, m, packed, nw, rows, cols, scales, zeros, ngroups,
                                      groupsize, y, ldy, maxmt, s);
      return launch_gemv_fast<8, 2>(x, ldx, m, packed, nw, rows, cols, scales, zeros, ngroups,
                                    groupsize, y, ldy, maxmt, s);
    }
  }
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
