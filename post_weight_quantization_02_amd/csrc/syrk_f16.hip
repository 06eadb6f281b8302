// H += alpha * X^T X for token-major fp16 X (tokens x d), fp32 result.
//
// The Hessian of the layer-output error is 2 X X^T with X feature-major
// ("GPTQ: fixing errors as you go", "Objective"); calibration batches are
// added one after another ("GPTQ-style round-to-nearest with Hessian
// weighting", collect_hessian listing).
//
// gfx950 design:
//   * Output tiles of 128x128 over the lower triangle only; the upper
//     triangle is written by mirroring in the reduction kernel.
//   * The token (K) range is split so the grid holds several waves of
//     workgroups per CU; every split writes its own fp32 partial tile and a
//     second kernel sums the partials in a fixed order (bitwise reproducible,
//     no float atomics).
//   * X arrives token-major (channels contiguous) but MFMA wants each lane to
//     hold a run of consecutive K (token) values.  Each thread loads a
//     4-token x 8-channel block with 16-byte loads, transposes it in
//     registers and stores four-token runs into a channel-major LDS tile.
//   * v_mfma_f32_16x16x32_f16: each of the 4 waves owns a 64x64 quadrant
//     (4x4 MFMA tiles); fp16 products are exact in fp32 and accumulate in
//     fp32.
#include "common.h"

namespace gptq {

namespace {

constexpr int T = kSyrkTile;   // 128
constexpr int KC = 32;         // tokens per K chunk
constexpr int PITCH = KC + 8;  // halves per LDS row (80 bytes: conflict-free 16B reads)

struct Chunk {
  uint32_t r[4][4];  // [token][channel pair]
};

template <bool VEC>
__device__ inline void load_chunk(const _Float16* __restrict__ X, int64_t ldx, int d, int64_t t0,
                                  int64_t tend, int c0, Chunk& ch) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t tok = t0 + t;
    if (VEC) {
      if (tok < tend && c0 + 8 <= d) {
        const uint4 v = *reinterpret_cast<const uint4*>(X + tok * ldx + c0);
        ch.r[t][0] = v.x;
        ch.r[t][1] = v.y;
        ch.r[t][2] = v.z;
        ch.r[t][3] = v.w;
        continue;
      }
    }
    const uint16_t* xs = reinterpret_cast<const uint16_t*>(X);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t lo = 0, hi = 0;
      if (tok < tend && c0 + 2 * p < d) lo = xs[tok * ldx + c0 + 2 * p];
      if (tok < tend && c0 + 2 * p + 1 < d) hi = xs[tok * ldx + c0 + 2 * p + 1];
      ch.r[t][p] = lo | (hi << 16);
    }
  }
}

// Write the 4x8 block channel-major: channel c gets tokens t..t+3 as 8 bytes.
__device__ inline void store_chunk(_Float16* __restrict__ s, int cl, int tq, const Chunk& ch) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t l0 = (ch.r[0][p] & 0xffffu) | (ch.r[1][p] << 16);
    const uint32_t l1 = (ch.r[2][p] & 0xffffu) | (ch.r[3][p] << 16);
    const uint32_t h0 = (ch.r[0][p] >> 16) | (ch.r[1][p] & 0xffff0000u);
    const uint32_t h1 = (ch.r[2][p] >> 16) | (ch.r[3][p] & 0xffff0000u);
    *reinterpret_cast<uint2*>(s + (cl + 2 * p) * PITCH + tq) = make_uint2(l0, l1);
    *reinterpret_cast<uint2*>(s + (cl + 2 * p + 1) * PITCH + tq) = make_uint2(h0, h1);
  }
}

template <bool VEC>
__global__ __launch_bounds__(256) void syrk_partial_kernel(const _Float16* __restrict__ X,
                                                           int64_t ldx, int d, int64_t n,
                                                           int64_t kper, float* __restrict__ P) {
  __shared__ __attribute__((aligned(16))) _Float16 sA[2][T * PITCH];
  __shared__ __attribute__((aligned(16))) _Float16 sB[2][T * PITCH];

  const int ntiles = gridDim.x;
  const int tile = blockIdx.x;
  const int split = blockIdx.y;
  int bi, bj;
  lower_tile(tile, bi, bj);
  const bool diag = (bi == bj);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const int64_t kbeg = (int64_t)split * kper;
  const int64_t kend = (kbeg + kper < n) ? kbeg + kper : n;

  // loader role: 128 tasks per operand block (8 token quads x 16 channel octets)
  const bool loadB = tid >= 128;
  const int task = tid & 127;
  const int tq = (task & 7) * 4;   // token offset within the chunk
  const int cl = (task >> 3) * 8;  // channel offset within the tile
  const int cbase = (loadB ? bj : bi) * T;
  const bool active_loader = !(loadB && diag);

  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  Chunk ch;
  const int64_t nk = (kend > kbeg) ? ceil_div(kend - kbeg, KC) : 0;
  if (nk > 0) {
    if (active_loader) {
      load_chunk<VEC>(X, ldx, d, kbeg + tq, kend, cbase + cl, ch);
      store_chunk(loadB ? sB[0] : sA[0], cl, tq, ch);
    }
    __syncthreads();
  }
  int buf = 0;
  for (int64_t kc = 0; kc < nk; ++kc) {
    const bool more = (kc + 1 < nk);
    if (more && active_loader) load_chunk<VEC>(X, ldx, d, kbeg + (kc + 1) * KC + tq, kend, cbase + cl, ch);

    const _Float16* a_s = sA[buf];
    const _Float16* b_s = diag ? sA[buf] : sB[buf];
    const int koff = 8 * (lane >> 4);
    half8 af[4], bf[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
      af[m] = *reinterpret_cast<const half8*>(a_s + (64 * wm + 16 * m + (lane & 15)) * PITCH + koff);
#pragma unroll
    for (int m = 0; m < 4; ++m)
      bf[m] = *reinterpret_cast<const half8*>(b_s + (64 * wn + 16 * m + (lane & 15)) * PITCH + koff);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[a], bf[b], acc[a][b], 0, 0, 0);

    if (more && active_loader) store_chunk(loadB ? sB[buf ^ 1] : sA[buf ^ 1], cl, tq, ch);
    __syncthreads();
    buf ^= 1;
  }

  // partial tile, row-major 128x128
  float* out = P + ((int64_t)split * ntiles + tile) * (T * T);
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 64 * wm + 16 * a + 4 * (lane >> 4) + i;
        const int c = 64 * wn + 16 * b + (lane & 15);
        out[r * T + c] = acc[a][b][i];
      }
}

// Sum the split partials of one 64x64 quarter of a lower tile in split
// order, add alpha * sum into H, and mirror into the upper triangle.
__global__ __launch_bounds__(256) void syrk_reduce_kernel(const float* __restrict__ P, int d,
                                                          int splits, int ntiles, float alpha,
                                                          float* __restrict__ H) {
  __shared__ float st[64][65];
  const int tile = blockIdx.x;
  const int q = blockIdx.y;  // quarter: (qr, qc)
  const int qr = q >> 1, qc = q & 1;
  int bi, bj;
  lower_tile(tile, bi, bj);
  if (bi == bj && qr < qc) return;  // strictly upper quarter of a diagonal tile
  const int tid = threadIdx.x;
  const int cx = tid & 63;
  const int ry = tid >> 6;
  const int gr0 = bi * T + 64 * qr;
  const int gc0 = bj * T + 64 * qc;
  const bool on_diag = (bi == bj && qr == qc);
  for (int rr = ry; rr < 64; rr += 4) {
    const int lr = 64 * qr + rr, lc = 64 * qc + cx;
    float v = 0.f;
    for (int s = 0; s < splits; ++s) v += P[((int64_t)s * ntiles + tile) * (T * T) + lr * T + lc];
    v *= alpha;
    st[rr][cx] = v;
    const int gr = gr0 + rr, gc = gc0 + cx;
    if (gr < d && gc < d && (!on_diag || gc <= gr)) H[(int64_t)gr * d + gc] += v;
  }
  __syncthreads();
  // mirror: element (gr, gc) with gr > gc goes to H[gc][gr]
  for (int rr = ry; rr < 64; rr += 4) {
    const int gr = gr0 + cx;  // source row (lower)
    const int gc = gc0 + rr;  // source column
    const float v = st[cx][rr];
    if (gr < d && gc < d && gr > gc) H[(int64_t)gc * d + gr] += v;
  }
}

}  // namespace

int syrk_splits(int64_t d, int64_t n) {
  const int64_t nb = ceil_div(d, T);
  const int64_t tiles = nb * (nb + 1) / 2;
  const int64_t chunks = ceil_div(n, KC);
  int64_t s = ceil_div(2048, tiles);
  if (s > chunks) s = chunks;
  if (s < 1) s = 1;
  return (int)s;
}

int64_t syrk_kper(int64_t n, int splits) {
  const int64_t chunks = ceil_div(n, KC);
  return ceil_div(chunks, splits) * KC;
}

hipError_t launch_syrk_partial(const _Float16* X, int64_t ldx, int d, int64_t n, int splits,
                               int64_t kper, float* P, hipStream_t s) {
  const int nb = (int)ceil_div(d, T);
  const int tiles = nb * (nb + 1) / 2;
  dim3 grid(tiles, splits);
  const bool vec = (ldx % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0);
  if (vec)
    hipLaunchKernelGGL(syrk_partial_kernel<true>, grid, dim3(256), 0, s, X, ldx, d, n, kper, P);
  else
    hipLaunchKernelGGL(syrk_partial_kernel<false>, grid, dim3(256), 0, s, X, ldx, d, n, kper, P);
  return hipGetLastError();
}

hipError_t launch_syrk_reduce(const float* P, int d, int splits, float alpha, float* H,
                              hipStream_t s) {
  const int nb = (int)ceil_div(d, T);
  const int tiles = nb * (nb + 1) / 2;
  hipLaunchKernelGGL(syrk_reduce_kernel, dim3(tiles, 4), dim3(256), 0, s, P, d, splits, tiles,
                     alpha, H);
  return hipGetLastError();
}

}  // namespace gptq
