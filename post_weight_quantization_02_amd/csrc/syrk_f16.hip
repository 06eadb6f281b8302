// H += alpha * X^T X for token-major fp16 X (tokens x d), fp32 result.
//
// The Hessian of the layer-output error is 2 X X^T with X feature-major
// ("GPTQ: fixing errors as you go", "Objective"); calibration batches are
// added one after another ("GPTQ-style round-to-nearest with Hessian
// weighting", collect_hessian listing).
//
// gfx950 design:
//   * 256x256 output tiles over the lower triangle only (the upper triangle
//     is written by mirroring in the reduction kernel).  Four waves, each
//     owning a 128x128 quadrant as 8x8 tiles of v_mfma_f32_16x16x32_f16
//     (256 fp32 accumulators per lane): 0.5 LDS fragment reads per MFMA keeps
//     LDS traffic well under its bandwidth at full MFMA rate.
//   * X chunks of 32 tokens go into LDS exactly as they sit in HBM
//     (token-major).  MFMA wants each lane to hold a run of K (token) values
//     for one channel; gfx950's transposing LDS read ds_read_b64_tr_b16
//     delivers exactly that from the token-major tile: in every 16-lane
//     group, lane s addresses row s/4, columns 4*(s%4).., and lane i receives
//     channel i at four consecutive rows.  Two such reads give the 8-token run
//     of a 16x16x32 operand.
//   * Fast path (whole 256x256 tiles, whole chunks, 16-byte aligned X):
//     global_load_lds_dwordx4 straight into a 4-stage LDS ring with an XOR
//     swizzle, explicit vmcnt waits and a bare barrier (see fast_body).
//     General path (ragged d or n, unaligned X): register-staged, double-
//     buffered LDS with padded rows.
//   * The token range is split so the grid fills every CU for several rounds
//     (at most 4096 tokens per split: a split sums in fp32); each split
//     writes its own fp32 partial tile and a second kernel sums the partials
//     in a fixed order in fp64 (bitwise reproducible, no float atomics).
//   * fp16 products are exact in fp32; accumulation is fp32.
#include "common.h"

namespace gptq {

namespace {

constexpr int T = kSyrkTile;     // 256
constexpr int KC = 32;           // tokens per K chunk
constexpr int PITCH = T + 16;    // halves per LDS row (544 bytes = 136 dwords: rows 8 banks apart)
constexpr int NLOAD = (KC * T * 2) / (16 * 256);  // 16-byte loads per thread per operand block

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// 8 consecutive tokens (rows kb..kb+7 of the LDS tile) of channel c0 + (lane % 16),
// as the K run of a 16x16x32 MFMA operand.
__device__ inline half8 tr_frag(const _Float16* tile, int kb, int c0, int lane) {
  const int s = lane & 15;
  const _Float16* p0 = tile + (kb + (s >> 2)) * PITCH + c0 + 4 * (s & 3);
  const _Float16* p1 = p0 + 4 * PITCH;
  // whole-vector bit casts (casting single elements of the result mis-lowers)
  const f16x4 lo = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0));
  const f16x4 hi = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p1));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Partial tiles are stored sub-block by sub-block: the 64x64 sub-block
// (r / 64, c / 64) of a 256x256 tile is one contiguous run of 4096 floats,
// row-major, so the reduction streams 16 KB runs.  Diagonal tiles skip their
// six strictly upper sub-blocks, which nothing reads.
__device__ inline int64_t part_index(int r, int c) {
  return (int64_t)(((r >> 6) * 4 + (c >> 6)) * 4096 + (r & 63) * 64 + (c & 63));
}

// Chunk layout: 32 rows (tokens) x 256 channels = 1024 16-byte pieces per
// operand block; thread t takes pieces t, t+256, ... (row = piece / 32).
template <bool VEC>
__device__ inline void load_block(const _Float16* __restrict__ X, int64_t ldx, int d,
                                  int64_t t0, int64_t tend, int c0, uint4 (&v)[NLOAD], int tid) {
#pragma unroll
  for (int q = 0; q < NLOAD; ++q) {
    const int piece = tid + 256 * q;
    const int r = piece >> 5, cp = (piece & 31) * 8;
    const int64_t tok = t0 + r;
    const int c = c0 + cp;
    uint4 u = make_uint4(0, 0, 0, 0);
    if (tok < tend) {
      if (VEC && c + 8 <= d) {
        u = *reinterpret_cast<const uint4*>(X + tok * ldx + c);
      } else {
        const uint16_t* xs = reinterpret_cast<const uint16_t*>(X) + tok * ldx;
        uint32_t w[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t lo = (c + 2 * p < d) ? xs[c + 2 * p] : 0u;
          const uint32_t hi = (c + 2 * p + 1 < d) ? xs[c + 2 * p + 1] : 0u;
          w[p] = lo | (hi << 16);
        }
        u = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
    v[q] = u;
  }
}

__device__ inline void store_block(_Float16* __restrict__ s, const uint4 (&v)[NLOAD], int tid) {
#pragma unroll
  for (int q = 0; q < NLOAD; ++q) {
    const int piece = tid + 256 * q;
    const int r = piece >> 5, cp = (piece & 31) * 8;
    *reinterpret_cast<uint4*>(s + r * PITCH + cp) = v[q];
  }
}

template <bool VEC>
__global__ __launch_bounds__(256, 1) void syrk_partial_kernel(const _Float16* __restrict__ X,
                                                              int64_t ldx, int d, int64_t n,
                                                              int64_t kper,
                                                              float* __restrict__ P) {
  __shared__ __attribute__((aligned(16))) _Float16 sA[2][KC * PITCH];
  __shared__ __attribute__((aligned(16))) _Float16 sB[2][KC * PITCH];

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
  const int64_t nk = (kend > kbeg) ? ceil_div(kend - kbeg, KC) : 0;

  f32x4 acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 va[NLOAD], vb[NLOAD];
  if (nk > 0) {
    load_block<VEC>(X, ldx, d, kbeg, kend, bi * T, va, tid);
    if (!diag) load_block<VEC>(X, ldx, d, kbeg, kend, bj * T, vb, tid);
    store_block(sA[0], va, tid);
    if (!diag) store_block(sB[0], vb, tid);
    __syncthreads();
  }
  int buf = 0;
  const int kg = 8 * (lane >> 4);  // token run of this lane's 16-lane group
  for (int64_t kc = 0; kc < nk; ++kc) {
    const bool more = kc + 1 < nk;
    if (more) {
      const int64_t t0 = kbeg + (kc + 1) * KC;
      load_block<VEC>(X, ldx, d, t0, kend, bi * T, va, tid);
      if (!diag) load_block<VEC>(X, ldx, d, t0, kend, bj * T, vb, tid);
    }
    const _Float16* a_s = sA[buf];
    const _Float16* b_s = diag ? sA[buf] : sB[buf];
    half8 bf[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) bf[b] = tr_frag(b_s, kg, 128 * wn + 16 * b, lane);
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const half8 af = tr_frag(a_s, kg, 128 * wm + 16 * a, lane);
#pragma unroll
      for (int b = 0; b < 8; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[b], acc[a][b], 0, 0, 0);
    }
    if (more) {
      store_block(sA[buf ^ 1], va, tid);
      if (!diag) store_block(sB[buf ^ 1], vb, tid);
    }
    __syncthreads();
    buf ^= 1;
  }

  // partial tile, sub-block by sub-block (part_index)
  float* out = P + ((int64_t)split * ntiles + tile) * ((int64_t)T * T);
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 128 * wm + 16 * a + 4 * (lane >> 4) + i;
        const int c = 128 * wn + 16 * b + (lane & 15);
        if (!diag || (r >> 6) >= (c >> 6)) out[part_index(r, c)] = acc[a][b][i];
      }
}

// XCD-aware tile order.  Workgroups are handed to the 8 XCDs round-robin by
// linear id, and each XCD has its own L2.  Tiles are listed group-pair by
// group-pair (groups of 4 block rows/columns), and XCD x takes the x-th
// contiguous segment of that list, so the ~17 tiles an XCD works on at once
// share few 256-channel blocks of X and re-read them from its L2.
constexpr int kXcds = 8;
constexpr int kGroup = 4;

__device__ inline void grouped_tile(int idx, int nb, int& bi, int& bj) {
  const int ng = (nb + kGroup - 1) / kGroup;
  for (int gi = 0; gi < ng; ++gi) {
    const int rows = min(kGroup, nb - gi * kGroup);
    for (int gj = 0; gj <= gi; ++gj) {
      const int cols = min(kGroup, nb - gj * kGroup);
      const int cnt = (gi == gj) ? rows * (rows + 1) / 2 : rows * cols;
      if (idx < cnt) {
        int r, c;
        if (gi == gj) {
          lower_tile(idx, r, c);
        } else {
          r = idx / cols;
          c = idx % cols;
        }
        bi = gi * kGroup + r;
        bj = gj * kGroup + c;
        return;
      }
      idx -= cnt;
    }
  }
  bi = bj = -1;
}

// Slot t of a split (grid padded to a multiple of 8 slots) -> tile, or false
// for a padding slot.
__device__ inline bool xcd_tile(int t, int slots, int ntiles, int nb, int& bi, int& bj) {
  const int per = slots / kXcds;
  const int idx = (t % kXcds) * per + t / kXcds;
  if (idx >= ntiles) return false;
  grouped_tile(idx, nb, bi, bj);
  return true;
}

// ------------------------------------------------------------------ fast path
// Interior 256x256 tiles with whole 32-token chunks: every chunk goes from HBM
// straight into LDS with global_load_lds_dwordx4 (no register staging) into a
// ring of NS stages, so several chunks are in flight while one is consumed.
// Rows are 512 bytes, unpadded; the 16-byte pieces of row R are XOR-permuted
// by sw(R) so the 16 rows one transposing read touches (R = 8g + r, g,r < 4)
// use 16 distinct bank groups.
constexpr int NS = 4;                 // LDS ring stages
constexpr int BLK = KC * T;           // halves per operand block per stage

__device__ inline int swz(int row) { return 2 * ((row & 3) | (((row >> 3) & 3) << 2)); }

// Swizzled transposing read: 8 tokens of channel c0 + lane%16 from rows kb..kb+7.
__device__ inline half8 tr_frag_sw(const _Float16* tile, int kb, int c0, int lane) {
  const int s = lane & 15;
  const int r0 = kb + (s >> 2);
  const int q = (c0 >> 3) + ((s & 3) >> 1);
  const int off = 4 * (s & 1);
  const _Float16* p0 = tile + r0 * T + 8 * (q ^ swz(r0)) + off;
  const _Float16* p1 = p0 + 4 * T;  // rows r0 + 4 share r0's swizzle
  const f16x4 lo = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0));
  const f16x4 hi = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p1));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Issue the direct loads of one 32 x 256 operand block: 16 wave instructions
// of two rows each; wave w issues row pairs w, w+4, w+8, w+12.
__device__ inline void issue_block(const _Float16* __restrict__ X, int64_t ldx, int64_t t0,
                                   int c0, _Float16* dst, int wave, int lane) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int rp = wave + 4 * u;
    const int row = 2 * rp + (lane >> 5);
    const int ql = (lane & 31) ^ swz(row);
    const _Float16* g = X + (t0 + row) * ldx + c0 + 8 * ql;
    __builtin_amdgcn_global_load_lds((const void*)g,
                                     (__attribute__((address_space(3))) void*)(dst + rp * 2 * T),
                                     16, 0, 0);
  }
}

// s_waitcnt immediate: vmcnt <= n, expcnt and lgkmcnt unconstrained (gfx9 encoding)
template <int N>
__device__ inline void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ inline void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Chunks k = 0..nk-1 of 32 tokens flow through an LDS ring of NS stages:
// direct loads for chunk k+NS-1 are issued right after the barrier that
// publishes chunk k, so up to NS-1 chunks are in flight while one is
// consumed.  Before that barrier each wave waits only for its own loads of
// stage k (vmcnt) -- the LDS reads of stage k-1 have already been consumed by
// its MFMAs -- so a bare s_barrier suffices; __syncthreads() would also
// drain the loads still in flight.
template <bool DIAG>
__device__ inline void fast_body(const _Float16* __restrict__ X, int64_t ldx, int64_t kbeg,
                                 int64_t nk, int ca, int cb, _Float16* ring, f32x4 (&acc)[8][8],
                                 int wave, int lane, int wm, int wn) {
  constexpr int LPS = DIAG ? 4 : 8;  // direct loads per stage per wave
  for (int64_t k = 0; k < NS - 1 && k < nk; ++k) {
    _Float16* st = ring + (int)(k % NS) * 2 * BLK;
    issue_block(X, ldx, kbeg + k * KC, ca, st, wave, lane);
    if (!DIAG) issue_block(X, ldx, kbeg + k * KC, cb, st + BLK, wave, lane);
  }
  const int kg = 8 * (lane >> 4);
  for (int64_t k = 0; k < nk; ++k) {
    // stage k must have landed; stages k+1, k+2 may still be in flight
    if (k + 2 < nk) wait_vm<2 * LPS>();
    else if (k + 1 < nk) wait_vm<LPS>();
    else wait_vm<0>();
    lds_barrier();
    if (k + NS - 1 < nk) {
      const int64_t kn = k + NS - 1;
      _Float16* st = ring + (int)(kn % NS) * 2 * BLK;
      issue_block(X, ldx, kbeg + kn * KC, ca, st, wave, lane);
      if (!DIAG) issue_block(X, ldx, kbeg + kn * KC, cb, st + BLK, wave, lane);
    }
    const _Float16* a_s = ring + (int)(k % NS) * 2 * BLK;
    const _Float16* b_s = DIAG ? a_s : a_s + BLK;
    half8 bf[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) bf[b] = tr_frag_sw(b_s, kg, 128 * wn + 16 * b, lane);
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const half8 af = tr_frag_sw(a_s, kg, 128 * wm + 16 * a, lane);
#pragma unroll
      for (int b = 0; b < 8; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[b], acc[a][b], 0, 0, 0);
    }
  }
}

__global__ __launch_bounds__(256, 1) void syrk_fast_kernel(const _Float16* __restrict__ X,
                                                           int64_t ldx, int64_t n, int64_t kper,
                                                           int nb, float* __restrict__ P) {
  __shared__ __attribute__((aligned(16))) _Float16 ring[NS * 2 * BLK];
  const int ntiles = nb * (nb + 1) / 2;
  const int split = blockIdx.y;
  int bi, bj;
  if (!xcd_tile(blockIdx.x, gridDim.x, ntiles, nb, bi, bj)) return;
  const int tile = bi * (bi + 1) / 2 + bj;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t kbeg = (int64_t)split * kper;
  const int64_t kend = (kbeg + kper < n) ? kbeg + kper : n;
  const int64_t nk = (kend > kbeg) ? (kend - kbeg) / KC : 0;  // whole chunks only

  f32x4 acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (bi == bj)
    fast_body<true>(X, ldx, kbeg, nk, bi * T, bj * T, ring, acc, wave, lane, wm, wn);
  else
    fast_body<false>(X, ldx, kbeg, nk, bi * T, bj * T, ring, acc, wave, lane, wm, wn);

  float* out = P + ((int64_t)split * ntiles + tile) * ((int64_t)T * T);
  const bool diag = bi == bj;
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 128 * wm + 16 * a + 4 * (lane >> 4) + i;
        const int c = 128 * wn + 16 * b + (lane & 15);
        if (!diag || (r >> 6) >= (c >> 6)) out[part_index(r, c)] = acc[a][b][i];
      }
}

// Sum the split partials of one 64x64 sub-block of a lower tile in split
// order, in fp64 (one rounding to fp32 per element), add alpha * sum into H,
// and mirror into the upper triangle.  Each thread reads float4 runs of four
// columns; a pass over 16 rows reads 4 KB of one split contiguously.
__global__ __launch_bounds__(256) void syrk_reduce_kernel(const float* __restrict__ P, int d,
                                                          int splits, int ntiles, float alpha,
                                                          float* __restrict__ H) {
  constexpr int SB = T / 64;  // sub-blocks per tile edge
  __shared__ float st[64][65];
  const int tile = blockIdx.x;
  const int q = blockIdx.y;
  const int qr = q / SB, qc = q % SB;
  int bi, bj;
  lower_tile(tile, bi, bj);
  if (bi == bj && qr < qc) return;  // strictly upper sub-block of a diagonal tile
  const int tid = threadIdx.x;
  const int gr0 = bi * T + 64 * qr;
  const int gc0 = bj * T + 64 * qc;
  if (gr0 >= d || gc0 >= d) return;
  const bool on_diag = (bi == bj && qr == qc);
  const int c4 = (tid & 15) * 4;
  const int64_t stride = (int64_t)ntiles * T * T;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int rr = 16 * pass + (tid >> 4);
    const float* src = P + (int64_t)tile * T * T + part_index(64 * qr + rr, 64 * qc + c4);
    double v0 = 0.0, v1 = 0.0, v2 = 0.0, v3 = 0.0;
    // eight splits' loads in flight at a time; the sums stay in split order
    int sp = 0;
    for (; sp + 8 <= splits; sp += 8) {
      float4 p[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) p[u] = *reinterpret_cast<const float4*>(src + (sp + u) * stride);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        v0 += (double)p[u].x;
        v1 += (double)p[u].y;
        v2 += (double)p[u].z;
        v3 += (double)p[u].w;
      }
    }
    for (; sp < splits; ++sp) {
      const float4 p = *reinterpret_cast<const float4*>(src + sp * stride);
      v0 += (double)p.x;
      v1 += (double)p.y;
      v2 += (double)p.z;
      v3 += (double)p.w;
    }
    const float o[4] = {(float)((double)alpha * v0), (float)((double)alpha * v1),
                        (float)((double)alpha * v2), (float)((double)alpha * v3)};
    const int gr = gr0 + rr;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      st[rr][c4 + u] = o[u];
      const int gc = gc0 + c4 + u;
      if (gr < d && gc < d && (!on_diag || gc <= gr)) H[(int64_t)gr * d + gc] += o[u];
    }
  }
  __syncthreads();
  const int cx = tid & 63, ry = tid >> 6;
  for (int rr = ry; rr < 64; rr += 4) {
    const int gr = gr0 + cx;  // source row (lower)
    const int gc = gc0 + rr;  // source column
    const float v = st[cx][rr];
    if (gr < d && gc < d && gr > gc) H[(int64_t)gc * d + gr] += v;
  }
}

}  // namespace

int syrk_splits(int64_t d, int64_t n) {
  // One 256x256 workgroup runs per CU at a time.  Pick the split count that
  // minimises (rounds of 256 workgroups) x (time of one split) plus the time
  // to write and re-read the fp32 partial tiles, with at most kMaxSplitChunks
  // chunks (4096 tokens) per split.  A partial sums its products in fp32, so
  // H's error grows with the tokens per split: at 262144 tokens of the
  // attention stream, 8192-token splits leave H 1.0e-7 from the exact sum
  // (Frobenius, relative) and Hinv 3.1e-6, 4096-token splits 6.6e-8 and
  // 1.8e-6.  The larger error moves late group scales of an 11008-row
  // layer up to 1.4e-5 (relative) from the exact-arithmetic result, past
  // the 1e-5 the quantizer's outputs are held to; the smaller one 8.0e-6.
  const int64_t nb = ceil_div(d, T);
  const int64_t tiles = nb * (nb + 1) / 2;
  const int64_t chunks = ceil_div(n, KC);
  const double t_tile = 2.0 * T * T * (double)(chunks * KC) / (4.0 * 1024.0 * 2.4e9);
  const double t_part = (double)T * T * 4.0 * 2.0 / 6.0e12;
  constexpr int64_t kMaxSplitChunks = 128;
  constexpr int64_t kMaxSplits = 128;
  int64_t lo = ceil_div(chunks, kMaxSplitChunks);
  if (lo < 1) lo = 1;
  if (lo > kMaxSplits) lo = kMaxSplits;
  int64_t best = lo;
  double best_cost = 1e30;
  for (int64_t s = lo; s <= kMaxSplits && s <= chunks; ++s) {
    const double rounds = (double)ceil_div(tiles * s, 256);
    const double cost = rounds * t_tile / (double)s + (double)(s * tiles) * t_part;
    if (cost < best_cost) {
      best_cost = cost;
      best = s;
    }
  }
  return (int)best;
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
  if (vec && d % T == 0 && n % KC == 0)
    hipLaunchKernelGGL(syrk_fast_kernel, dim3((unsigned)round_up(tiles, kXcds), splits), dim3(256),
                       0, s, X, ldx, n, kper, nb, P);
  else if (vec)
    hipLaunchKernelGGL(syrk_partial_kernel<true>, grid, dim3(256), 0, s, X, ldx, d, n, kper, P);
  else
    hipLaunchKernelGGL(syrk_partial_kernel<false>, grid, dim3(256), 0, s, X, ldx, d, n, kper, P);
  return hipGetLastError();
}

hipError_t launch_syrk_reduce(const float* P, int d, int splits, float alpha, float* H,
                              hipStream_t s) {
  const int nb = (int)ceil_div(d, T);
  const int tiles = nb * (nb + 1) / 2;
  hipLaunchKernelGGL(syrk_reduce_kernel, dim3(tiles, (T / 64) * (T / 64)), dim3(256), 0, s, P, d,
                     splits, tiles, alpha, H);
  return hipGetLastError();
}

}  // namespace gptq
