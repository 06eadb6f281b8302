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
//   * Step j: all 16 lanes of a row quantize column j themselves from its
//     current value (held identically in every lane), so the dependency
//     chain from one column to the next is five operations with no
//     cross-lane step on it; the owner's copy of the next column arrives by
//     DPP broadcast a step earlier (see sweep_step).  Hinv's 128x128
//     diagonal block is in LDS row by row.
//   * The columns of later 16-column groups take a group's errors at the
//     end of the group or during the next group's steps, in step order.
//   * Operand loads are branch-free (clamped addresses, masks at the point
//     of use), so a tile's loads are all in flight together.
//   * Group min/max is a per-lane reduction followed by a 4-step xor shuffle
//     across the 16 lanes of the row.
//   * Per-column loss partials are reduced inside the workgroup and written
//     per workgroup; a final kernel adds them in a fixed order.
//   * With groups inside blocks, the workgroup first applies to its rows the
//     errors of the earlier blocks of the same superblock (fp32 MFMA, one
//     128x128 Hinv tile at a time through LDS), so no separate launch carries
//     them.
//
// The lazy update W[:, c0:c1] -= Err[:, k0:k1] Hinv[k0:k1, c0:c1] is an fp32
// MFMA GEMM (v_mfma_f32_16x16x4_f32) on (32*MT)x128 output tiles, K streamed
// through double-buffered LDS in chunks of 32.
#include "common.h"

#include <utility>

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

// Row min/max of the current group across the 16 lanes of a row and the
// resulting grid; lane 0 of the row records it.
__device__ inline void group_stats(float mn, float mx, float qm, float& s, float& z, float& rs,
                                   bool rv, int l, int64_t row, int64_t ngroups, int64_t gi,
                                   float* __restrict__ scales, float* __restrict__ zeros) {
  row_minmax(mn, mx);
  grid_params(mn, mx, qm, s, z);
  rs = 1.0f / s;
  if (rv && l == 0) {
    scales[row * ngroups + gi] = s;
    zeros[row * ngroups + gi] = z;
  }
}

// Value of `v` held by lane `src + 16*rg` of the wave, for each lane's row
// group rg (src is wave-uniform): four readlanes combined with the lane's 0/1
// row-group masks (branch-free; exact because each product is v or 0).
// Value of v held by lane LJ of this lane's row of 16 (DPP row_newbcast):
// each row of 16 lanes is one row of W, so this is the owner's value.
template <int LJ>
__device__ inline float row_bcast(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + LJ, 0xF, 0xF, true));
}

// Column step j = 16*kj + LJ of the sweep for this lane's row (see
// sweep_columns).
//
// Every lane of the row quantizes column j itself, from c, the column's
// current value (the same in all 16 lanes), so no broadcast sits on the
// dependency chain, which is five operations: t = c/s + z as one fused
// multiply-add with 1/s, rint, the clamp to [0, qm] (med3), the scaled error
// e = (c - (q - z) s) / Hinv[j][j] as two fused multiply-adds (the first one,
// off the chain, of c alone), and the next column's value
// c' = bn - e Hinv[j][j+1].  bn is column j+1 with every earlier step's
// update, broadcast from its owner one step earlier.  The owner's register
// receives the same update, so c' equals the owner's copy bit for bit.
// Registers kj and kj+1 are updated here (the next broadcasts read them).
// The later groups' columns take a group's 16 errors in step order
// elsewhere: register kj+2 at the end of the group (group_tail), registers
// kj+3.. during the next group's steps (lag: step LJ of group kj applies
// error LJ of group kj-1, egp, to registers kj+2..), where those multiply-adds
// fill issue slots the dependency chain leaves free.
template <int LJ>
__device__ inline void sweep_step(int kj, int l, float s, float z, float rs, float qm,
                                  const float* __restrict__ urow, const float* __restrict__ rdg,
                                  float (&w)[CPL], float& c, float& bn, float& rdj, float& ujn,
                                  float& u0, float& u1, float (&eg)[RL], float (&qc)[CPL],
                                  float (&ev)[CPL], bool lag, const float* __restrict__ uprev,
                                  const float (&egp)[RL]) {
  constexpr int J1 = LJ + 1;
  // the previous group's row LJ for the lagged updates
  float ul[CPL];
#pragma unroll
  for (int k = 0; k < CPL; ++k) ul[k] = (lag && k >= kj + 2) ? uprev[LJ * BC + l + RL * k] : 0.f;
  // the next step's Hinv entries: its row of this lane's columns in
  // registers kj and kj+1, and the shared 1 / Hinv[j][j] and Hinv[j][j+1]
  const float* ujn1 = urow + J1 * BC;
  const float u0n = (J1 < RL) ? ujn1[l + RL * kj] : 0.f;
  const float u1n = (J1 < RL && kj + 1 < CPL) ? ujn1[l + RL * (kj + 1)] : 0.f;
  const float rdn = (J1 < RL) ? rdg[J1] : 0.f;
  const bool nx = J1 < RL && RL * kj + J1 + 1 < BC;  // the next step's U[j+1][j+2] exists
  const float ujnn = nx ? urow[J1 * BC + RL * kj + J1 + 1] : 0.f;
  const float srd = s * rdj;
  const float zsrd = z * srd;
  const float t = __builtin_fmaf(c, rs, z);
  const float q = __builtin_amdgcn_fmed3f(rintf(t), 0.f, qm);
  const float xr = __builtin_fmaf(c, rdj, zsrd);
  const float eb = __builtin_fmaf(-q, srd, xr);
  c = __builtin_fmaf(-eb, ujn, bn);
  eg[LJ] = eb;
  if (l == LJ) {
    qc[kj] = q;
    ev[kj] = eb;
  }
  w[kj] = __builtin_fmaf(-eb, u0, w[kj]);
  if (kj + 1 < CPL) w[kj + 1] = __builtin_fmaf(-eb, u1, w[kj + 1]);
  if (lag) {
#pragma unroll
    for (int k = 0; k < CPL; ++k)
      if (k >= kj + 2) w[k] = __builtin_fmaf(-egp[LJ], ul[k], w[k]);
  }
  // column j + 2 after this step, for the step after next
  if constexpr (LJ + 2 < RL)
    bn = row_bcast<LJ + 2>(w[kj]);
  else
    bn = (kj + 1 < CPL) ? row_bcast<LJ + 2 - RL>(w[kj + 1 < CPL ? kj + 1 : kj]) : 0.f;
  rdj = rdn;
  ujn = ujnn;
  u0 = u0n;
  u1 = u1n;
  __builtin_amdgcn_sched_barrier(0);  // keep steps apart: bounded register pressure
}

template <int... LJ>
__device__ inline void sweep_steps(int kj, int l, float s, float z, float rs, float qm,
                                   const float* __restrict__ urow, const float* __restrict__ rdg,
                                   float (&w)[CPL], float& c, float& bn, float& rdj, float& ujn,
                                   float& u0, float& u1, float (&eg)[RL], float (&qc)[CPL],
                                   float (&ev)[CPL], bool lag, const float* __restrict__ uprev,
                                   const float (&egp)[RL], std::integer_sequence<int, LJ...>) {
  (sweep_step<LJ>(kj, l, s, z, rs, qm, urow, rdg, w, c, bn, rdj, ujn, u0, u1, eg, qc, ev, lag,
                  uprev, egp),
   ...);
}

// End of group kj: registers kj+2 .. kmax-1 take the group's 16 errors,
// w[k] -= sum_j eg[j] Hinv[16 kj + j][16 k + l] in step order (register kj+1
// was updated step by step; registers kmax.. take them during the next
// group's steps).  The empty asm statements pin each updated w[k] here:
// otherwise the compiler defers these updates to the group that first reads
// w[k] and keeps every earlier group's errors alive until then (hundreds of
// registers).
__device__ inline void group_tail(int kj, int kmax, int l, const float* __restrict__ urow,
                                  float (&w)[CPL], const float (&eg)[RL]) {
#pragma unroll
  for (int k = kj + 2; k < CPL; ++k) {
    if (k >= kmax) break;
#pragma unroll
    for (int j = 0; j < RL; ++j) w[k] = __builtin_fmaf(-eg[j], urow[j * BC + l + RL * k], w[k]);
    asm volatile("" : "+v"(w[k]));
  }
}

// Loads of a block's operands are branch-free: each reads from an address
// clamped into the matrix and the value is masked only where it is consumed.
// A load under a condition makes the compiler wait for it at the join of the
// branches, so the loads of a tile would not be in flight together.

// Hinv[r0 + j][c0 + c] for the 16 float4 this thread moves into a 128x128
// LDS tile (row j at U + 128 j), raw: the row is clamped below r0 + nrows and
// the column below c0 + nbc (both inside the matrix).  VEC: cols % 4 == 0 and
// Hinv 16-byte aligned, so nbc % 4 == 0 and each float4 lies wholly inside
// or wholly outside the block's columns.
template <bool VEC>
__device__ inline void hinv_tile_fetch(float4 (&v)[16], const float* __restrict__ Hinv,
                                       int64_t cols, int64_t r0, int c0, int nbc, int nrows,
                                       int tid) {
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int e = tid + 256 * q;  // float4 index: row e/32, columns 4*(e%32)..
    const int j = e >> 5, c = (e & 31) * 4;
    const float* p = Hinv + (r0 + (j < nrows ? j : nrows - 1)) * cols + c0;
    if constexpr (VEC) {
      v[q] = *reinterpret_cast<const float4*>(p + (c < nbc ? c : nbc - 4));
    } else {
      const int cl = nbc - 1;
      v[q].x = p[c < cl ? c : cl];
      v[q].y = p[c + 1 < cl ? c + 1 : cl];
      v[q].z = p[c + 2 < cl ? c + 2 : cl];
      v[q].w = p[c + 3 < cl ? c + 3 : cl];
    }
  }
}

// The fetched tile into LDS with the entries outside rows < nrows and
// columns < nbc zeroed.  With TRI (the block's own diagonal tile) the part
// left of the diagonal is zeroed too, and rdiag[j] = 1 / Hinv[j][j] for the
// block's columns (0 past the last one) comes from the same registers.
template <bool TRI>
__device__ inline void hinv_tile_put(float* __restrict__ U, float* __restrict__ rdiag,
                                     const float4 (&v)[16], int nbc, int nrows, int tid) {
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int e = tid + 256 * q;
    const int j = e >> 5, c = (e & 31) * 4;
    const bool in = j < nrows;
    float4 u = v[q];
    u.x = (in && c + 0 < nbc && (!TRI || c + 0 >= j)) ? u.x : 0.f;
    u.y = (in && c + 1 < nbc && (!TRI || c + 1 >= j)) ? u.y : 0.f;
    u.z = (in && c + 2 < nbc && (!TRI || c + 2 >= j)) ? u.z : 0.f;
    u.w = (in && c + 3 < nbc && (!TRI || c + 3 >= j)) ? u.w : 0.f;
    *reinterpret_cast<float4*>(U + j * BC + c) = u;
    if (TRI) {
      // selects, not a dynamic index (which would put v in scratch memory)
      const int dj = j - c;
      const float d = (dj == 0) ? u.x : (dj == 1) ? u.y : (dj == 2) ? u.z : u.w;
      if (dj >= 0 && dj < 4) rdiag[j] = (j < nbc) ? 1.f / d : 0.f;
    }
  }
}

// Err[row0 + r][c0 + c] for the workgroup's 16 rows x 128 columns, raw (2
// float4 per thread; rows clamped below `rows`); err_slice_put zeroes the
// rows past `rows` on the way to LDS.
__device__ inline void err_slice_fetch(float4 (&v)[2], const float* __restrict__ Err, int64_t ldk,
                                       int64_t rows, int64_t row0, int c0, int tid) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = tid + 256 * q;
    const int64_t r = row0 + (e >> 5);
    const int c = (e & 31) * 4;
    v[q] = *reinterpret_cast<const float4*>(Err + (r < rows ? r : rows - 1) * ldk + c0 + c);
  }
}

constexpr int EP = BC + 4;  // row pitch of the pending-update tile

template <typename F, int... K>
__device__ inline void for_each_group(F& f, std::integer_sequence<int, K...>) {
  (f(std::integral_constant<int, K>{}), ...);
}

// Group statistics, the 128 column steps and the outputs of the block at
// column i1 (nbc columns), for this thread's row: the block's Hinv tile and
// 1 / diagonal are in LDS (Ub, rdiag), its current weights in w.
template <int G>
__device__ __attribute__((always_inline)) inline void sweep_columns(
    float (&w)[CPL], const float* __restrict__ Ub, const float* __restrict__ rdiag,
    float (*lsum)[BC], float* __restrict__ Wk, int64_t ldk,
    int64_t rows, int64_t cols, int i1, int nbc, int bits, int groupsize,
    uint8_t* __restrict__ codes, float* __restrict__ scales, float* __restrict__ zeros,
    float* __restrict__ Err, float* __restrict__ lpart, int tid) {
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l = lane & 15;
  const int rg = lane >> 4;
  const int64_t row = (int64_t)blockIdx.x * kSweepRows + wave * 4 + rg;
  const bool rv = row < rows;
  const int64_t ngroups = ceil_div(cols, groupsize);

  const float qm = (float)((1 << bits) - 1);
  float s = 1.f, z = 0.f, rs = 1.f;
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
      group_stats(mn, mx, qm, s, z, rs, rv, l, row, ngroups, gi, scales, zeros);
    } else if (rv) {
      s = scales[row * ngroups + gi];
      z = zeros[row * ngroups + gi];
      rs = 1.0f / s;
    }
  }

  float qc[CPL], ev[CPL];
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    qc[k] = 0.f;
    ev[k] = 0.f;
  }
  // the row's columns 0 and 1, in every lane of the row
  float c = row_bcast<0>(w[0]);
  float bn = row_bcast<1>(w[0]);
  bool lag = false;  // the previous group's errors still owed to registers kj+2..
  float egp[RL];
#pragma unroll
  for (int j = 0; j < RL; ++j) egp[j] = 0.f;

  // One group of 16 columns; expanded for kj = 0..7 at compile time (a loop
  // this large is not unrolled by the compiler), so every register index is
  // a constant.  Groups past a short last block are skipped.
  auto group = [&](auto kjc) {
    constexpr int kj = decltype(kjc)::value;
    if (RL * kj >= nbc) return;
    if (G != 0 && (RL * kj) % (G > 0 ? G : 1) == 0) {
      // a group starts at column 16*kj: statistics over its current values
      float mn = INFINITY, mx = -INFINITY;
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        const int c = l + RL * k;
        if (k >= kj && k < kj + (G > 0 ? G : RL) / RL && c < nbc) {
          mn = fminf(mn, w[k]);
          mx = fmaxf(mx, w[k]);
        }
      }
      group_stats(mn, mx, qm, s, z, rs, rv, l, row, ngroups, (i1 + RL * kj) / groupsize, scales,
                  zeros);
    }
    const float* urow = Ub + (RL * kj) * BC;
    const float* rdg = rdiag + RL * kj;
    // the group's first step: 1 / Hinv[j][j], Hinv[j][j+1] and this lane's
    // entries of row j in registers kj and kj+1
    float rdj = rdg[0];
    float ujn = urow[RL * kj + 1];
    float u0 = urow[l + RL * kj];
    float u1 = (kj + 1 < CPL) ? urow[l + RL * (kj + 1)] : 0.f;
    float eg[RL];
    sweep_steps(kj, l, s, z, rs, qm, urow, rdg, w, c, bn, rdj, ujn, u0, u1, eg, qc, ev, lag,
                urow - RL * BC, egp, std::make_integer_sequence<int, RL>{});
    // The next group's statistics read registers kj+1 .. kj+G/16: with more
    // than two of them (G >= 64 and a group starting there) every update is
    // applied now; otherwise registers kj+3.. take this group's errors during
    // the next group's steps.
    const bool flush = G >= 64 && (RL * (kj + 1)) % (G > 0 ? G : 1) == 0;
    group_tail(kj, flush ? CPL : kj + 3, l, urow, w, eg);
    lag = !flush;
#pragma unroll
    for (int j = 0; j < RL; ++j) egp[j] = eg[j];
  };
  for_each_group(group, std::make_integer_sequence<int, CPL>{});

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

// Pending errors of the superblock for one block: dacc += E Hinv[c0 block,
// block] for the Hinv tile in Ub and the 16 x 128 error slice E (row pitch
// ep), wave w forming columns 32w..32w+31 of the 16 rows.  Element i of
// dacc[b] at lane (n, q) is row 4q + i, column 32w + 16b + n (the fp32
// 16x16x4 result layout).
__device__ inline void pending_tile_mma(const float* __restrict__ E, int ep,
                                        const float* __restrict__ Ub, f32x4 (&dacc)[2], int lane,
                                        int wave) {
  // the operands of the k-step two ahead are read while this one's products
  // run (held in that order by scheduling barriers): read right before their
  // products, every k-step waited for its own LDS reads
  constexpr int NK = BC / 4;
  const float* ub = Ub + 32 * wave + (lane & 15) + (lane >> 4) * BC;
  const float* ea = E + (lane & 15) * ep + (lane >> 4);
  float a0 = ea[0], a1 = ea[4];
  float b00 = ub[0], b01 = ub[16], b10 = ub[4 * BC], b11 = ub[4 * BC + 16];
#pragma unroll 8
  for (int s4 = 0; s4 < NK; ++s4) {
    const int kn = 4 * ((s4 + 2) & (NK - 1));
    const float an = ea[kn];
    const float bn0 = ub[kn * BC], bn1 = ub[kn * BC + 16];
    dacc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b00, dacc[0], 0, 0, 0);
    dacc[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b01, dacc[1], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x0100, 3, 0);
    __builtin_amdgcn_sched_group_barrier(0x0008, 2, 0);
    a0 = a1;
    b00 = b10;
    b01 = b11;
    a1 = an;
    b10 = bn0;
    b11 = bn1;
  }
}

// w -= the pending update in dacc, through the tile Es.
__device__ inline void apply_pending(float (&w)[CPL], const f32x4 (&dacc)[2], float* __restrict__ Es,
                                     int lane, int wave, int rg, int l) {
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      Es[(4 * (lane >> 4) + i) * EP + 32 * wave + 16 * b + (lane & 15)] = dacc[b][i];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < CPL; ++k) w[k] -= Es[(wave * 4 + rg) * EP + l + RL * k];
}

// One 128-column block at column i1 for the workgroup's 16 rows, one launch
// per block (groups spanning blocks, G == 0; any group size works).  p0 < i1
// (groups inside blocks only): the blocks [p0, i1) of this superblock were
// swept by earlier launches and their errors have not yet been applied to
// this block; the workgroup applies them to its own rows first,
// W[rows, block] -= Err[rows, p0:i1] Hinv[p0:i1, block], one 128x128 Hinv
// tile at a time through LDS and fp32 MFMA.
template <int G, bool VEC>
__global__ __launch_bounds__(256) void sweep_kernel(float* __restrict__ Wk, int64_t ldk,
                                                    int64_t rows, int64_t cols, int i1, int p0,
                                                    const float* __restrict__ Hinv, int bits,
                                                    int groupsize, uint8_t* __restrict__ codes,
                                                    float* __restrict__ scales,
                                                    float* __restrict__ zeros,
                                                    float* __restrict__ Err,
                                                    float* __restrict__ lpart) {
  __shared__ __attribute__((aligned(16))) float Ub[BC * BC];  // Hinv block, row j at Ub + 128 j
  __shared__ float rdiag[BC];
  __shared__ float lsum[4][BC];
  __shared__ __attribute__((aligned(16))) float Es[kSweepRows * EP];  // Err slice / update tile

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l = lane & 15;
  const int rg = lane >> 4;
  const int64_t row = (int64_t)blockIdx.x * kSweepRows + wave * 4 + rg;
  const bool rv = row < rows;
  const int nbc = (int)((cols - i1) < BC ? (cols - i1) : BC);

  // this thread's weights (raw: row and column clamped), masked below
  float wr[CPL];
  {
    const float* wp = Wk + (rv ? row : rows - 1) * ldk + i1;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      const int c = l + RL * k;
      wr[k] = wp[c < nbc ? c : nbc - 1];
    }
  }

  float4 hv[16];  // next Hinv tile on its way to LDS
  f32x4 dacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  const bool pending = G != 0 && p0 < i1;
  if (pending) {
    // the next tile (and finally the block's own diagonal tile) is loaded
    // during each tile's MFMAs
    const int64_t row0 = (int64_t)blockIdx.x * kSweepRows;
    float4 ev4[2];
    hinv_tile_fetch<VEC>(hv, Hinv, cols, p0, i1, nbc, BC, tid);
    err_slice_fetch(ev4, Err, ldk, rows, row0, p0, tid);
    for (int c0 = p0; c0 < i1; c0 += BC) {
      hinv_tile_put<false>(Ub, rdiag, hv, nbc, BC, tid);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int e = tid + 256 * q;
        *reinterpret_cast<float4*>(Es + (e >> 5) * EP + (e & 31) * 4) =
            (row0 + (e >> 5) < rows) ? ev4[q] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      __syncthreads();
      if (c0 + BC < i1) {
        hinv_tile_fetch<VEC>(hv, Hinv, cols, c0 + BC, i1, nbc, BC, tid);
        err_slice_fetch(ev4, Err, ldk, rows, row0, c0 + BC, tid);
      } else {
        hinv_tile_fetch<VEC>(hv, Hinv, cols, i1, i1, nbc, nbc, tid);  // the diagonal tile
      }
      pending_tile_mma(Es, EP, Ub, dacc, lane, wave);
      __syncthreads();  // Ub and Es are refilled next
    }
  } else {
    hinv_tile_fetch<VEC>(hv, Hinv, cols, i1, i1, nbc, nbc, tid);
  }
  float w[CPL];
#pragma unroll
  for (int k = 0; k < CPL; ++k) w[k] = (rv && l + RL * k < nbc) ? wr[k] : 0.f;
  if (pending) apply_pending(w, dacc, Es, lane, wave, rg, l);
  // Hinv[i1:i1+128, i1:i1+128] with the part left of the diagonal (and past
  // the last column) zeroed, and its 1 / diagonal
  hinv_tile_put<true>(Ub, rdiag, hv, nbc, nbc, tid);
  __syncthreads();
  sweep_columns<G>(w, Ub, rdiag, lsum, Wk, ldk, rows, cols, i1, nbc, bits, groupsize, codes, scales,
                   zeros, Err, lpart, tid);
}

// ---------------------------------------------------------------- lazy GEMM
// W[:, c0:c1] -= Err[:, k0:k1] * Hinv[k0:k1, c0:c1]  (fp32, MFMA 16x16x4).
// 128x128 output tiles, 4 waves of 64x64; K streamed in chunks of 32 through
// double-buffered LDS stored k-major (pitch 144 floats: the four k rows an
// operand read touches fall in four different 16-bank groups); the next
// chunk's global loads are issued before the current chunk's MFMAs, and the
// C tile is fetched before the last chunk so its latency overlaps the math.
constexpr int LT = 128;  // output tile edge
constexpr int LK = 32;   // K chunk
constexpr int LP = LT + 16;

// MT: 16x16 MFMA tiles per wave along rows (workgroup tile (32*MT) x 128).
// ALL: K <= 4 chunks, and every chunk's loads and the W tile's loads are
// issued up front (one memory round trip for the whole update instead of
// one per chunk: the small updates inside a superblock are latency-bound).
template <int MT, bool ALL>
__global__ __launch_bounds__(256, 2) void lazy_kernel(float* __restrict__ Wk, int64_t ldk,
                                                   int64_t rows, int64_t cols, int k0, int k1,
                                                   int c0, int c1, const float* __restrict__ Err,
                                                   const float* __restrict__ Hinv) {
  constexpr int TM = 32 * MT;      // rows per workgroup tile
  constexpr int PA = LK + 4;       // A is m-major: a row of 32 k at pitch 36 floats, so
                                   // float4 stores and the operand reads (16 rows x 4 k)
                                   // hit distinct banks
  constexpr int AV = TM * LK / 4 / 256;  // float4 A loads per thread
  __shared__ __attribute__((aligned(16))) float As[2][TM * PA];  // [m][k]
  __shared__ __attribute__((aligned(16))) float Bs[2][LK][LP];   // [k][n]
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t r0 = (int64_t)blockIdx.y * TM;
  const int64_t n0 = (int64_t)c0 + (int64_t)blockIdx.x * LT;
  const int K = k1 - k0;

  f32x4 acc[MT][4];
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Loads read in-bounds addresses unconditionally and keep the raw values;
  // entries past K, past c1 or past the last row are zeroed (or ignored)
  // when the chunk goes to LDS, so no MFMA waits for the next chunk's loads.
  // Whole chunks of tiles inside the rows and columns skip the clamps and
  // masks (vector loads of Hinv when its rows are 16-byte aligned).
  // A = Err[r0.., k0..k1]: the row stride ldk is a multiple of 128 and k0 a
  // multiple of 128, so a whole chunk stays inside each (clamped) row.
  // B = Hinv[k0..k1, n0..]: row and column indices are clamped.
  constexpr int NR = ALL ? 4 : 1;  // register sets of chunk loads in flight
  float4 av[NR][AV], bv[NR][4];
  // uniform: the chunk is whole, the tile inside the rows and columns, and
  // Hinv's rows 16-byte aligned, so loads and LDS stores need no clamps or masks
  const bool vec_b = (reinterpret_cast<uintptr_t>(Hinv) % 16 == 0) && (cols % 4 == 0);
  const bool tile_in = r0 + TM <= rows && n0 + LT <= c1 && vec_b;
  auto whole = [&](int kc) { return tile_in && kc + LK <= K; };
  auto gload = [&](int set, int kc) {
    if (whole(kc)) {
#pragma unroll
      for (int q = 0; q < AV; ++q) {
        const int e = tid + 256 * q;
        const int m = e >> 3, kk = (e & 7) * 4;
        av[set][q] = *reinterpret_cast<const float4*>(Err + (r0 + m) * ldk + k0 + kc + kk);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = tid + 256 * q;
        const int kb = e >> 5, nn = (e & 31) * 4;
        bv[set][q] = *reinterpret_cast<const float4*>(Hinv + (int64_t)(k0 + kc + kb) * cols + n0 + nn);
      }
      return;
    }
#pragma unroll
    for (int q = 0; q < AV; ++q) {
      const int e = tid + 256 * q;
      const int m = e >> 3, kk = (e & 7) * 4;  // A: 8 float4 per row
      const int64_t gr = (r0 + m < rows) ? r0 + m : rows - 1;
      av[set][q] = *reinterpret_cast<const float4*>(Err + gr * ldk + k0 + kc + kk);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + 256 * q;
      const int kb = e >> 5, nn = (e & 31) * 4;  // B: 32 float4 per k-row
      const int krow = min(k0 + kc + kb, k1 - 1);
      const float* p = Hinv + (int64_t)krow * cols;
      const int64_t gc = n0 + nn;
      const int64_t cl = cols - 1;
      bv[set][q] = make_float4(p[gc < cl ? gc : cl], p[gc + 1 < cl ? gc + 1 : cl],
                               p[gc + 2 < cl ? gc + 2 : cl], p[gc + 3 < cl ? gc + 3 : cl]);
    }
  };
  auto lstore = [&](int set, int buf, int kc) {
    if (whole(kc)) {
#pragma unroll
      for (int q = 0; q < AV; ++q) {
        const int e = tid + 256 * q;
        *reinterpret_cast<float4*>(&As[buf][(e >> 3) * PA + (e & 7) * 4]) = av[set][q];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = tid + 256 * q;
        *reinterpret_cast<float4*>(&Bs[buf][e >> 5][(e & 31) * 4]) = bv[set][q];
      }
      return;
    }
#pragma unroll
    for (int q = 0; q < AV; ++q) {
      const int e = tid + 256 * q;
      const int m = e >> 3, kk = (e & 7) * 4;
      const int gk = kc + kk;
      float4 v = av[set][q];
      v.x = (gk + 0 < K) ? v.x : 0.f;
      v.y = (gk + 1 < K) ? v.y : 0.f;
      v.z = (gk + 2 < K) ? v.z : 0.f;
      v.w = (gk + 3 < K) ? v.w : 0.f;
      *reinterpret_cast<float4*>(&As[buf][m * PA + kk]) = v;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + 256 * q;
      const int kb = e >> 5, nn = (e & 31) * 4;
      const bool kv = kc + kb < K;
      const int64_t gc = n0 + nn;
      float4 u = bv[set][q];
      u.x = (kv && gc + 0 < c1) ? u.x : 0.f;
      u.y = (kv && gc + 1 < c1) ? u.y : 0.f;
      u.z = (kv && gc + 2 < c1) ? u.z : 0.f;
      u.w = (kv && gc + 3 < c1) ? u.w : 0.f;
      *reinterpret_cast<float4*>(&Bs[buf][kb][nn]) = u;
    }
  };

  // this lane's output elements: rows rb + 16a + i, columns cb + 16b
  const int64_t rb = r0 + 16 * MT * wm + 4 * (lane >> 4);
  const int64_t cb = n0 + 64 * wn + (lane & 15);
  float* const wbase = Wk + rb * ldk + cb;
  const int ldi = (int)ldk;
  const int nchunks = (K + LK - 1) / LK;
  auto mma_chunk = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < LK; ks += 4) {
      const int kr = ks + (lane >> 4);
      float af[MT], bf[4];
#pragma unroll
      for (int a = 0; a < MT; ++a) af[a] = As[buf][(16 * MT * wm + 16 * a + (lane & 15)) * PA + kr];
#pragma unroll
      for (int b = 0; b < 4; ++b) bf[b] = Bs[buf][kr][64 * wn + 16 * b + (lane & 15)];
#pragma unroll
      for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[a], bf[b], acc[a][b], 0, 0, 0);
    }
  };
  // the W tile this lane updates: rows rb + 16a + i, columns cb + 16b
  float cv[MT][4][4];
  auto wload = [&]() {
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool rv = rb + 16 * a + i < rows;
#pragma unroll
        for (int b = 0; b < 4; ++b) cv[a][i][b] = rv ? wbase[(16 * a + i) * ldi + 16 * b] : 0.f;
      }
  };
  if (ALL) {
    // every chunk (K <= 4 * LK) and the W tile in flight at once
#pragma unroll
    for (int c = 0; c < NR; ++c) gload(c, c * LK);
    wload();
#pragma unroll
    for (int c = 0; c < NR; ++c) {
      if (c < nchunks) {
        lstore(c, c & 1, c * LK);
        __syncthreads();
        mma_chunk(c & 1);
      }
    }
  } else {
    gload(0, 0);
    lstore(0, 0, 0);
    __syncthreads();
    int buf = 0;
    for (int ch = 0; ch < nchunks; ++ch) {
      const bool more = ch + 1 < nchunks;
      if (more) gload(0, (ch + 1) * LK);
      mma_chunk(buf);
      if (more) lstore(0, buf ^ 1, (ch + 1) * LK);
      __syncthreads();
      buf ^= 1;
    }
    wload();
  }
  // W tile update
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool rv = rb + 16 * a + i < rows;
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (rv && cb + 16 * b < c1) wbase[(16 * a + i) * ldi + 16 * b] = cv[a][i][b] - acc[a][b][i];
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

// Act-order variant: Wk[r][j] = W[r][perm[j]] (columns in processing order;
// perm entries clamped into [0, cols)).  One workgroup per row; with `stage`
// the row of W is first copied to LDS (dynamic, cols * sizeof(T) bytes) so
// the gather reads LDS and both global passes are coalesced.
template <typename T>
__global__ __launch_bounds__(256) void convert_perm_kernel(const T* __restrict__ W, int64_t rows,
                                                           int64_t cols, int64_t ldw,
                                                           const int* __restrict__ perm,
                                                           float* __restrict__ Wk, int64_t ldk,
                                                           bool stage) {
  extern __shared__ __attribute__((aligned(16))) uint8_t convert_row[];
  T* rowbuf = reinterpret_cast<T*>(convert_row);
  const int64_t r = blockIdx.x;
  const T* src = W + r * ldw;
  if (stage) {
    for (int64_t c = threadIdx.x; c < cols; c += 256) rowbuf[c] = src[c];
    __syncthreads();
    src = rowbuf;
  }
  const int cmax = (int)(cols - 1);
  for (int64_t c = threadIdx.x; c < ldk; c += 256)
    Wk[r * ldk + c] = (c < cols) ? (float)src[min(max(perm[c], 0), cmax)] : 0.f;
}

// fp16 rows whose start is 16-byte aligned (ldw % 8 == 0): 8 columns per
// thread with one 16-byte load and two 16-byte stores.  ldk is a multiple of
// 128, so every 8-column run of Wk is whole.
__global__ __launch_bounds__(256) void convert_f16x8_kernel(const _Float16* __restrict__ W,
                                                            int64_t cols, int64_t ldw,
                                                            float* __restrict__ Wk, int64_t ldk) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  const int64_t r = blockIdx.x;
  for (int64_t c = ((int64_t)blockIdx.y * 256 + threadIdx.x) * 8; c < ldk;
       c += (int64_t)gridDim.y * 256 * 8) {
    float o[8];
    if (c + 8 <= cols) {
      const h8 v = *reinterpret_cast<const h8*>(W + r * ldw + c);
#pragma unroll
      for (int u = 0; u < 8; ++u) o[u] = (float)v[u];
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) o[u] = (c + u < cols) ? (float)W[r * ldw + c + u] : 0.f;
    }
    float4* dst = reinterpret_cast<float4*>(Wk + r * ldk + c);
    dst[0] = make_float4(o[0], o[1], o[2], o[3]);
    dst[1] = make_float4(o[4], o[5], o[6], o[7]);
  }
}

// losses[c] = sum over parts p of lpart[p][c], in a fixed order: a workgroup
// takes 16 columns; thread (s, c) sums parts s, s+16, ... and the 16 slices
// are added in slice order.
__global__ __launch_bounds__(256) void loss_reduce_kernel(const float* __restrict__ lpart,
                                                          int64_t nparts, int64_t ldk,
                                                          int64_t cols, float* __restrict__ out) {
  __shared__ float part[16][17];
  const int cl = threadIdx.x & 15, sl = threadIdx.x >> 4;
  const int64_t c = (int64_t)blockIdx.x * 16 + cl;
  float acc = 0.f;
  if (c < cols)
    for (int64_t p = sl; p < nparts; p += 16) acc += lpart[p * ldk + c];
  part[sl][cl] = acc;
  __syncthreads();
  if (sl == 0 && c < cols) {
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) tot += part[i][cl];
    out[c] = tot;
  }
}

}  // namespace

hipError_t launch_convert_w(const void* W, int w_dtype, int64_t rows, int64_t cols, int64_t ldw,
                            const int* perm, float* Wk, int64_t ldk, hipStream_t s) {
  dim3 grid((unsigned)rows, (unsigned)((ceil_div(ldk, 256) < 16) ? ceil_div(ldk, 256) : 16));
  if (perm != nullptr) {
    const int64_t rb = cols * (w_dtype == GPTQ_DTYPE_F16 ? 2 : 4);
    const bool stage = rb <= kStageBytes;
    const unsigned lds = stage ? (unsigned)rb : 0u;
    if (w_dtype == GPTQ_DTYPE_F16)
      hipLaunchKernelGGL(convert_perm_kernel<_Float16>, dim3((unsigned)rows), dim3(256), lds, s,
                         reinterpret_cast<const _Float16*>(W), rows, cols, ldw, perm, Wk, ldk,
                         stage);
    else
      hipLaunchKernelGGL(convert_perm_kernel<float>, dim3((unsigned)rows), dim3(256), lds, s,
                         reinterpret_cast<const float*>(W), rows, cols, ldw, perm, Wk, ldk, stage);
    return hipGetLastError();
  }
  const bool v8 = (ldw % 8 == 0) && ((reinterpret_cast<uintptr_t>(W) & 15) == 0) &&
                  ((reinterpret_cast<uintptr_t>(Wk) & 15) == 0);
  if (w_dtype == GPTQ_DTYPE_F16 && v8)
    hipLaunchKernelGGL(convert_f16x8_kernel, dim3((unsigned)rows, (unsigned)ceil_div(ldk, 2048)),
                       dim3(256), 0, s, reinterpret_cast<const _Float16*>(W), cols, ldw, Wk, ldk);
  else if (w_dtype == GPTQ_DTYPE_F16)
    hipLaunchKernelGGL(convert_kernel<_Float16>, grid, dim3(256), 0, s,
                       reinterpret_cast<const _Float16*>(W), rows, cols, ldw, Wk, ldk);
  else
    hipLaunchKernelGGL(convert_kernel<float>, grid, dim3(256), 0, s,
                       reinterpret_cast<const float*>(W), rows, cols, ldw, Wk, ldk);
  return hipGetLastError();
}

hipError_t launch_sweep_block(float* Wk, int64_t ldk, int64_t rows, int64_t cols, int i1, int p0,
                              const float* Hinv, int bits, int groupsize, uint8_t* codes,
                              float* scales, float* zeros, float* Err, float* lpart,
                              hipStream_t s) {
  dim3 grid((unsigned)ceil_div(rows, kSweepRows));
  const bool vec = (cols % 4 == 0) && (reinterpret_cast<uintptr_t>(Hinv) % 16 == 0);
#define GPTQ_SWEEP(G)                                                                          \
  if (vec)                                                                                     \
    hipLaunchKernelGGL((sweep_kernel<G, true>), grid, dim3(256), 0, s, Wk, ldk, rows, cols,  \
                       i1, p0, Hinv, bits, groupsize, codes, scales, zeros, Err, lpart);       \
  else                                                                                         \
    hipLaunchKernelGGL((sweep_kernel<G, false>), grid, dim3(256), 0, s, Wk, ldk, rows, cols, \
                       i1, p0, Hinv, bits, groupsize, codes, scales, zeros, Err, lpart)
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

hipError_t launch_lazy_update(float* Wk, int64_t ldk, int64_t rows, int64_t cols, int k0, int k1,
                              int c0, int c1, const float* Err, const float* Hinv, hipStream_t s) {
  if (c1 <= c0 || k1 <= k0) return hipSuccess;
  const int64_t ncol = ceil_div(c1 - c0, LT);
  // big updates: 128x128 tiles; small ones: 32x128 tiles so more CUs take
  // part, with all of K (at most 128) and the W tile loaded up front.  The
  // far updates (K > 128: a superblock's errors) keep 128x128 or 64x128
  // tiles while those still give about one workgroup per CU: with K = 512 a
  // narrow tile's K loop waits on every chunk's loads (measured at attn:
  // 90, 58, 37 us against 108, 77, 41 us for the last three far updates).
  const bool far = k1 - k0 > 4 * LK;
  if (ncol * ceil_div(rows, 128) >= (far ? 256 : 512)) {
    dim3 grid((unsigned)ncol, (unsigned)ceil_div(rows, 128));
    hipLaunchKernelGGL((lazy_kernel<4, false>), grid, dim3(256), 0, s, Wk, ldk, rows, cols, k0, k1,
                       c0, c1, Err, Hinv);
  } else if (far && ncol * ceil_div(rows, 64) >= 256) {
    dim3 grid((unsigned)ncol, (unsigned)ceil_div(rows, 64));
    hipLaunchKernelGGL((lazy_kernel<2, false>), grid, dim3(256), 0, s, Wk, ldk, rows, cols, k0, k1,
                       c0, c1, Err, Hinv);
  } else {
    dim3 grid((unsigned)ncol, (unsigned)ceil_div(rows, 32));
    if (k1 - k0 <= 4 * LK)
      hipLaunchKernelGGL((lazy_kernel<1, true>), grid, dim3(256), 0, s, Wk, ldk, rows, cols, k0,
                         k1, c0, c1, Err, Hinv);
    else
      hipLaunchKernelGGL((lazy_kernel<1, false>), grid, dim3(256), 0, s, Wk, ldk, rows, cols, k0,
                         k1, c0, c1, Err, Hinv);
  }
  return hipGetLastError();
}

hipError_t launch_loss_reduce(const float* lpart, int64_t nparts, int64_t cols, float* losses,
                              hipStream_t s) {
  const int64_t ldk = round_up(cols, kBlock);
  hipLaunchKernelGGL(loss_reduce_kernel, dim3((unsigned)ceil_div(cols, 16)), dim3(256), 0, s,
                     lpart, nparts, ldk, cols, losses);
  return hipGetLastError();
}

}  // namespace gptq
