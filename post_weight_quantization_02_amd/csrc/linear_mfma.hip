// The layer's forward product from its stored form, for many tokens:
// y = act(x W_hat^T) in fp16 with W_hat[r][c] = (code - zero[r][g]) *
// scale[r][g], the codes packed 8 per 32-bit word (4 bits).  Quantizing
// layer by layer, a layer's calibration inputs are recorded from the model
// as it stands, so the layers already quantized run with these weights
// ("GPTQ: fixing errors as you go", "The algorithm, in words": run the
// calibration data through the model, record the layer's inputs, quantize,
// move to the next layer; the stored form is the low-bit integers with one
// scale per 128 weights).
//
// gfx950 design (a dense contraction, so MFMA):
//   * 128 tokens x 256 outputs per workgroup, eight waves (two per SIMD) of
//     128 x 32, each as 8 x 2 tiles of v_mfma_f32_16x16x32_f16: a lane holds
//     64 running sums and 64 group partials, so two waves fit one SIMD's
//     registers, and no two waves convert the same packed words.
//   * Per 128 input columns one ring stage (3 stages, 50 KB each) receives,
//     by direct global->LDS loads, the 128 x 128 fp16 tile of x, the 256 x 64
//     bytes of packed words and the 256 scales and zeros of the group.  Every
//     load address is clamped into the operand, so every wave issues the same
//     loads on every stage and waits on fixed vmcnt values.
//   * Exact products: the B operand is (q - z) in fp16, built from the packed
//     nibbles with v_perm_b32, a magic-number OR (0x6400 | q = 1024 + q,
//     0x6400 | 16q = 1024 + 16q) and one packed fp16 FMA; every step is exact
//     for integer zeros in [0, 15].  x * (q - z) is exact in fp32, so a
//     group's MFMA sum has only fp32 summation error; it is kept apart and
//     added as acc += scale * partial at the group's last column.
//   * The K order inside an MFMA is free as long as both operands follow it:
//     over a group's 128 columns, lane group k (lanes 16k..16k+15) takes
//     columns 32k..32k+31, so the words of a lane's four K steps are one
//     16-byte piece of the packed row.
//   * XCD-aware order: an XCD works on groups of 4 token tiles x all output
//     tiles, 4 x 8 tiles at a time, so its L2 serves both operands.
#include "common.h"

namespace gptq {
namespace {

constexpr int TM = 128;    // tokens per workgroup
constexpr int TN = 256;    // outputs per workgroup
constexpr int KG = 128;    // input columns per stage
constexpr int NSTAGE = 3;
constexpr int X_BYTES = TM * KG * 2;        // 32 KB
constexpr int B_BYTES = TN * (KG / 2);      // 16 KB (4-bit codes)
constexpr int S_BYTES = TN * 4;             // 1 KB
constexpr int STAGE = X_BYTES + B_BYTES + 2 * S_BYTES;  // 50 KB
constexpr int NWAVE = 8;
// Wave layout: WAVES_M x WAVES_N waves, each WTM tokens x WTN outputs as AT x BT
// MFMA tiles.  1 x 8: each wave owns distinct outputs, so every packed word is
// turned into fp16 operands once per workgroup (2 x 4 would do it twice),
// at the price of twice the x fragment reads from LDS.
constexpr int WAVES_M = 1, WAVES_N = NWAVE / WAVES_M;
constexpr int WTM = TM / WAVES_M, WTN = TN / WAVES_N;
constexpr int AT = WTM / 16, BT = WTN / 16;
constexpr int LOADS_PER_STAGE = (X_BYTES / 1024 + B_BYTES / 1024) / NWAVE + 1;  // per wave: 7
constexpr int kXcds = 8;
constexpr int kGroupM = 4;  // token tiles per XCD-local group

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

// physical 16-byte piece of an x row (256 bytes) holding logical piece p
__device__ inline int x_piece(int row, int p) { return p ^ (row & 15); }
// physical 16-byte piece of a packed-word row (64 bytes) holding logical piece p
__device__ inline int b_piece(int row, int p) { return p ^ (((row >> 1) ^ (row >> 2)) & 3); }

// s_waitcnt vmcnt <= N (expcnt and lgkmcnt unconstrained; gfx9 encoding)
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

// (q - z) for the 8 codes of one word, in column order, as an MFMA operand.
// Byte p of the word holds codes 2p (low nibble) and 2p + 1 (high nibble).
__device__ inline half8 codes_minus_zero(uint32_t w, half2_t mul, half2_t off, uint32_t magic) {
  half8 r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    // 0x00bb00bb with byte p of w in both halves (selector 12 gives 0x00)
    const uint32_t b = __builtin_amdgcn_perm(w, w, (12u << 24) | ((uint32_t)p << 16) | (12u << 8) | p);
    // low half 0x6400 | q_lo = 1024 + q_lo, high half 0x6400 | 16 q_hi = 1024 + 16 q_hi, in
    // one v_and_or_b32 (a VOP3 op takes no literal here: the mask goes in an SGPR,
    // the magic number in a VGPR)
    uint32_t m;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(m) : "v"(b), "s"(0x00F0000Fu), "v"(magic));
    const half2_t h = __builtin_bit_cast(half2_t, m) * mul + off;  // exact: (q_lo - z, q_hi - z)
    r[2 * p] = h[0];
    r[2 * p + 1] = h[1];
  }
  return r;
}

// Per-lane byte offsets of one stage's direct loads, relative to wave-uniform
// bases (x row t0, packed row n0, scale/zero row n0, all at column 0):
// clamped rows, swizzled pieces.  They fit 32 bits (at most 256 rows of at
// most 2^22 bytes, plus the column offset), so the loads use a scalar base and
// one VGPR each.
struct DmaOffsets {
  uint32_t x[4];  // x: 32 wave loads of 4 rows x 256 bytes, this wave's 4
  uint32_t w[2];  // packed words: 16 wave loads of 16 rows x 64 bytes, this wave's 2
  uint32_t sz;    // scales (waves 0-3) or zeros (waves 4-7) of 64 outputs
};

__device__ inline DmaOffsets dma_offsets(int64_t ldx, int64_t t0, int64_t m, int64_t nw,
                                         int64_t ngroups, int64_t n0, int64_t rows, int wave,
                                         int lane) {
  DmaOffsets d;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = 4 * (wave + NWAVE * u) + (lane >> 4);
    const int64_t t = min(t0 + row, m - 1) - t0;
    d.x[u] = (uint32_t)((t * ldx + 8 * x_piece(row, lane & 15)) * 2);
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = 16 * (wave + NWAVE * u) + (lane >> 2);
    const int64_t r = min(n0 + row, rows - 1) - n0;
    d.w[u] = (uint32_t)((r * nw + 4 * b_piece(row, lane & 3)) * 4);
  }
  const int64_t r = min(n0 + 64 * (wave & 3) + lane, rows - 1) - n0;
  d.sz = (uint32_t)(r * ngroups * 4);
  return d;
}

// Issue one stage's direct loads (input columns c0..c0+127) into `st`.
__device__ inline void issue_stage(const char* xb, const char* wbase, const char* szb,
                                   const DmaOffsets& d, int k, int grp, char* st, int wave) {
  const uint32_t c0 = (uint32_t)k * KG;
  // the column offset goes into the 32-bit lane offset (at most 2^21 more),
  // which keeps each address a scalar base plus one VGPR inside the loop
  const uint32_t cx = c0 * 2, cw = c0 / 2, cs = (uint32_t)grp * 4;
#pragma unroll
  for (int u = 0; u < 4; ++u)
    __builtin_amdgcn_global_load_lds((const void*)(xb + (d.x[u] + cx)),
                                     (lds_void*)(st + 1024 * (wave + NWAVE * u)), 16, 0, 0);
#pragma unroll
  for (int u = 0; u < 2; ++u)
    __builtin_amdgcn_global_load_lds((const void*)(wbase + (d.w[u] + cw)),
                                     (lds_void*)(st + X_BYTES + 1024 * (wave + NWAVE * u)), 16, 0,
                                     0);
  __builtin_amdgcn_global_load_lds(
      (const void*)(szb + (d.sz + cs)),
      (lds_void*)(st + X_BYTES + B_BYTES + (wave >> 2) * S_BYTES + 256 * (wave & 3)), 4, 0, 0);
}

// Position of a stage inside its scale group (groups are gk stages long);
// kept as running counters so the loop does no division.
struct GroupCursor {
  int in = 0;   // stage index inside the group
  int grp = 0;  // group index
  __device__ void advance(int gk) {
    if (++in == gk) {
      in = 0;
      ++grp;
    }
  }
};

// One stage of the main loop: wait for stage k (held in `cur`), publish it
// with a barrier, start the loads of stage k + 2 into `nxt` (the stage read
// in the previous step), then the four K steps of this stage's 128 columns.
// The stages are three distinct LDS arrays named at compile time, so the
// compiler can tell that reading `cur` does not touch the direct loads still
// landing in the other two and adds no wait for them.
// Per-lane LDS byte offsets inside a stage.  With row = WTM wm + 16 a + li the
// x swizzle (p ^ (row & 15)) depends on li only, and with row = WTN wn + 16 b
// + li so does the word swizzle, so every read is one of these offsets plus
// a compile-time constant.
struct LaneOffsets {
  int x[4];   // A operand of K step s, a-tile 0 (a-tile a adds 4096 a)
  int w;      // packed words of b-tile 0 (b-tile b adds 1024 b)
  int sz;     // scale / zero of b-tile 0 (b-tile b adds 64 b)
};

// acc += scale * partial for every output of the lane (the group's last stage)
__device__ inline void fold_group(f32x4 (&acc)[AT][BT], const f32x4 (&part)[AT][BT],
                                  const float (&fsc)[BT]) {
#pragma unroll
  for (int b = 0; b < BT; ++b)
#pragma unroll
    for (int a = 0; a < AT; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[a][b][i] = __builtin_fmaf(fsc[b], part[a][b][i], acc[a][b][i]);
}

__device__ inline void stage_step(int k, int nk, const char* cur, char* nxt, const char* xb,
                                  const char* wbase, const char* szb, const DmaOffsets& dm,
                                  int gk, GroupCursor& use, GroupCursor& iss, int wave,
                                  const LaneOffsets& lo, f32x4 (&acc)[AT][BT], f32x4 (&part)[AT][BT],
                                  bool& fold, float (&fsc)[BT]) {
  // stage k has landed for this wave; stage k + 1 may still be in flight
  if (k + 1 < nk) wait_vm<LOADS_PER_STAGE>();
  else wait_vm<0>();
  lds_barrier();
  const char* sb = cur + X_BYTES;
  const float* ss = reinterpret_cast<const float*>(cur + X_BYTES + B_BYTES);
  const float* sz = reinterpret_cast<const float*>(cur + X_BYTES + B_BYTES + S_BYTES);
  // The zero points are read before the next stage's loads are issued: where
  // the compiler cannot rule out that this read overlaps loads still in
  // flight (after the loop's back edge) it waits for them, and at this point
  // that is only stage k + 1, issued a whole stage earlier.
  half2_t off[BT];
#pragma unroll
  for (int b = 0; b < BT; ++b) {
    const float z = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(sz) + lo.sz + 64 * b);
    off[b] = half2_t{(_Float16)(-1024.0f - z), (_Float16)(-64.0f - z)};
  }
  // a lane's four words of the stage, one 16-byte read per b-tile (the word
  // swizzle keeps these reads free of bank conflicts; 4-byte reads of the
  // same layout would not be)
  uint4 wb[BT];
#pragma unroll
  for (int b = 0; b < BT; ++b) wb[b] = *reinterpret_cast<const uint4*>(sb + lo.w + 1024 * b);
  if (k + 2 < nk) {
    issue_stage(xb, wbase, szb, dm, k + 2, iss.grp, nxt, wave);
    iss.advance(gk);
  }
  // The previous group's partial sums enter the running sums here, after the
  // barrier, where these FMAs fill the wait for this stage's first LDS reads
  // instead of delaying the barrier.
  if (fold) {
    fold_group(acc, part, fsc);
    fold = false;
  }

  const bool gstart = use.in == 0;
  const bool gend = use.in == gk - 1 || k + 1 == nk;
  use.advance(gk);
  const half2_t mul = {(_Float16)1.0f, (_Float16)0.0625f};
  const uint32_t magic = 0x64006400u;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    half8 af[AT];
#pragma unroll
    for (int a = 0; a < AT; ++a)
      af[a] = *reinterpret_cast<const half8*>(cur + lo.x[s] + 4096 * a);
    half8 bf[BT];
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      const uint32_t w = s == 0 ? wb[b].x : s == 1 ? wb[b].y : s == 2 ? wb[b].z : wb[b].w;
      bf[b] = codes_minus_zero(w, mul, off[b], magic);
    }
    if (s == 0 && gstart) {
#pragma unroll
      for (int a = 0; a < AT; ++a)
#pragma unroll
        for (int b = 0; b < BT; ++b)
          part[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[a], bf[b],
                                                              f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    } else {
#pragma unroll
      for (int a = 0; a < AT; ++a)
#pragma unroll
        for (int b = 0; b < BT; ++b)
          part[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[a], bf[b], part[a][b], 0, 0, 0);
    }
  }
  if (gend) {  // the group's scales now; its fold at the next stage (or after the loop)
#pragma unroll
    for (int b = 0; b < BT; ++b)
      fsc[b] = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(ss) + lo.sz + 64 * b);
    fold = true;
  }
}

template <bool RELU>
__global__ __launch_bounds__(512, 1) void linear_int4_kernel(
    const _Float16* __restrict__ x, int64_t ldx, int64_t m, const uint32_t* __restrict__ packed,
    int64_t nw, int64_t rows, int64_t cols, const float* __restrict__ scales,
    const float* __restrict__ zeros, int64_t ngroups, int gk, int64_t ntn, int64_t ntm,
    _Float16* __restrict__ y, int64_t ldy) {
  __shared__ __attribute__((aligned(1024))) char st0[STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[STAGE];
  __shared__ __attribute__((aligned(1024))) char st2[STAGE];

  // XCD-aware tile order.  Workgroup b runs on XCD b % 8, which takes token
  // tiles xcd, xcd + 8, ...; its local index walks them in groups of kGroupM
  // token tiles, and within a group output tile by output tile, so the ~32
  // workgroups an XCD runs at once share 4 x tiles and 8 weight tiles in its
  // L2 (32 KB and 16 KB per stage: the split that minimises its misses).
  const int64_t bid = blockIdx.x;
  const int64_t xcd = bid % kXcds, local = bid / kXcds;
  const int64_t grp = local / (kGroupM * ntn), idx = local % (kGroupM * ntn);
  const int64_t tm = (grp * kGroupM + idx % kGroupM) * kXcds + xcd;
  const int64_t tn = idx / kGroupM;
  if (tm >= ntm) return;
  const int64_t t0 = tm * TM, n0 = tn * TN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar bases
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int li = lane & 15, kg = lane >> 4;
  const int nk = (int)(cols / KG);
  LaneOffsets lo;
#pragma unroll
  for (int s = 0; s < 4; ++s) lo.x[s] = 256 * (WTM * wm + li) + 16 * x_piece(li, 4 * kg + s);
  lo.w = 64 * (WTN * wn + li) + 16 * b_piece(li, kg);
  lo.sz = 4 * (WTN * wn + li);

  f32x4 acc[AT][BT], part[AT][BT];
#pragma unroll
  for (int a = 0; a < AT; ++a)
#pragma unroll
    for (int b = 0; b < BT; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const DmaOffsets dm = dma_offsets(ldx, t0, m, nw, ngroups, n0, rows, wave, lane);
  const char* xb = reinterpret_cast<const char*>(x + t0 * ldx);
  const char* wbase = reinterpret_cast<const char*>(packed + n0 * nw);
  const char* szb = reinterpret_cast<const char*>((wave < 4 ? scales : zeros) + n0 * ngroups);

  GroupCursor use, iss;
  issue_stage(xb, wbase, szb, dm, 0, iss.grp, st0, wave);
  iss.advance(gk);
  if (nk > 1) {
    issue_stage(xb, wbase, szb, dm, 1, iss.grp, st1, wave);
    iss.advance(gk);
  }
  bool fold = false;
  float fsc[BT];
  for (int k = 0; k < nk; k += NSTAGE) {
    stage_step(k, nk, st0, st2, xb, wbase, szb, dm, gk, use, iss, wave, lo, acc, part, fold, fsc);
    if (k + 1 < nk)
      stage_step(k + 1, nk, st1, st0, xb, wbase, szb, dm, gk, use, iss, wave, lo, acc, part, fold,
                 fsc);
    if (k + 2 < nk)
      stage_step(k + 2, nk, st2, st1, xb, wbase, szb, dm, gk, use, iss, wave, lo, acc, part, fold,
                 fsc);
  }
  fold_group(acc, part, fsc);  // the last stage always ends a group

  // lane holds rows 4 * kg + i of each 16 x 16 tile, column li
#pragma unroll
  for (int a = 0; a < AT; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t t = t0 + WTM * wm + 16 * a + 4 * kg + i;
      if (t >= m) continue;
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        const int64_t r = n0 + WTN * wn + 16 * b + li;
        if (r >= rows) continue;
        float v = acc[a][b][i];
        if (RELU) v = v > 0.f ? v : 0.f;
        y[t * ldy + r] = (_Float16)v;
      }
    }
}

}  // namespace

namespace {
int64_t linear_blocks(int64_t m, int64_t rows) {
  // every XCD gets the same whole number of kGroupM-token-tile groups
  return kXcds * round_up(ceil_div(ceil_div(m, TM), kXcds), kGroupM) * ceil_div(rows, TN);
}
}  // namespace

bool linear_int4_supported(int64_t m, int64_t rows, int64_t cols, int groupsize, const void* x,
                           int64_t ldx, const void* packed) {
  // ldx < 2^23: a token tile's lane offsets (< 128 rows of 2 ldx bytes) fit 32 bits;
  // the grid's work-items must fit 32 bits
  return cols % KG == 0 && (groupsize % KG == 0 || groupsize >= cols) && ldx % 8 == 0 &&
         ldx < ((int64_t)1 << 23) &&
         (reinterpret_cast<uintptr_t>(x) & 15) == 0 &&
         (reinterpret_cast<uintptr_t>(packed) & 15) == 0 &&
         linear_blocks(m, rows) * 64 * NWAVE <= (int64_t)UINT32_MAX;
}

hipError_t launch_linear_int4(const _Float16* x, int64_t ldx, int64_t m, const uint32_t* packed,
                              int64_t rows, int64_t cols, const float* scales, const float* zeros,
                              int groupsize, bool relu, _Float16* y, int64_t ldy, hipStream_t s) {
  const int g = groupsize >= cols ? (int)cols : groupsize;
  const int64_t ngroups = ceil_div(cols, g);
  const int gk = (int)ceil_div(g, KG);  // stages per group (a short last group ends at cols)
  const int64_t nw = cols / 8;
  const int64_t ntm = ceil_div(m, TM), ntn = ceil_div(rows, TN);
  const int64_t blocks = linear_blocks(m, rows);
  if (relu)
    hipLaunchKernelGGL(linear_int4_kernel<true>, dim3((unsigned)blocks), dim3(512), 0, s, x, ldx, m,
                       packed, nw, rows, cols, scales, zeros, ngroups, gk, ntn, ntm, y, ldy);
  else
    hipLaunchKernelGGL(linear_int4_kernel<false>, dim3((unsigned)blocks), dim3(512), 0, s, x, ldx,
                       m, packed, nw, rows, cols, scales, zeros, ngroups, gk, ntn, ntm, y, ldy);
  return hipGetLastError();
}

}  // namespace gptq
