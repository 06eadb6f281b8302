// The layer's forward product from its stored form, for many tokens:
// y = act(x W_hat^T) in fp16 with W_hat[r][c] = (code - zero[r][g]) *
// scale[r][g], the codes packed 8 (4 bits) or 4 (8 bits) per 32-bit word.
// Quantizing layer by layer, a layer's calibration inputs are recorded from
// the model as it stands, so the layers already quantized run with these
// weights ("GPTQ: fixing errors as you go", "The algorithm, in words": run
// the calibration data through the model, record the layer's inputs,
// quantize, move to the next layer; the stored form is the low-bit integers
// with one scale per 128 weights).
//
// gfx950 design (a dense contraction, so MFMA):
//   * 128 tokens x 256 outputs (4 bits) or 128 outputs (8 bits: the same
//     16 KB of packed words per stage) per workgroup, eight waves (two per
//     SIMD) of 128 tokens each, as 8 x 2 (8 x 1) tiles of
//     v_mfma_f32_16x16x32_f16.  A lane holds its running sums and group
//     partials, so two waves fit one SIMD's registers, and no two waves
//     convert the same packed words.
//   * Per 128 input columns one ring stage (3 stages, 50 or 49 KB each)
//     receives, by direct global->LDS loads, the 128 x 128 fp16 tile of x,
//     the 16 KB of packed words and the scales and zeros of the group.  Every
//     load address is clamped into the operand, so every wave issues the same
//     loads on every stage and waits on fixed vmcnt values.
//   * Exact products: the B operand is (q - z) in fp16.  4 bits: v_perm_b32
//     puts a byte in both halves, a magic-number OR gives 0x6400 | q =
//     1024 + q and 0x6400 | 16q = 1024 + 16q, one packed fp16 FMA with
//     (1, 1/16) and (-1024 - z, -64 - z) leaves q - z.  8 bits: v_perm_b32
//     interleaves two code bytes with 0x64 bytes (1024 + q) and one packed
//     fp16 add with -1024 - z leaves q - z.  Every step is exact for integer
//     zeros in [0, 2^bits - 1].  x * (q - z) is exact in fp32, so a group's
//     MFMA sum has only fp32 summation error; it is kept apart and added as
//     acc += scale * partial when the group ends.
//   * The K order inside an MFMA is free as long as both operands follow it:
//     over a group's 128 columns, lane group k (lanes 16k..16k+15) takes
//     columns 32k..32k+31, so the words of a lane's four K steps are one
//     (4 bits) or two (8 bits) 16-byte pieces of the packed row.
//   * XCD-aware order: an XCD works on groups of 4 token tiles x all output
//     tiles, 4 x 8 tiles at a time, so its L2 serves both operands.
#include "common.h"

namespace gptq {
namespace {

constexpr int TM = 128;    // tokens per workgroup
constexpr int KG = 128;    // input columns per stage
constexpr int NSTAGE = 3;
constexpr int X_BYTES = TM * KG * 2;  // 32 KB
constexpr int NWAVE = 8;
constexpr int AT = TM / 16;           // a-tiles per wave (each wave owns all 128 tokens)
constexpr int kXcds = 8;
constexpr int kGroupM = 4;  // token tiles per XCD-local group

// What depends on the code width.  `piece` is the XOR swizzle of the 16-byte
// pieces of a stage's packed row: the 16-byte reads of 16 consecutive rows at
// one logical piece hit distinct bank groups, for 8- and for 16-lane LDS
// service groups.
template <int BITS>
struct Geo;
template <>
struct Geo<4> {
  static constexpr int TN = 256;  // outputs per workgroup
  static constexpr int RB = 64;   // packed bytes of one output row per stage
  static constexpr int LP = 1;    // 16-byte pieces per lane per stage
  __device__ static int piece(int row, int p) { return p ^ (((row >> 1) ^ (row >> 2)) & 3); }
};
template <>
struct Geo<8> {
  static constexpr int TN = 128;
  static constexpr int RB = 128;
  static constexpr int LP = 2;
  __device__ static int piece(int row, int p) { return p ^ ((row ^ (row >> 3)) & 7); }
};

template <int BITS>
struct Lay {
  static constexpr int TN = Geo<BITS>::TN, RB = Geo<BITS>::RB, LP = Geo<BITS>::LP;
  static constexpr int PPR = RB / 16;          // pieces per packed row
  static constexpr int B_BYTES = TN * RB;      // 16 KB
  static constexpr int S_BYTES = TN * 4;       // scales (zeros follow)
  static constexpr int STAGE = X_BYTES + B_BYTES + 2 * S_BYTES;
  static constexpr int WTN = TN / NWAVE;       // outputs per wave
  static constexpr int BT = WTN / 16;          // b-tiles per wave
  static constexpr int BROWS = 1024 / RB;      // packed rows per 1 KB wave load
  static constexpr int XU = X_BYTES / 1024 / NWAVE;  // x loads per wave per stage
  static constexpr int WU = B_BYTES / 1024 / NWAVE;  // word loads per wave per stage
  static constexpr int SZL = 2 * S_BYTES / 256;      // 256-byte scale/zero loads per stage
  static constexpr int LOADS_PER_STAGE = XU + WU + 1;
  static_assert(B_BYTES == 16384 && XU == 4 && WU == 2 && SZL <= NWAVE, "stage layout");
};

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

// physical 16-byte piece of an x row (256 bytes) holding logical piece p
__device__ inline int x_piece(int row, int p) { return p ^ (row & 15); }

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

// (q - z) for the 8 codes of one 4-bit word, in column order, as an MFMA
// operand.  Byte p of the word holds codes 2p (low nibble) and 2p + 1.
__device__ inline half8 codes_minus_zero4(uint32_t w, half2_t mul, half2_t off, uint32_t magic) {
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

// (q - z) for the 8 codes of two 8-bit words (4 codes each, lowest column in
// the lowest byte).  v_perm_b32 selects bytes of the 64-bit {src0, src1},
// 0-3 from src1 (here the word) and 4-7 from src0 (here 0x64646464), so
// selector 0x04010400 gives 0x64 b1 0x64 b0: the halves 1024 + q0, 1024 + q1.
__device__ inline half8 codes_minus_zero8(uint32_t w0, uint32_t w1, half2_t off) {
  half8 r;
  const uint32_t words[2] = {w0, w1};
#pragma unroll
  for (int v = 0; v < 2; ++v)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const uint32_t sel = 0x04000400u | ((uint32_t)(2 * p + 1) << 16) | (uint32_t)(2 * p);
      const uint32_t m = __builtin_amdgcn_perm(0x64646464u, words[v], sel);
      const half2_t h = __builtin_bit_cast(half2_t, m) + off;  // exact: (q - z, q' - z)
      r[4 * v + 2 * p] = h[0];
      r[4 * v + 2 * p + 1] = h[1];
    }
  return r;
}

// Per-lane byte offsets of one stage's direct loads, relative to wave-uniform
// bases (x row t0, packed row n0, scale/zero row n0, all at column 0):
// clamped rows, swizzled pieces.  They fit 32 bits (at most 256 rows of at
// most 2^22 bytes, plus the column offset), so the loads use a scalar base and
// one VGPR each.
template <int BITS>
struct DmaOffsets {
  uint32_t x[Lay<BITS>::XU];  // x: wave loads of 4 rows x 256 bytes
  uint32_t w[Lay<BITS>::WU];  // packed words: wave loads of 1 KB of packed rows
  uint32_t sz;                // the scales or zeros of 64 outputs
};

// Load q = wave % SZL of a stage's scale/zero loads: the scales (q < SZL / 2)
// or zeros of outputs 64 (q % (SZL / 2)) + 0..63.  With SZL < NWAVE (8 bits)
// waves q and q + SZL issue the same load, so every wave issues one.
template <int BITS>
__device__ inline int sz_load(int wave) {
  return wave % Lay<BITS>::SZL;
}

template <int BITS>
__device__ inline DmaOffsets<BITS> dma_offsets(int64_t ldx, int64_t t0, int64_t m, int64_t nw,
                                               int64_t ngroups, int64_t n0, int64_t rows,
                                               int wave, int lane) {
  using L = Lay<BITS>;
  DmaOffsets<BITS> d;
#pragma unroll
  for (int u = 0; u < L::XU; ++u) {
    const int row = 4 * (wave + NWAVE * u) + (lane >> 4);
    const int64_t t = min(t0 + row, m - 1) - t0;
    d.x[u] = (uint32_t)((t * ldx + 8 * x_piece(row, lane & 15)) * 2);
  }
#pragma unroll
  for (int u = 0; u < L::WU; ++u) {
    const int row = L::BROWS * (wave + NWAVE * u) + lane / L::PPR;
    const int64_t r = min(n0 + row, rows - 1) - n0;
    d.w[u] = (uint32_t)(r * nw * 4 + 16 * Geo<BITS>::piece(row, lane % L::PPR));
  }
  const int q = sz_load<BITS>(wave);
  const int64_t r = min(n0 + 64 * (q % (L::SZL / 2)) + lane, rows - 1) - n0;
  d.sz = (uint32_t)(r * ngroups * 4);
  return d;
}

// Issue one stage's direct loads (input columns c0..c0+127) into `st`.
template <int BITS>
__device__ inline void issue_stage(const char* xb, const char* wbase, const char* szb,
                                   const DmaOffsets<BITS>& d, int k, int grp, char* st, int wave) {
  using L = Lay<BITS>;
  const uint32_t c0 = (uint32_t)k * KG;
  // the column offset goes into the 32-bit lane offset (at most 2^21 more),
  // which keeps each address a scalar base plus one VGPR inside the loop
  const uint32_t cx = c0 * 2, cw = c0 * BITS / 8, cs = (uint32_t)grp * 4;
#pragma unroll
  for (int u = 0; u < L::XU; ++u)
    __builtin_amdgcn_global_load_lds((const void*)(xb + (d.x[u] + cx)),
                                     (lds_void*)(st + 1024 * (wave + NWAVE * u)), 16, 0, 0);
#pragma unroll
  for (int u = 0; u < L::WU; ++u)
    __builtin_amdgcn_global_load_lds((const void*)(wbase + (d.w[u] + cw)),
                                     (lds_void*)(st + X_BYTES + 1024 * (wave + NWAVE * u)), 16, 0,
                                     0);
  __builtin_amdgcn_global_load_lds(
      (const void*)(szb + (d.sz + cs)),
      (lds_void*)(st + X_BYTES + L::B_BYTES + 256 * sz_load<BITS>(wave)), 4, 0, 0);
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

// Per-lane LDS byte offsets inside a stage.  With row = 16 a + li the x
// swizzle (p ^ (row & 15)) depends on li only, so every x read is x[s] plus a
// compile-time constant; the word pieces are read at w[h] (b-tile b adds
// 16 RB b: the 4-bit swizzle does not change over 16 rows).
template <int BITS>
struct LaneOffsets {
  int x[4];                  // A operand of K step s, a-tile 0 (a-tile a adds 4096 a)
  int w[Geo<BITS>::LP];      // packed-word piece h of b-tile 0
  int sz;                    // scale / zero of b-tile 0 (b-tile b adds 64 b)
};

// acc += scale * partial for every output of the lane (the group's last stage)
template <int BT>
__device__ inline void fold_group(f32x4 (&acc)[AT][BT], const f32x4 (&part)[AT][BT],
                                  const float (&fsc)[BT]) {
#pragma unroll
  for (int b = 0; b < BT; ++b)
#pragma unroll
    for (int a = 0; a < AT; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[a][b][i] = __builtin_fmaf(fsc[b], part[a][b][i], acc[a][b][i]);
}

// One stage of the main loop: wait for stage k (held in `cur`), publish it
// with a barrier, start the loads of stage k + 2 into `nxt` (the stage read
// in the previous step), then the four K steps of this stage's 128 columns.
// The stages are three distinct LDS arrays named at compile time, so the
// compiler can tell that reading `cur` does not touch the direct loads still
// landing in the other two and adds no wait for them.
template <int BITS>
__device__ inline void stage_step(int k, int nk, const char* cur, char* nxt, const char* xb,
                                  const char* wbase, const char* szb,
                                  const DmaOffsets<BITS>& dm, int gk, GroupCursor& use,
                                  GroupCursor& iss, int wave, const LaneOffsets<BITS>& lo,
                                  f32x4 (&acc)[AT][Lay<BITS>::BT],
                                  f32x4 (&part)[AT][Lay<BITS>::BT], bool& fold,
                                  float (&fsc)[Lay<BITS>::BT]) {
  using L = Lay<BITS>;
  constexpr int BT = L::BT;
  // stage k has landed for this wave; stage k + 1 may still be in flight
  if (k + 1 < nk) wait_vm<L::LOADS_PER_STAGE>();
  else wait_vm<0>();
  lds_barrier();
  const char* sb = cur + X_BYTES;
  const char* ss = cur + X_BYTES + L::B_BYTES;
  const char* sz = ss + L::S_BYTES;
  // The zero points are read before the next stage's loads are issued: where
  // the compiler cannot rule out that this read overlaps loads still in
  // flight (after the loop's back edge) it waits for them, and at this point
  // that is only stage k + 1, issued a whole stage earlier.
  half2_t off[BT];
#pragma unroll
  for (int b = 0; b < BT; ++b) {
    const float z = *reinterpret_cast<const float*>(sz + lo.sz + 64 * b);
    off[b] = BITS == 4 ? half2_t{(_Float16)(-1024.0f - z), (_Float16)(-64.0f - z)}
                       : half2_t{(_Float16)(-1024.0f - z), (_Float16)(-1024.0f - z)};
  }
  // a lane's words of the stage, 16-byte reads (the word swizzle keeps these
  // reads free of bank conflicts; 4-byte reads of the same layout would not be)
  uint4 wb[BT][L::LP];
#pragma unroll
  for (int b = 0; b < BT; ++b)
#pragma unroll
    for (int h = 0; h < L::LP; ++h)
      wb[b][h] = *reinterpret_cast<const uint4*>(sb + lo.w[h] + 16 * L::RB * b);
  if (k + 2 < nk) {
    issue_stage<BITS>(xb, wbase, szb, dm, k + 2, iss.grp, nxt, wave);
    iss.advance(gk);
  }
  // The previous group's partial sums enter the running sums here, after the
  // barrier, where these FMAs fill the wait for this stage's first LDS reads
  // instead of delaying the barrier.
  if (fold) {
    fold_group<BT>(acc, part, fsc);
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
      if constexpr (BITS == 4) {
        const uint4 v = wb[b][0];
        const uint32_t w = s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w;
        bf[b] = codes_minus_zero4(w, mul, off[b], magic);
      } else {
        // K step s: columns 8s..8s+7, words 2s and 2s + 1 of the lane's 8
        const uint4 v = wb[b][s >> 1];
        bf[b] = (s & 1) ? codes_minus_zero8(v.z, v.w, off[b]) : codes_minus_zero8(v.x, v.y, off[b]);
      }
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
    for (int b = 0; b < BT; ++b) fsc[b] = *reinterpret_cast<const float*>(ss + lo.sz + 64 * b);
    fold = true;
  }
}

template <int BITS, bool RELU>
__global__ __launch_bounds__(512, 1) void linear_kernel(
    const _Float16* __restrict__ x, int64_t ldx, int64_t m, const uint32_t* __restrict__ packed,
    int64_t nw, int64_t rows, int64_t cols, const float* __restrict__ scales,
    const float* __restrict__ zeros, int64_t ngroups, int gk, int64_t ntn, int64_t ntm,
    _Float16* __restrict__ y, int64_t ldy) {
  using L = Lay<BITS>;
  constexpr int BT = L::BT;
  __shared__ __attribute__((aligned(1024))) char st0[L::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[L::STAGE];
  __shared__ __attribute__((aligned(1024))) char st2[L::STAGE];

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
  const int64_t t0 = tm * TM, n0 = tn * L::TN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar bases
  const int li = lane & 15, kg = lane >> 4;
  const int nk = (int)(cols / KG);
  LaneOffsets<BITS> lo;
#pragma unroll
  for (int s = 0; s < 4; ++s) lo.x[s] = 256 * li + 16 * x_piece(li, 4 * kg + s);
  {
    const int row = L::WTN * wave + li;  // b-tile 0
#pragma unroll
    for (int h = 0; h < L::LP; ++h)
      lo.w[h] = L::RB * row + 16 * Geo<BITS>::piece(row, L::LP * kg + h);
    lo.sz = 4 * row;
  }

  f32x4 acc[AT][BT], part[AT][BT];
#pragma unroll
  for (int a = 0; a < AT; ++a)
#pragma unroll
    for (int b = 0; b < BT; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const DmaOffsets<BITS> dm = dma_offsets<BITS>(ldx, t0, m, nw, ngroups, n0, rows, wave, lane);
  const char* xb = reinterpret_cast<const char*>(x + t0 * ldx);
  const char* wbase = reinterpret_cast<const char*>(packed + n0 * nw);
  const char* szb = reinterpret_cast<const char*>(
      (sz_load<BITS>(wave) < L::SZL / 2 ? scales : zeros) + n0 * ngroups);

  GroupCursor use, iss;
  issue_stage<BITS>(xb, wbase, szb, dm, 0, iss.grp, st0, wave);
  iss.advance(gk);
  if (nk > 1) {
    issue_stage<BITS>(xb, wbase, szb, dm, 1, iss.grp, st1, wave);
    iss.advance(gk);
  }
  bool fold = false;
  float fsc[BT];
  for (int k = 0; k < nk; k += NSTAGE) {
    stage_step<BITS>(k, nk, st0, st2, xb, wbase, szb, dm, gk, use, iss, wave, lo, acc, part, fold,
                     fsc);
    if (k + 1 < nk)
      stage_step<BITS>(k + 1, nk, st1, st0, xb, wbase, szb, dm, gk, use, iss, wave, lo, acc, part,
                       fold, fsc);
    if (k + 2 < nk)
      stage_step<BITS>(k + 2, nk, st2, st1, xb, wbase, szb, dm, gk, use, iss, wave, lo, acc, part,
                       fold, fsc);
  }
  fold_group<BT>(acc, part, fsc);  // the last stage always ends a group

  // lane holds rows 4 * kg + i of each 16 x 16 tile, column li
#pragma unroll
  for (int a = 0; a < AT; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t t = t0 + 16 * a + 4 * kg + i;
      if (t >= m) continue;
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        const int64_t r = n0 + L::WTN * wave + 16 * b + li;
        if (r >= rows) continue;
        float v = acc[a][b][i];
        if (RELU) v = v > 0.f ? v : 0.f;
        y[t * ldy + r] = (_Float16)v;
      }
    }
}

int64_t linear_blocks(int bits, int64_t m, int64_t rows) {
  const int tn = bits == 4 ? Geo<4>::TN : Geo<8>::TN;
  // every XCD gets the same whole number of kGroupM-token-tile groups
  return kXcds * round_up(ceil_div(ceil_div(m, TM), kXcds), kGroupM) * ceil_div(rows, tn);
}

template <int BITS>
hipError_t launch_bits(const _Float16* x, int64_t ldx, int64_t m, const uint32_t* packed,
                       int64_t rows, int64_t cols, const float* scales, const float* zeros,
                       int groupsize, bool relu, _Float16* y, int64_t ldy, hipStream_t s) {
  const int g = groupsize >= cols ? (int)cols : groupsize;
  const int64_t ngroups = ceil_div(cols, g);
  const int gk = (int)ceil_div(g, KG);  // stages per group (a short last group ends at cols)
  const int64_t nw = cols * BITS / 32;
  const int64_t ntm = ceil_div(m, TM), ntn = ceil_div(rows, Geo<BITS>::TN);
  const int64_t blocks = linear_blocks(BITS, m, rows);
  if (relu)
    hipLaunchKernelGGL((linear_kernel<BITS, true>), dim3((unsigned)blocks), dim3(64 * NWAVE), 0, s,
                       x, ldx, m, packed, nw, rows, cols, scales, zeros, ngroups, gk, ntn, ntm, y,
                       ldy);
  else
    hipLaunchKernelGGL((linear_kernel<BITS, false>), dim3((unsigned)blocks), dim3(64 * NWAVE), 0,
                       s, x, ldx, m, packed, nw, rows, cols, scales, zeros, ngroups, gk, ntn, ntm,
                       y, ldy);
  return hipGetLastError();
}

}  // namespace

bool linear_forward_supported(int bits, int64_t m, int64_t rows, int64_t cols, int groupsize,
                              const void* x, int64_t ldx, const void* packed) {
  // ldx < 2^23: a token tile's lane offsets (< 128 rows of 2 ldx bytes) fit 32 bits;
  // the grid's work-items must fit 32 bits
  return (bits == 4 || bits == 8) && cols % KG == 0 &&
         (groupsize % KG == 0 || groupsize >= cols) && ldx % 8 == 0 &&
         ldx < ((int64_t)1 << 23) && (reinterpret_cast<uintptr_t>(x) & 15) == 0 &&
         (reinterpret_cast<uintptr_t>(packed) & 15) == 0 &&
         linear_blocks(bits, m, rows) * 64 * NWAVE <= (int64_t)UINT32_MAX;
}

hipError_t launch_linear_forward(int bits, const _Float16* x, int64_t ldx, int64_t m,
                                 const uint32_t* packed, int64_t rows, int64_t cols,
                                 const float* scales, const float* zeros, int groupsize, bool relu,
                                 _Float16* y, int64_t ldy, hipStream_t s) {
  if (bits == 4)
    return launch_bits<4>(x, ldx, m, packed, rows, cols, scales, zeros, groupsize, relu, y, ldy, s);
  return launch_bits<8>(x, ldx, m, packed, rows, cols, scales, zeros, groupsize, relu, y, ldy, s);
}

}  // namespace gptq
