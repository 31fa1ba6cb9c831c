// Q2_K down projection of one token per grid row (the single-token layer, and the
// direct path of a few tokens) on the block-scaled FP8 matrix instruction
// v_mfma_scale_f32_16x16x128_f8f6f4, with no weight decode beyond a shift and a
// mask per four weights.
//
// Q2_K (IQ2_XXS + Q2_K + FP8 hybrid card, format table; DeepSeek-V4.1-Flash mixed-Q2
// GGUF card, Recipe): a 256-weight superblock of 2-bit codes q with a 4-bit scale
// sc and a 4-bit min m per 16 weights and fp16 d, dmin per superblock; weight =
// d sc q - dmin m. A code zero-extended to a byte is an E4M3 subnormal, q 2^-9, so
// the crumbs of a 16-byte chunk become FP8 operand bytes with one shift and one
// mask per dword and plane, and a B scale of 2^9 makes them the exact integers q.
//
// Device layout of a row's superblock: 64 data bytes as four 16-byte chunks c; bits
// 2p..2p+1 of byte j of chunk c (c = 2 h + s) hold weight 128 h + 32 p + 16 s + j,
// so plane p of chunk c is the 16 weights of sub-block 8 h + 2 p + s in order. Its
// 20-byte scale record holds sc | m << 4 of the 16 sub-blocks, then d | dmin << 16.
//
// Operands. Lane (row n, group g) loads chunk g of row n's superblock and passes
// two planes as its 32 B bytes (p0 at K = 16 g + [0, 16), p1 at K = 64 + 16 g +
// [0, 16)). h (fp32) enters as four base-16 digits on a grid of each 16-value
// sub-block (h_digits below): integers of at most 32 in magnitude, exact E4M3
// values, each digit row with its own e8m0 scale. Inside one 32-wide scale block the
// instruction drops products more than 2^-13 below the block's largest (measured on
// the device; its sums across blocks are exact fp32), so floating E4M3 terms of h
// would keep only about 13 bits; with integer digits every product of a row is a
// multiple of one unit and at most 96 units, so each dot is exact and h keeps 17
// bits relative to its sub-block's maximum. A row 4 q + t carries digit t of the
// sub-block that lane group q supplies at one of those two K ranges and zeros
// elsewhere, so two instructions per B operand (one per plane) give output lane
// (n, q), registers t = 0..3, the four digit products of sub-block (chunk q, plane
// p) of row n: exactly the sub-block whose scale byte that lane holds. The lane
// sums the digits' products, multiplies by sc, and adds m times the sub-block's
// exact sum of h for the min term; d and dmin apply once per superblock.
//
// Work: a work-group takes 16 output rows for all routed slots of its token, two
// waves per slot (half of K each). Every wave issues its scale-record and weight
// loads before it converts h; the slots' partial sums are combined in LDS in slot
// order with the route weights.
#include <hip/hip_runtime.h>

#include "moeq_device.h"
#include "moeq_kernels.h"

namespace moeq {

namespace {

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int QD_TERMS = 4;                         // digits of h
constexpr int QD_KPARTS = 2;                        // waves per slot
constexpr int QD_SB = 4;                            // superblocks per wave
constexpr int QD_KMAX = 256 * QD_SB * QD_KPARTS;    // 2048
constexpr int QD_SLOTS = 6;                         // routed slots (top-6)
constexpr int QD_REC = 5;                           // dwords of a scale record
constexpr int QD_WREC = 16 * QD_SB * QD_REC;        // a wave's records: 320 dwords

// Four digits of 4 NQ consecutive fp32 values (a Q2_K sub-block for NQ = 4, two for
// NQ = 8; v: NQ loads of 4 values) on a grid of their own, in base 2^STEP. With M
// their largest magnitude and s the exponent with M / 2^s in [16, 32), digit t is an
// integer on the grid 2^(s - STEP t): d_t = rint(r_t / 2^(s - STEP t)) if that is at
// most 16 in magnitude, else twice rint(r_t / 2^(s - STEP t + 1)) (E4M3 holds every
// integer up to 16 but only even ones up to 32), with r_0 = v and r_(t+1) = r_t -
// d_t 2^(s - STEP t) (exact in fp32). |r_0| < 2^(s + 5) and each later |r_t| is at
// most one grid step of the digit before, so every |d_t| <= 32 is an exact E4M3
// value (for STEP = 4 the later digits stay within 16 and skip the even case), and
// |v - sum_t d_t 2^(s - STEP t)| <= 2^(s - 4 STEP + 3): 2^-17 M for STEP = 4 and
// 2^-19 M for STEP = 5. store(t, j, code) gets the E4M3 codes of digit t of values
// 4j .. 4j + 3, scale(t, E) its e8m0 code E = s - STEP t + 127 (clamped at 0, where
// the grid only gets coarser for tiny M). (h_digits_of: the same for values that are
// part of a larger block, whose largest magnitude is amax.)
template <int NQ, int STEP, class Store, class Scale>
__device__ __forceinline__ void h_digits_of(const u32x4 (&v)[NQ], float amax, Store&& store, Scale&& scale) {
  float x[4 * NQ];
#pragma unroll
  for (int i = 0; i < NQ; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) x[4 * i + j] = u2f(v[i][j]);
  const int s = (int)((f2u(amax) >> 23) & 0xFFu) - 131;  // floor(log2 M) - 4 (zero or subnormal M: -131)
#pragma unroll
  for (int t = 0; t < 4; t++) {
    const int st = max(s - STEP * t, -127);
    const float inv = u2f((uint32_t)(127 - st) << 23);  // 2^-st
    const float sc = e8m0_f32((uint32_t)(st + 127));     // 2^st
#pragma unroll
    for (int j = 0; j < NQ; j++) {
      float d[4];
#pragma unroll
      for (int k = 0; k < 4; k++) {
        const float q = x[4 * j + k] * inv;
        d[k] = __builtin_rintf(q);
        if (t == 0 || STEP > 4) d[k] = __builtin_fabsf(q) <= 16.f ? d[k] : 2.f * __builtin_rintf(0.5f * q);
        x[4 * j + k] = __builtin_fmaf(-d[k], sc, x[4 * j + k]);
      }
      const i16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(i16x2_t{0, 0}, d[0], d[1], 1.0f, false);
      const i16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, d[2], d[3], 1.0f, true);
      store(t, j, __builtin_bit_cast(uint32_t, hi));
    }
    scale(t, (uint32_t)(st + 127));
  }
}

template <int NQ, int STEP, class Store, class Scale>
__device__ __forceinline__ void h_digits(const u32x4 (&v)[NQ], Store&& store, Scale&& scale) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < NQ; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) amax = __builtin_fmaxf(amax, __builtin_fabsf(u2f(v[i][j])));
  h_digits_of<NQ, STEP>(v, amax, store, scale);
}

struct QdStage {
  uint8_t code[QD_TERMS][QD_SLOTS * QD_KMAX];       // E4M3 codes of h's digits, [slot][k]
  uint8_t sc[QD_TERMS][QD_SLOTS * QD_KMAX / 16];    // their e8m0 per 16 (sub-block)
  float hsum[QD_SLOTS * QD_KMAX / 16];              // exact sub-block sums, [slot][superblock][chunk][plane]
  uint32_t rec[QD_SLOTS * QD_KPARTS][QD_WREC];      // each wave's scale records, [row][superblock][dword]
};

// MOEQ_DQ_WPE: a minimum of waves per SIMD for the register allocation (6 would fit
// two work-groups per CU in 80 VGPRs, but spills a weight chunk).
#ifndef MOEQ_DQ_WPE
#define MOEQ_DQ_WPE 0
#endif
#if MOEQ_DQ_WPE
#define QD_ATTR __attribute__((amdgpu_waves_per_eu(MOEQ_DQ_WPE)))
#else
#define QD_ATTR
#endif
__global__ __launch_bounds__(64 * QD_KPARTS * QD_SLOTS) QD_ATTR void k_down1_q2k(Down1Params P) {
  __shared__ QdStage st;
  __shared__ float red[QD_SLOTS * QD_KPARTS][16];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot = wave / QD_KPARTS, part = wave % QD_KPARTS;
  const int n0 = blockIdx.x * 16;
  const int K = P.cols;
  const int nsb = K / 256;
  // Token blockIdx.y: its slots' ids, route weights, h and y.
  const int32_t* ids = P.ids + (size_t)blockIdx.y * P.top_k;
  const float* rwt = P.rw + (size_t)blockIdx.y * P.top_k;
  const float* ht = P.h + (size_t)blockIdx.y * P.top_k * K;
  float* yt = P.y + (size_t)blockIdx.y * P.rows;
  const int e = ids[slot];
  const bool ok = e >= 0 && e < P.n_experts;

  // Route weights and h first (thread t converts values 16t .. 16t + 15 of the
  // slots' concatenated h, [top_k][K]; threads past the end re-read the last 16).
  const int total = P.top_k * K;
  const int v0i = min(16 * (int)threadIdx.x, total - 16);
  const float rwv = rwt[min(lane, P.top_k - 1)];
  const float* hp = ht + v0i;
  const u32x4 hv[4] = {ld16(hp), ld16(hp + 4), ld16(hp + 8), ld16(hp + 12)};
  __builtin_amdgcn_sched_barrier(0);

  // The wave's superblocks [s0, s0 + my_sb); past the end, loads re-read the last.
  const int spw = (nsb + QD_KPARTS - 1) / QD_KPARTS;
  const int s0 = part * spw;
  const int my_sb = max(0, min(spw, nsb - s0));
  const int ec = ok ? e : 0;
  // Scale records of rows n0 .. n0 + 15 for the wave's superblocks: dword
  // d = lane + 64 j is dword d % 5 of record (row d / 20, superblock (d / 5) % 4).
  const uint8_t* sbase = P.w.scales + (size_t)ec * P.w.sestride;
  uint32_t rv[QD_WREC / 64];
#pragma unroll
  for (int j = 0; j < QD_WREC / 64; j++) {
    const int d = lane + 64 * j;
    const int r = min(n0 + d / (QD_SB * QD_REC), P.rows - 1);
    const int sbg = min(s0 + (d / QD_REC) % QD_SB, nsb - 1);
    rv[j] = *reinterpret_cast<const uint32_t*>(sbase + ((size_t)r * nsb + sbg) * (4 * QD_REC) + 4 * (d % QD_REC));
  }
  const int n = lane & 15, g = lane >> 4;
  const int rn = min(n0 + n, P.rows - 1);
  const uint8_t* wd = P.w.data + (size_t)ec * P.w.estride + (size_t)rn * nsb * 64 + 16 * g;
  u32x4 q[QD_SB];
#pragma unroll
  for (int i = 0; i < QD_SB; i++) q[i] = ld16(wd + (size_t)min(s0 + min(i, max(my_sb - 1, 0)), nsb - 1) * 64);
  __builtin_amdgcn_sched_barrier(0);

  // h -> four digits and the exact sum of each 16-value sub-block.
  if (16 * (int)threadIdx.x < total) {
    h_digits<4, 4>(
        hv, [&](int t, int j, uint32_t w) { *reinterpret_cast<uint32_t*>(&st.code[t][v0i + 4 * j]) = w; },
        [&](int t, uint32_t E) { st.sc[t][v0i / 16] = (uint8_t)E; });
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; i++) s += (u2f(hv[i][0]) + u2f(hv[i][1])) + (u2f(hv[i][2]) + u2f(hv[i][3]));
    // sub-block j of the slot (j = 16 sb + 8 h + 2 p + s) -> [sb][chunk 2 h + s][plane p]
    const int sl = v0i / K, j = (v0i % K) / 16;
    const int c = 2 * ((j >> 3) & 1) + (j & 1), p = (j >> 1) & 3;
    st.hsum[sl * (K / 16) + (j & ~15) + 4 * c + p] = s;
  }
#pragma unroll
  for (int j = 0; j < QD_WREC / 64; j++) st.rec[wave][lane + 64 * j] = rv[j];
  __syncthreads();

  const int hb = slot * K;
  const int t = n & 3, qa = n >> 2;  // A row n = 4 qa + t: term t of lane group qa's sub-block
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < QD_SB; i++) {
    if (i < my_sb) {
      const int sb = s0 + i;
      const uint32_t* rec = &st.rec[wave][(n * QD_SB + i) * QD_REC];
      const int hh = g >> 1, ss = g & 1;
      // sc | m << 4 of planes 0, 1 (bytes 0, 2) and 2, 3 (bytes 0, 2)
      const uint32_t sw[2] = {rec[2 * hh] >> (8 * ss), rec[2 * hh + 1] >> (8 * ss)};
      const uint32_t dd = rec[4];
      const f32x4_t hs = *reinterpret_cast<const f32x4_t*>(&st.hsum[slot * (K / 16) + 16 * sb + 4 * g]);
      float acc_s = 0.f, acc_m = 0.f;
#pragma unroll
      for (int pp = 0; pp < 2; pp++) {
        // registers 0-3: plane 2 pp of the chunk, 4-7: plane 2 pp + 1
        i32x8_t bv;
#pragma unroll
        for (int j = 0; j < 4; j++) {
          bv[j] = (int32_t)((q[i][j] >> (4 * pp)) & 0x03030303u);
          bv[4 + j] = (int32_t)((q[i][j] >> (4 * pp + 2)) & 0x03030303u);
        }
#pragma unroll
        for (int half = 0; half < 2; half++) {
          const int p = 2 * pp + half;
          u32x4 a = u32x4{0u, 0u, 0u, 0u};
          int sa = 0;
          {
            const int pos = hb + 256 * sb + 128 * (qa >> 1) + 32 * p + 16 * (qa & 1);
            sa = st.sc[t][pos / 16];
            if (qa == g) a = *reinterpret_cast<const u32x4*>(&st.code[t][pos]);
          }
          const u32x4 z = u32x4{0u, 0u, 0u, 0u};
          const i32x8_t av = half == 0 ? __builtin_bit_cast(i32x8_t, __builtin_shufflevector(a, z, 0, 1, 2, 3, 4, 5, 6, 7))
                                       : __builtin_bit_cast(i32x8_t, __builtin_shufflevector(z, a, 0, 1, 2, 3, 4, 5, 6, 7));
          // B scale 2^9: the E4M3 subnormal codes q become the integers q.
          const f32x4_t cr =
              __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, sa, 0, 136);
          const uint32_t sm = sw[pp] >> (16 * half);
          acc_s = __builtin_fmaf((float)(sm & 15u), (cr[0] + cr[1]) + (cr[2] + cr[3]), acc_s);
          acc_m = __builtin_fmaf((float)((sm >> 4) & 15u), hs[p], acc_m);
        }
      }
      acc = __builtin_fmaf(half_bits_f32(dd), acc_s, acc);
      acc = __builtin_fmaf(-half_bits_f32(dd >> 16), acc_m, acc);
    }
  }
  // Loads past the wave's last superblock are never used: let them land first.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // the four chunks of each superblock: lane groups of column n
  acc += __shfl_xor(acc, 16, 64);
  acc += __shfl_xor(acc, 32, 64);
  if (lane < 16) red[wave][lane] = ok ? acc : 0.f;
  __syncthreads();
  if (threadIdx.x < 16) {
    float y = 0.f;
    for (int k = 0; k < P.top_k; k++) {
      float pk = 0.f;
#pragma unroll
      for (int h = 0; h < QD_KPARTS; h++) pk += red[k * QD_KPARTS + h][threadIdx.x];
      y += pk * u2f(__builtin_amdgcn_readlane(f2u(rwv), k));
    }
    const int r = n0 + (int)threadIdx.x;
    if (r < P.rows) yt[r] = y;
  }
  if (!ok && blockIdx.x == 0 && lane == 0 && part == 0) atomicOr(P.err, 1u);
}


// ---------------------------------------------------------------- token-grouped (T > 1)
// The down projection of a batch, each routed expert's weights read once for all of
// its pairs, on the same instruction. The weights stay operand B (16 columns = 16
// weight rows; lane (row n, group g) holds chunk g of the row's superblock, planes
// 2 pp and 2 pp + 1 as its two 16-byte halves in pass pp). Q2_K's sub-block scale
// and min are folded into B: with sc = sl + 4 sh (sl, sh < 4) the products sl q and
// sh q (at most 9) and the min m (at most 15) are integers below 16, and E4M3 codes
// 0 .. 15 are exactly the values c 2^-9 (the subnormals and the first binade share
// one spacing), so a byte-wise multiply of the crumbs makes each operand and the B
// scales 2^9, 2^11 and 2^9 make them sl q, 4 sh q and m. A whole 128-wide K step then
// accumulates in one instruction: for a row, sum over K of (sl + 4 sh) q h = sc sum q h
// per sub-block, and sum of m h = m times the sub-block's sum of h; only d and dmin
// remain, once per superblock.
//
// Operand A: four pairs by four digits (row 4 i + t: digit t of pair i) of h, now on
// the grid of each 32-value block, since every row spans the four scale blocks of
// the step; a block's two sub-blocks sit in one scale block of the instruction (the
// halves of lane groups 0, 1 or 2, 3). The digits are base 32 here (base 16 on the
// wider grid kept too few bits: 1.0e-4 elementwise against the oracle). Digits and
// products stay integers (at most 32 times 15 units), so each dot is exact and h
// keeps 19 bits relative to its block's maximum. Output lane (n, g) register t is digit t of pair g against row n.
//
// k_q2k_digits writes every pair's digits once per step, in the operand order: per
// (pair, superblock) 1024 code bytes [pp][half][group][digit][16] and 32 scale bytes
// [pp][digit][scale group]. A work-group (one expert, 64 weight rows in four waves)
// loads its weights and scale records for all of K into registers, then copies the
// digits of up to 4 NG of the expert's pairs into LDS (one 16-byte piece per lane,
// straight from memory into the operand order) and runs the pass; an expert with
// more pairs takes further passes over the same weight registers. Outputs are
// route-weighted partials per (pair, row) for the combine. One group per pass (NG =
// 1: 34 KB of LDS, three work-groups per CU) ran faster than two (67.5 KB, two per
// CU) at every batch measured, from 2 to 48 pairs per expert.
constexpr int QG_WAVES = 4;
constexpr int QG_ROWS = 16 * QG_WAVES;
constexpr int QG_SB = 8;  // superblocks along K (K <= 2048)
constexpr int QG_WLOADS = QG_SB;  // a wave's weight loads (the records go through LDS)

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// Bytes of x (each below 4) times f (below 4), byte by byte: one 16-bit pair multiply.
__device__ __forceinline__ uint32_t crumb_mul(uint32_t x, uint32_t f) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2_t, x) * __builtin_bit_cast(u16x2_t, f * 0x10001u));
}

// Four lanes per 32-value block of h (8 values each; the block's largest magnitude
// by two lane exchanges): its four digits and their e8m0 codes.
__global__ __launch_bounds__(256) void k_q2k_digits(const float* __restrict__ h, int nval8, int nsb,
                                                    uint8_t* __restrict__ dq, uint8_t* __restrict__ dsc) {
  const int i8 = blockIdx.x * 256 + (int)threadIdx.x;  // 8-value piece; nval8 is a multiple of 4
  if (i8 >= nval8) return;                              // whole groups of four leave together
  const int b = i8 >> 2, q = i8 & 3;
  const int pair = b / (8 * nsb), r = b % (8 * nsb), sb = r >> 3, kb = r & 7;
  const float* src = h + (size_t)i8 * 8;  // [pair][K]: piece i8 starts at value 8 i8
  const u32x4 v[2] = {ld16(src), ld16(src + 4)};
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) amax = __builtin_fmaxf(amax, __builtin_fabsf(u2f(v[i][j])));
  amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1, 4));
  amax = __builtin_fmaxf(amax, __shfl_xor(amax, 2, 4));
  // Sub-blocks 2 kb, 2 kb + 1 of the superblock: pass pp, half, lane groups g0, g0 + 1
  // (values 0-15 and 16-31 of the block, piece q in sub-block q >> 1 at byte 8 (q & 1));
  // the scale of the pair's 32-wide block comes from lane group gs.
  const int pp = (kb >> 1) & 1, half = kb & 1, g0 = 2 * (kb >> 2), gs = 2 * (kb & 1) + (kb >> 2);
  uint8_t* cb = dq + ((size_t)pair * nsb + sb) * 1024 + (pp * 2 + half) * 256 + (g0 + (q >> 1)) * 64 + 8 * (q & 1);
  uint8_t* sbp = dsc + ((size_t)pair * nsb + sb) * 32 + pp * 16 + gs;
  uint32_t w[4][2];
  h_digits_of<2, 5>(
      v, amax, [&](int t, int j, uint32_t code) { w[t][j] = code; },
      [&](int t, uint32_t E) {
        if (q == 0) sbp[4 * t] = (uint8_t)E;
      });
#pragma unroll
  for (int t = 0; t < 4; t++) *reinterpret_cast<u32x2*>(cb + 16 * t) = u32x2{w[t][0], w[t][1]};
}

// The three B operands of pass pp (planes 2 pp and 2 pp + 1 of the lane's chunk q):
// sl q, sh q and m as E4M3 codes 0 .. 15, from rs = the scale/min bytes of the two
// planes' sub-blocks in bytes 0 and 2.
__device__ __forceinline__ void qg_operands(const u32x4& q, uint32_t rs, int pp, i32x8_t& B1, i32x8_t& B2,
                                            i32x8_t& B3) {
  const uint32_t b0 = rs & 0xFFu, b1 = (rs >> 16) & 0xFFu;
  const uint32_t mn = (rs >> 4) & 0x000F000Fu;  // the two mins in bytes 0 and 2
  const uint32_t m0 = __builtin_amdgcn_perm(mn, mn, 0x00000000u), m1 = __builtin_amdgcn_perm(mn, mn, 0x02020202u);
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const uint32_t x0 = (q[j] >> (4 * pp)) & 0x03030303u, x1 = (q[j] >> (4 * pp + 2)) & 0x03030303u;
    B1[j] = (int32_t)crumb_mul(x0, b0 & 3u);
    B1[4 + j] = (int32_t)crumb_mul(x1, b1 & 3u);
    B2[j] = (int32_t)crumb_mul(x0, (b0 >> 2) & 3u);
    B2[4 + j] = (int32_t)crumb_mul(x1, (b1 >> 2) & 3u);
    B3[j] = (int32_t)m0;
    B3[4 + j] = (int32_t)m1;
  }
}

// The instruction with A's scale taken from byte sel of sa (sel a constant once the
// callers' loops are unrolled).
__device__ __forceinline__ f32x4_t mfma_sel(const i32x8_t& a, const i32x8_t& b, const f32x4_t& c, int sel, int sa,
                                            int sbv) {
  switch (sel) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sbv);
    case 1: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 1, sa, 0, sbv);
    case 2: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 2, sa, 0, sbv);
    default: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 3, sa, 0, sbv);
  }
}

template <int NG>
struct QgStage {
  u32x4 code[QG_SB][NG][2][2][64];  // [sb][group][pp][half][lane]: lane 16 g + 4 i + t's A bytes
  uint32_t sc[QG_SB][64];           // [sb][lane]: byte 2 G + pp = the lane's e8m0 for group G, pass pp
};

template <int NG>
__global__ __launch_bounds__(64 * QG_WAVES) void k_dn_q2k_g(GemvParams P, const uint8_t* __restrict__ dq,
                                                            const uint8_t* __restrict__ dsc) {
  // Each wave's 16 rows of scale records (20 bytes per row and superblock), copied
  // in once: read from memory by every lane, each record dword came from 16 rows'
  // lines per instruction, two instructions per superblock against one for the
  // weights (IQ2_XXS + Q2_K layer at T = 64: 537 against 517 us).
  __shared__ uint32_t srec[QG_WAVES][16 * QG_SB * 5];
  constexpr int CH = 4 * NG;  // pairs per pass
  __shared__ QgStage<NG> st;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int slot = blockIdx.y;
  if (slot >= P.route.n_slots()[0]) return;
  const int e = P.route.slots()[slot];
  const int pstart = P.route.offsets()[e];
  const int M = P.route.offsets()[e + 1] - pstart;
  const int r0 = blockIdx.x * QG_ROWS;
  if (r0 >= P.rows || M <= 0) return;  // uniform per work-group: the barriers below are reached by all
  const int32_t* perm = P.route.perm() + pstart;

  if (e < 0 || e >= P.n_experts) {
    // Out-of-range expert id (its bucket): its pairs contribute nothing.
    for (int m = 0; m < M; m++)
      for (int i = threadIdx.x; i < QG_ROWS; i += 64 * QG_WAVES)
        if (r0 + i < P.rows) P.out[(size_t)perm[m] * P.rows + r0 + i] = 0.f;
    return;
  }

  const int nsb = P.cols / 256;
  const int n0 = r0 + 16 * wave;
  const int rn = min(n0 + n, P.rows - 1);
  // row rn of the expert: its data and its scale records
  const uint8_t* wrow = P.w[0].data + (size_t)e * P.w[0].estride + (size_t)rn * nsb * 64 + 16 * g;
  // the records of rows rb .. rb + nrow - 1 (the wave's rows, or the expert's last
  // row for a wave past the end), contiguous in the scale plane
  const int rb = min(n0, P.rows - 1), nrow = max(1, min(16, P.rows - rb));
  const int nrec = nrow * nsb * 5;  // dwords
  const __amdgpu_buffer_rsrc_t rec_buf = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(P.w[0].scales + (size_t)e * P.w[0].sestride + (size_t)rb * nsb * 20), (short)0,
      0x7FFFFFFF, 0x00020000);
  const uint32_t* srow = &srec[wave][(rn - rb) * nsb * 5];
  const int t = lane & 3, ip = (lane >> 2) & 3;  // this lane's A row: digit t of pair 4 G + ip
  int pa[NG], po[NG];
  float rwo[NG];
  u32x2 sv = u32x2{0u, 0u};
  const int pl = threadIdx.x >> 5, sx = (threadIdx.x >> 2) & 7, pc = threadIdx.x & 3;
  const bool scl = pl < CH && sx < nsb;
  // A pass's stage, first half: its pair ids and route weights, the digit codes copied
  // straight into LDS (wave w copies the (pass w >> 1, half w & 1) pieces of every
  // superblock and group, lane l = 16 g + 4 ip + t taking (pair 4 G + ip, group g,
  // digit t)), and the loads of its scale codes (thread (pair pl, superblock sx, piece
  // pc): 8 bytes [pp][t][gs]).
  auto stage_issue = [&](int c0) {
#pragma unroll
    for (int G = 0; G < NG; G++) {
      pa[G] = perm[min(c0 + 4 * G + ip, M - 1)];  // pairs past the last repeat it and are not stored
      po[G] = perm[min(c0 + 4 * G + g, M - 1)];
    }
    const int pid = perm[min(c0 + pl, M - 1)];
    const int pp = wave >> 1, half = wave & 1;
#pragma unroll
    for (int i = 0; i < QG_SB; i++)
#pragma unroll
      for (int G = 0; G < NG; G++)
        if (i < nsb) {
          const uint8_t* src = dq + ((size_t)pa[G] * nsb + i) * 1024 + (pp * 2 + half) * 256 + g * 64 + t * 16;
          __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)&st.code[i][G][pp][half][0], 16, 0, 0);
        }
    if (scl) sv = *reinterpret_cast<const u32x2*>(dsc + ((size_t)pid * nsb + sx) * 32 + 8 * pc);
#pragma unroll
    for (int G = 0; G < NG; G++) rwo[G] = P.rw[po[G]];
  };
  // Second half: the scale codes into the lanes' bytes.
  auto stage_store = [&]() {
    if (scl) {
      uint8_t* dst = reinterpret_cast<uint8_t*>(&st.sc[sx][0]);
      const int pp = pc >> 1;
#pragma unroll
      for (int k = 0; k < 8; k++) {
        const int tt = 2 * (pc & 1) + (k >> 2), gs = k & 3;
        dst[4 * (16 * gs + 4 * (pl & 3) + tt) + 2 * (pl >> 2) + pp] = (uint8_t)(sv[k >> 2] >> (8 * (k & 3)));
      }
    }
  };

  // The first pass's stage and the records go out before the weights, so that the
  // wait for them below leaves the weight loads in flight and each superblock waits
  // only for its own. All of K for row rn: chunk g of each superblock (superblocks
  // past the end re-read the last and are not used), QG_WLOADS loads. Lane (n, g)
  // later takes from its row's records the dwords of chunk g's sub-blocks (planes
  // 0, 1: dword 2 (g >> 1); planes 2, 3: the next) and d | dmin.
  stage_issue(0);
  __builtin_amdgcn_sched_barrier(0);
  // the wave's records straight into LDS, one dword per lane per load
  for (int k = 0; 64 * k < nrec; k++)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rec_buf, (lds_void_t*)&srec[wave][64 * k], 4,
                                             4 * min(64 * k + lane, nrec - 1), 0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  u32x4 q[QG_SB];
#pragma unroll
  for (int i = 0; i < QG_SB; i++) q[i] = ld16(wrow + min(i, nsb - 1) * 64);
  __builtin_amdgcn_sched_barrier(0);

  // One pass over the stage (pairs c0 .. c0 + CH - 1). The empty asm at the top of
  // each superblock ties everything derived from its weight registers (and the wait
  // for them) to that superblock and pass: nothing is hoisted out of the passes
  // (eight superblocks' B operands would not fit in registers) or ahead of the
  // superblock's own loads.
  auto pass = [&](int c0) {
    const int ng = min(NG, (M - c0 + 3) / 4);  // groups holding pairs (uniform)
    f32x4_t acc[NG];
#pragma unroll
    for (int G = 0; G < NG; G++) acc[G] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < QG_SB; i++) {
      if (i < nsb) {
        uint32_t rlo_i = srow[5 * i + 2 * (g >> 1)], rhi_i = srow[5 * i + 2 * (g >> 1) + 1], rdd_i = srow[5 * i + 4];
        asm volatile("" : "+v"(q[i]), "+v"(rlo_i), "+v"(rhi_i), "+v"(rdd_i));
        const int sa = (int)st.sc[i][lane];
        f32x4_t cr[NG], cm[NG];
#pragma unroll
        for (int pp = 0; pp < 2; pp++) {
          i32x8_t B1, B2, B3;
          qg_operands(q[i], (pp ? rhi_i : rlo_i) >> (8 * (g & 1)), pp, B1, B2, B3);
#pragma unroll
          for (int G = 0; G < NG; G++) {
            if (G < ng) {
              const u32x4 lo = st.code[i][G][pp][0][lane], hi = st.code[i][G][pp][1][lane];
              const i32x8_t A = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
              const f32x4_t z = f32x4_t{0.f, 0.f, 0.f, 0.f};
              // B scales 2^9, 2^11, 2^9: sl q, 4 sh q, m
              cr[G] = mfma_sel(A, B1, pp ? cr[G] : z, 2 * G + pp, sa, 136);
              cr[G] = mfma_sel(A, B2, cr[G], 2 * G + pp, sa, 138);
              cm[G] = mfma_sel(A, B3, pp ? cm[G] : z, 2 * G + pp, sa, 136);
            }
          }
        }
        const float d = half_bits_f32(rdd_i), dmin = half_bits_f32(rdd_i >> 16);
#pragma unroll
        for (int G = 0; G < NG; G++)
          if (G < ng)
#pragma unroll
            for (int r = 0; r < 4; r++) acc[G][r] = __builtin_fmaf(d, cr[G][r], __builtin_fmaf(-dmin, cm[G][r], acc[G][r]));
      }
    }
    // Lane (n, g): pair 4 G + g of the pass, weight row n0 + n.
#pragma unroll
    for (int G = 0; G < NG; G++) {
      if (G < ng && c0 + 4 * G + g < M && n0 + n < P.rows) {
        const float v = (acc[G][0] + acc[G][1]) + (acc[G][2] + acc[G][3]);
        P.out[(size_t)po[G] * P.rows + n0 + n] = v * rwo[G];
      }
    }
  };

  stage_store();
  // the first stage's copies, issued before the QG_WLOADS weight loads
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(QG_WLOADS) : "memory");
  __syncthreads();
  pass(0);
  for (int c0 = CH; c0 < M; c0 += CH) {
    __syncthreads();  // the previous pass has read the stage
    stage_issue(c0);
    stage_store();
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the copies into LDS have landed
    __syncthreads();
    pass(c0);
  }
}

}  // namespace

// K a multiple of 256 up to 2048, at most 6 slots.
bool down1_q2k_fits(int rows, int cols, int top_k) {
  return rows > 0 && cols > 0 && cols % 256 == 0 && cols <= QD_KMAX && top_k >= 1 && top_k <= QD_SLOTS;
}

hipError_t launch_down1_q2k(const Down1Params& p, hipStream_t s) {
  if (!down1_q2k_fits(p.rows, p.cols, p.top_k)) return hipErrorInvalidValue;
  dim3 g((unsigned)((p.rows + 15) / 16), (unsigned)(p.T > 1 ? p.T : 1)), b((unsigned)(64 * QD_KPARTS * p.top_k));
  hipLaunchKernelGGL(k_down1_q2k, g, b, 0, s, p);
  return hipGetLastError();
}


bool dn_q2k_g_fits(int rows, int cols) { return rows > 0 && cols > 0 && cols % 256 == 0 && cols <= 256 * QG_SB; }

size_t dn_q2k_g_digit_bytes(long pairs, int cols) { return (size_t)pairs * (size_t)cols * 4; }
size_t dn_q2k_g_scale_bytes(long pairs, int cols) { return (size_t)pairs * (size_t)cols / 8; }

hipError_t launch_dn_q2k_g(const GemvParams& p, int n_slots, uint8_t* dq, uint8_t* dsc, hipStream_t s) {
  if (!dn_q2k_g_fits(p.rows, p.cols) || (uintptr_t)p.act % 16 || (uintptr_t)dq % 16 || (uintptr_t)dsc % 8)
    return hipErrorInvalidValue;
  const long nval8 = (long)p.T * p.top_k * (p.cols / 8);
  if (nval8 <= 0 || nval8 > (long)0x7FFFFFFF - 255) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_q2k_digits, dim3((unsigned)((nval8 + 255) / 256)), dim3(256), 0, s, (const float*)p.act,
                     (int)nval8, p.cols / 256, dq, dsc);
  const dim3 g((unsigned)((p.rows + QG_ROWS - 1) / QG_ROWS), (unsigned)n_slots), b(64 * QG_WAVES);
  hipLaunchKernelGGL(k_dn_q2k_g<1>, g, b, 0, s, p, dq, dsc);
  return hipGetLastError();
}

}  // namespace moeq
