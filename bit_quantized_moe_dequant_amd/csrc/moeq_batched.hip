// Batched decode of MXFP4 experts on the block-scaled matrix instruction
// v_mfma_scale_f32_16x16x128_f8f6f4: a few tokens per routed expert, as when N
// decode sessions are co-scheduled and each step's tokens are grouped by expert
// (DeepSeekv4 Flash for 1x Spark forum thread, second post, "Next up": one
// weight sweep over N co-scheduled sessions). Each expert's weights are read
// once per step and fed to the instruction as they sit in memory (FP4 operand B,
// e8m0 block scale as the B scale); no weight is decoded on the VALU.
//
// The tokens are operand A as E4M3 terms with e8m0 scales per 32, their rows
// carrying (pair, term) couples:
//   * gate/up: x (bf16) as two terms; rows 2j, 2j + 1 = pair j of a staged tile
//     (up to eight per instruction; two staged, see MOEQ_GU_TILE_MX)
//     (the split is exact to 2^-21.8 of each 32-block's maximum);
//   * down: h (fp32) as three terms; rows 3j .. 3j + 2 = pair j of a staged tile
//     (up to five per instruction; two staged, see MOEQ_DN_TILE)
//     (about 12 significant bits of h).
// A pair is a (token, slot) of the routing; the route table (the counting sort of
// the pairs by expert) gives each work-group its expert and the expert's pairs.
//
// Work: a work-group is (routed expert, 16 weight rows), four waves on contiguous
// runs of K steps; a wave issues the first tile's
// activation loads, then all of its weight loads, then converts the activations
// (waiting only for them); the weights stay in registers and serve every tile of
// the expert's pairs; the waves' partial sums meet in LDS and are added in wave
// order.
// Gate/up writes h[pair][row] = silu(g) * u; down writes route-weighted partials
// [pair][row] for the slot-order combine. The bucket of out-of-range ids writes
// zeros.
//
// NVFP4 gate/up (e2m1 codes, an E4M3 scale per 16 along K, an fp32 scale_2 per
// expert tensor: DeepSeek V4 Flash - REAP K180 Mixed NVFP4 card, section "NVFP4:
// lossless MXFP4->NVFP4 conversion") runs in the same kernel with the single-token
// kernel's operand layout: its block scale is neither a power of two nor 32 wide,
// so B takes scale 1 and each instruction serves one pair, A row 8 t + d carrying
// term t of x on 16-block d of the step (zeros elsewhere); the lane holding output
// rows 4 q .. 4 q + 3 multiplies them by their blocks' E4M3 scales (one 32-bit word
// of the row's scale plane, converted once per step for all pairs of the tile).
#include <hip/hip_runtime.h>

#include "moeq_device.h"
#include "moeq_kernels.h"

namespace moeq {

namespace {

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int GB_WAVES = 4;         // down: four waves of up to eight K steps (K <= 2048 uses four)
constexpr int GB_NT = 64 * GB_WAVES;
constexpr int GB_STEPS = 8;
#ifndef MOEQ_DN_ROWSPLIT
#define MOEQ_DN_ROWSPLIT 1
#endif
// Down work split: 1 = each wave takes its own 16 weight rows over all of K (64 rows
// per work-group); 0 = the four waves take quarters of K of the same 16 rows.
constexpr bool DN_ROWSPLIT = MOEQ_DN_ROWSPLIT;
constexpr int DN_ROWS = DN_ROWSPLIT ? 16 * GB_WAVES : 16;  // weight rows per work-group
#ifndef MOEQ_GU_G_WAVES
#define MOEQ_GU_G_WAVES 4
#endif
constexpr int GU_WAVES = MOEQ_GU_G_WAVES;  // gate/up waves; their K steps cover K <= 4096
constexpr int GU_NT = 64 * GU_WAVES;
constexpr int GU_STEPS = 32 / GU_WAVES;
// Gate/up pairs staged per tile: two. MXFP4: an instruction's 16 A rows could take
// eight pairs of two terms, but at the loads this path serves most experts have one
// or two pairs, and the smaller stage fits three work-groups per CU instead of two
// (the MXFP4 layer at T = 64 / 96 took 725 / 882 us with eight-pair tiles, 704 / 862
// with four, 645 / 802 with two). NVFP4 (one pair per instruction): with two the
// kernel fits 147 VGPRs and three work-groups per CU (NVFP4 + Q2_K at T = 64 / 256:
// 583 / 1485 us with four-pair tiles, 510 / 1269 with two).
#ifndef MOEQ_GU_TILE_MX
#define MOEQ_GU_TILE_MX 2
#endif
#ifndef MOEQ_GU_TILE_NV
#define MOEQ_GU_TILE_NV 2
#endif
constexpr int GU_KMAX = 4096;
// Down pairs per staged tile (three terms each; an instruction's A rows hold at most
// five): two, so that the h staging registers allow four waves per SIMD (110 VGPRs,
// 17 KB of LDS). The MXFP4 layer at T = 48 / 64 / 96 took 545 / 645 / 803 us with
// five-pair tiles, 543 / 649 / 824 with three, 511 / 614 / 781 with two.
#ifndef MOEQ_DN_TILE
#define MOEQ_DN_TILE 2
#endif
constexpr int DN_TILE = MOEQ_DN_TILE;
static_assert(DN_TILE >= 1 && DN_TILE <= 5, "an instruction's A rows hold at most five pairs");
constexpr int DN_KMAX = 2048;

// Wave w takes K steps [w spw, (w + 1) spw), spw a multiple of 4 (16-byte runs of
// scale bytes stay inside the row).
__device__ __forceinline__ int steps_per_wave(int nsteps, int waves) { return 4 * ((nsteps + 4 * waves - 1) / (4 * waves)); }

template <int TILE>
struct GuStage {
  uint8_t code[2][TILE * GU_KMAX];
  uint8_t sc[2][TILE * GU_KMAX / 32];
};

template <int FMT>
// A budget of three waves per SIMD (147 VGPRs for both formats, no spills; 155 for
// MXFP4 unasked): NVFP4 + Q2_K at T = 256 1265 -> 1224 us, T = 64 503 -> 498 us, the
// MXFP4 layer at T = 64 479.5 -> 476 us. Four waves spill 16-20 VGPRs and lose 25-40%.
__global__ __launch_bounds__(GU_NT) __attribute__((amdgpu_waves_per_eu(3))) void k_gu_fp4_g(GemvParams P) {
  constexpr bool NV = FMT == FMT_NVFP4;
  constexpr int SPB = NV ? 8 : 4;            // scale bytes per row and 128-wide step
  constexpr int NSB = GU_STEPS * SPB / 16;   // 16-byte scale runs per wave and row
  constexpr int TILE = NV ? MOEQ_GU_TILE_NV : MOEQ_GU_TILE_MX;  // pairs per staged tile
  static_assert(TILE >= 1 && TILE <= 8, "an instruction's A rows hold at most eight pairs");
  __shared__ GuStage<TILE> st;
  // partial sums per pair of one instruction: its 16 A rows hold up to eight pairs
  // (lane group g writes pairs 2g and 2g + 1 whatever the tile)
  __shared__ float red[GU_WAVES][2][8][16];
  __shared__ __attribute__((aligned(16))) uint8_t scs[GU_WAVES][2][1024];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot = blockIdx.y;
  if (slot >= P.route.n_slots()[0]) return;
  const int e = P.route.slots()[slot];
  const int pstart = P.route.offsets()[e];
  const int M = P.route.offsets()[e + 1] - pstart;
  const int n0 = blockIdx.x * 16;
  if (e >= P.n_experts) {  // out-of-range ids: their h rows are zero
    for (int i = threadIdx.x; i < M * 16; i += GU_NT) {
      const int r = n0 + (i & 15);
      if (r < P.rows) P.out[(size_t)P.route.perm()[pstart + (i >> 4)] * P.rows + r] = 0.f;
    }
    return;
  }
  const int K = P.cols;
  const int nsteps = K / 128;
  const int cpt = K / 16;
  const int spw = steps_per_wave(nsteps, GU_WAVES);
  const int s0 = wave * spw;
  const int my = max(0, min(spw, nsteps - s0));
  const int n = lane & 15, g = lane >> 4;
  const int rn = min(n0 + n, P.rows - 1);
  constexpr int XC = TILE * GU_KMAX / 16 / GU_NT;  // chunk loads per thread per tile, at most

  // A tile's tokens -> two E4M3 terms in LDS: stage_load issues the loads,
  // stage_convert converts and stores (it waits only for those loads).
  u32x4 xa[XC], xb[XC];
  auto stage_load = [&](int m0) {
    const int tn = min(TILE, M - m0);
    const int nc = (tn * cpt + GU_NT - 1) / GU_NT;  // uniform
#pragma unroll
    for (int j = 0; j < XC; j++) {
      xa[j] = u32x4{0u, 0u, 0u, 0u};
      xb[j] = xa[j];
      const int c = j * GU_NT + (int)threadIdx.x;
      if (j < nc && c < tn * cpt) {
        const int tok = P.route.perm()[pstart + m0 + c / cpt] / P.top_k;
        const uint16_t* xr = reinterpret_cast<const uint16_t*>(P.act) + (size_t)tok * K + (c % cpt) * 16;
        xa[j] = ld16(xr);
        xb[j] = ld16(xr + 8);
      }
    }
  };
  auto stage_convert = [&](int m0) {
    const int tn = min(TILE, M - m0);
    const int nc = (tn * cpt + GU_NT - 1) / GU_NT;  // uniform
#pragma unroll
    for (int j = 0; j < XC; j++) {
      if (j < nc) {
        const int c = j * GU_NT + (int)threadIdx.x;
        uint32_t w[2][4], E[2];
        bf16_terms(xa[j], xb[j], w, E);
        if (c < tn * cpt) {
          const int off = (c / cpt) * K + (c % cpt) * 16;
#pragma unroll
          for (int tm = 0; tm < 2; tm++) {
            *reinterpret_cast<u32x4*>(&st.code[tm][off]) = u32x4{w[tm][0], w[tm][1], w[tm][2], w[tm][3]};
            if ((c & 1) == 0) st.sc[tm][off / 32] = (uint8_t)E[tm];
          }
        }
      }
    }
  };

  // The first tile's activation loads, then every weight load of the wave, then the
  // conversion (which waits only for the activations).
  stage_load(0);
  __builtin_amdgcn_sched_barrier(0);
  u32x4 q[2][GU_STEPS];
  u32x4 sbv4[2][NSB];
  const float s2g = NV ? P.w[0].scale2[e] : 1.f, s2u = NV ? P.w[1].scale2[e] : 1.f;
  static_assert(16 * NSB <= 64, "a wave's scale runs fit one copy instruction per matrix");
  {
    // The wave's 16 rows' scale runs copied into LDS once: lane l takes run l % NSB
    // of row l / NSB (row r at bytes 16 NSB r of the wave's buffer). Loaded by each
    // lane instead, every run came from 16 rows' lines per instruction, four lanes
    // per row asking for the same bytes (NVFP4 + Q2_K at T = 64: 639 against 594 us,
    // the MXFP4 layer 741 against 725 us).
    const int pr = min(lane / NSB, 15), pc = lane % NSB;
    const int r = min(n0 + pr, P.rows - 1);
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
      const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(P.w[mt].scales + (size_t)e * P.w[mt].sestride), (short)0, 0x7FFFFFFF, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          sr, (__attribute__((address_space(3))) void*)&scs[wave][mt][0], 16,
          r * (K / 128 * SPB) + min(SPB * s0 + 16 * pc, SPB * nsteps - 16), 0, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // the copies before every weight load
#pragma unroll
  for (int mt = 0; mt < 2; mt++) {
    const uint8_t* wd = P.w[mt].data + (size_t)e * P.w[mt].estride + (size_t)rn * (K / 2);
#pragma unroll
    for (int i = 0; i < GU_STEPS; i++)
      q[mt][i] = ld16(wd + (size_t)min(s0 + min(i, max(my - 1, 0)), nsteps - 1) * 64 + 16 * g);
  }
  __builtin_amdgcn_sched_barrier(0);
  stage_convert(0);
  // the copies landed: only the weight loads issued after them may still be in flight
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * GU_STEPS) : "memory");
#pragma unroll
  for (int mt = 0; mt < 2; mt++)
#pragma unroll
    for (int j = 0; j < NSB; j++) sbv4[mt][j] = *reinterpret_cast<const u32x4*>(&scs[wave][mt][16 * (NSB * n + j)]);

  const int pj = n >> 1, term = n & 1;  // this lane's A row: pair pj of the tile, its term
  for (int m0 = 0; m0 < M; m0 += TILE) {
    const int tn = min(TILE, M - m0);
    if (m0 > 0) {
      __syncthreads();  // the previous tile has read the staging and the partials
      stage_load(m0);
      stage_convert(m0);
    }
    __syncthreads();
    if constexpr (!NV) {
      f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int i = 0; i < GU_STEPS; i++) {
        if (i < my) {
          const int s = s0 + i;
          u32x4 a0 = u32x4{0u, 0u, 0u, 0u}, a1 = a0;
          int sa = 0;
          if (pj < tn) {
            const int off = pj * K + 128 * s + 16 * g;
            a0 = *reinterpret_cast<const u32x4*>(&st.code[term][off]);
            a1 = *reinterpret_cast<const u32x4*>(&st.code[term][off + 64]);
            sa = st.sc[term][(pj * K) / 32 + 4 * s + g];
          }
          const i32x8_t av = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int mt = 0; mt < 2; mt++) {
            const i32x8_t bv =
                __builtin_bit_cast(i32x8_t, __builtin_shufflevector(q[mt][i], q[mt][i], 0, 1, 2, 3, -1, -1, -1, -1));
            const int sbv = (int)(sbv4[mt][i >> 2][i & 3] >> (8 * g));
            acc[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[mt], 0, 4, 0, sa, 0, sbv);
          }
        }
      }
      // lane (column n, g): registers 0, 1 = pair 2g (its terms), 2, 3 = pair 2g + 1
#pragma unroll
      for (int mt = 0; mt < 2; mt++) {
        red[wave][mt][2 * g][n] = acc[mt][0] + acc[mt][1];
        red[wave][mt][2 * g + 1][n] = acc[mt][2] + acc[mt][3];
      }
    } else {
      // A row n = 8 t + d: term t of the pair on block d, whose 16 bytes are lane group
      // d & 3's low (d < 4) or high half; the scale is term t's e8m0 of the lane
      // group's own K-block (it multiplies zeros elsewhere).
      const int t = n >> 3, d = n & 7;
      // Pair by pair (one instruction per pair and step), so that only one pair's
      // sums are live; the scale words are converted again for each pair.
#pragma unroll 1
      for (int j = 0; j < tn; j++) {
        float accn[2] = {0.f, 0.f};
#pragma unroll
        for (int i = 0; i < GU_STEPS; i++) {
          if (i < my) {
            const int s = s0 + i;
            u32x4 a0 = u32x4{0u, 0u, 0u, 0u}, a1 = a0;
            const int sa = st.sc[t][(j * K) / 32 + 4 * s + g];
            if ((d & 3) == g) {
              const u32x4 v = *reinterpret_cast<const u32x4*>(&st.code[t][j * K + 128 * s + 16 * d]);
              if (d < 4) a0 = v;
              else a1 = v;
            }
            const i32x8_t av = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
            for (int mt = 0; mt < 2; mt++) {
              const i32x8_t bv =
                  __builtin_bit_cast(i32x8_t, __builtin_shufflevector(q[mt][i], q[mt][i], 0, 1, 2, 3, -1, -1, -1, -1));
              const f32x4_t c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  av, bv, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 4, 0, sa, 0, 127);
              // E4M3 scales of blocks 4 (g & 1) + r of step s for row n: one word
              uint32_t sw = sbv4[mt][i >> 1][2 * (i & 1) + (g & 1)];
              // converted again for each pair: hoisted out of the pair loop, the 64
              // converted scales took 48 registers (223 against 175 VGPRs)
              asm volatile("" : "+v"(sw));
              const f32x2_t s01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sw, 1.0f, false);
              const f32x2_t s23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sw, 1.0f, true);
              float a = accn[mt];
              a = __builtin_fmaf(s01[0], c[0], a);
              a = __builtin_fmaf(s01[1], c[1], a);
              a = __builtin_fmaf(s23[0], c[2], a);
              accn[mt] = __builtin_fmaf(s23[1], c[3], a);
            }
          }
          // one step at a time: unbounded overlap of the steps' results would take
          // the registers of a second wave per SIMD
          __builtin_amdgcn_sched_barrier(0);
        }
        // the four lane groups of column n: both terms, both halves of each step
#pragma unroll
        for (int mt = 0; mt < 2; mt++) {
          float a = accn[mt];
          a += __shfl_xor(a, 16, 64);
          a += __shfl_xor(a, 32, 64);
          if (lane < 16) red[wave][mt][j][n] = a;
        }
      }
    }
    __syncthreads();
    if (threadIdx.x < 16 * TILE) {
      const int j = threadIdx.x >> 4, col = threadIdx.x & 15;
      const int r = n0 + col;
      if (j < tn && r < P.rows) {
        float gs = 0.f, us = 0.f;
#pragma unroll
        for (int w = 0; w < GU_WAVES; w++) {
          gs += red[w][0][j][col];
          us += red[w][1][j][col];
        }
        P.out[(size_t)P.route.perm()[pstart + m0 + j] * P.rows + r] = silu_mul(gs * s2g, us * s2u);
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // unused weight re-reads land before the end
}

struct DnStage {
  uint8_t code[3][DN_TILE * DN_KMAX];
  uint8_t sc[3][DN_TILE * DN_KMAX / 32];
};

__global__ __launch_bounds__(GB_NT) void k_dn_mx4_g(GemvParams P) {
  __shared__ DnStage st;
  __shared__ float red[GB_WAVES][16][16];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot = blockIdx.y;
  if (slot >= P.route.n_slots()[0]) return;
  const int e = P.route.slots()[slot];
  const int pstart = P.route.offsets()[e];
  const int M = P.route.offsets()[e + 1] - pstart;
  const int n0 = blockIdx.x * DN_ROWS;
  if (e >= P.n_experts) {  // out-of-range ids contribute nothing
    for (int i = threadIdx.x; i < M * DN_ROWS; i += GB_NT) {
      const int r = n0 + (i % DN_ROWS);
      if (r < P.rows) P.out[(size_t)P.route.perm()[pstart + i / DN_ROWS] * P.rows + r] = 0.f;
    }
    return;
  }
  const int K = P.cols;
  const int nsteps = K / 128;
  const int cpt = K / 16;
  constexpr int DSTEPS = DN_ROWSPLIT ? DN_KMAX / 128 : GB_STEPS;  // K steps per wave, at most
  const int spw = DN_ROWSPLIT ? nsteps : steps_per_wave(nsteps, GB_WAVES);
  const int s0 = DN_ROWSPLIT ? 0 : wave * spw;
  const int my = max(0, min(spw, nsteps - s0));
  const int n = lane & 15, g = lane >> 4;
  const int rn = min(n0 + (DN_ROWSPLIT ? 16 * wave : 0) + n, P.rows - 1);
  constexpr int XC = (DN_TILE * DN_KMAX / 16 + GB_NT - 1) / GB_NT;

  u32x4 hv[XC][4];
  auto stage_load = [&](int m0) {
    const int tn = min(DN_TILE, M - m0);
    const int nc = (tn * cpt + GB_NT - 1) / GB_NT;  // uniform
#pragma unroll
    for (int j = 0; j < XC; j++) {
#pragma unroll
      for (int i = 0; i < 4; i++) hv[j][i] = u32x4{0u, 0u, 0u, 0u};
      const int c = j * GB_NT + (int)threadIdx.x;
      if (j < nc && c < tn * cpt) {
        const int pair = P.route.perm()[pstart + m0 + c / cpt];
        const float* hr = reinterpret_cast<const float*>(P.act) + (size_t)pair * K + (c % cpt) * 16;
#pragma unroll
        for (int i = 0; i < 4; i++) hv[j][i] = ld16(hr + 4 * i);
      }
    }
  };
  auto stage_convert = [&](int m0) {
    const int tn = min(DN_TILE, M - m0);
    const int nc = (tn * cpt + GB_NT - 1) / GB_NT;  // uniform
#pragma unroll
    for (int j = 0; j < XC; j++) {
      if (j < nc) {
        const int c = j * GB_NT + (int)threadIdx.x;
        uint32_t w[3][4], E[3];
        f32_terms3(hv[j], w, E);
        if (c < tn * cpt) {
          const int off = (c / cpt) * K + (c % cpt) * 16;
#pragma unroll
          for (int tm = 0; tm < 3; tm++) {
            *reinterpret_cast<u32x4*>(&st.code[tm][off]) = u32x4{w[tm][0], w[tm][1], w[tm][2], w[tm][3]};
            if ((c & 1) == 0) st.sc[tm][off / 32] = (uint8_t)E[tm];
          }
        }
      }
    }
  };

  stage_load(0);
  __builtin_amdgcn_sched_barrier(0);
  u32x4 q[DSTEPS];
  u32x4 sbv4[DSTEPS / 4];
  {
    const uint8_t* wd = P.w[0].data + (size_t)e * P.w[0].estride + (size_t)rn * (K / 2);
    const uint8_t* ws = P.w[0].scales + (size_t)e * P.w[0].sestride + (size_t)rn * (K / 32);
#pragma unroll
    for (int j = 0; j < DSTEPS / 4; j++) sbv4[j] = ld16(ws + (size_t)min(4 * (s0 + 4 * j), 4 * (nsteps - 4)));
#pragma unroll
    for (int i = 0; i < DSTEPS; i++) q[i] = ld16(wd + (size_t)min(s0 + min(i, max(my - 1, 0)), nsteps - 1) * 64 + 16 * g);
  }
  __builtin_amdgcn_sched_barrier(0);
  stage_convert(0);

  const int pj = n / 3, term = n % 3;  // this lane's A row (row 15 unused)
  for (int m0 = 0; m0 < M; m0 += DN_TILE) {
    const int tn = min(DN_TILE, M - m0);
    if (m0 > 0) {
      __syncthreads();
      stage_load(m0);
      stage_convert(m0);
    }
    __syncthreads();
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < DSTEPS; i++) {
      if (i < my) {
        const int s = s0 + i;
        u32x4 a0 = u32x4{0u, 0u, 0u, 0u}, a1 = a0;
        int sa = 0;
        if (pj < tn) {
          const int off = pj * K + 128 * s + 16 * g;
          a0 = *reinterpret_cast<const u32x4*>(&st.code[term][off]);
          a1 = *reinterpret_cast<const u32x4*>(&st.code[term][off + 64]);
          sa = st.sc[term][(pj * K) / 32 + 4 * s + g];
        }
        const i32x8_t av = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
        const i32x8_t bv = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(q[i], q[i], 0, 1, 2, 3, -1, -1, -1, -1));
        const int sbv = (int)(sbv4[i >> 2][i & 3] >> (8 * g));
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0, 4, 0, sa, 0, sbv);
      }
    }
    // lane (column n, g) register r = A row 4g + r
#pragma unroll
    for (int r = 0; r < 4; r++) red[wave][4 * g + r][n] = acc[r];
    __syncthreads();
    // rows split: wave w's own 16 rows; K split: the waves' quarters of K in order
    if (threadIdx.x < (DN_ROWSPLIT ? GB_WAVES : 1) * 16 * DN_TILE) {
      const int wr = DN_ROWSPLIT ? (int)threadIdx.x / (16 * DN_TILE) : 0;
      const int j = ((int)threadIdx.x % (16 * DN_TILE)) >> 4, col = threadIdx.x & 15;
      const int r = n0 + 16 * wr + col;
      if (j < tn && r < P.rows) {
        float v = 0.f;
        if constexpr (DN_ROWSPLIT) {
          v = (red[wr][3 * j][col] + red[wr][3 * j + 1][col]) + red[wr][3 * j + 2][col];
        } else {
#pragma unroll
          for (int w = 0; w < GB_WAVES; w++) v += (red[w][3 * j][col] + red[w][3 * j + 1][col]) + red[w][3 * j + 2][col];
        }
        const int pair = P.route.perm()[pstart + m0 + j];
        P.out[(size_t)pair * P.rows + r] = v * P.rw[pair];
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

}  // namespace

// K a multiple of 512 (16-byte scale runs), at most 4096 (gate/up) or 2048 (down).
bool gu_mx4_g_fits(int rows, int cols) { return rows > 0 && cols > 0 && cols % 512 == 0 && cols <= GU_KMAX; }
bool dn_mx4_g_fits(int rows, int cols) { return rows > 0 && cols > 0 && cols % 512 == 0 && cols <= DN_KMAX; }

hipError_t launch_gu_fp4_g(int fmt, const GemvParams& p, int n_slots, hipStream_t s) {
  if (!gu_mx4_g_fits(p.rows, p.cols) || (fmt != FMT_MXFP4 && fmt != FMT_NVFP4)) return hipErrorInvalidValue;
  const dim3 g((unsigned)((p.rows + 15) / 16), (unsigned)n_slots);
  if (fmt == FMT_NVFP4)
    hipLaunchKernelGGL(k_gu_fp4_g<FMT_NVFP4>, g, dim3(GU_NT), 0, s, p);
  else
    hipLaunchKernelGGL(k_gu_fp4_g<FMT_MXFP4>, g, dim3(GU_NT), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_dn_mx4_g(const GemvParams& p, int n_slots, hipStream_t s) {
  if (!dn_mx4_g_fits(p.rows, p.cols)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_dn_mx4_g, dim3((unsigned)((p.rows + DN_ROWS - 1) / DN_ROWS), (unsigned)n_slots), dim3(GB_NT), 0, s,
                     p);
  return hipGetLastError();
}

}  // namespace moeq
