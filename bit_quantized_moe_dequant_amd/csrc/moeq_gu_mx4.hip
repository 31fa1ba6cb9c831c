// Single-token gate/up + SwiGLU for MXFP4 (and NVFP4, see k_gu1_fp4) experts on the
// block-scaled matrix instruction v_mfma_scale_f32_16x16x128_f8f6f4, with no weight
// decode on the VALU, and the single-token MXFP4 down projection.
//
// The MXFP4 weights (e2m1 codes, one e8m0 scale per 32 along K: DeepSeek V4 Flash -
// REAP K180 Mixed NVFP4 card, section "NVFP4: lossless MXFP4->NVFP4 conversion";
// DeepSeekv4 Flash for 1x Spark forum thread, first post) are the instruction's FP4
// operand B as they sit in memory: lane (row n, group g) passes the 16-byte chunk
// of its row at K = 32g + [0, 32) and that chunk's e8m0 as its B scale. The bf16
// token is operand A, split into two E4M3 terms, x = hi + lo, each with an e8m0
// scale per 32: hi holds the top four significant bits of every value and lo the
// rest (a bf16 value has eight), so the split is exact except for values more than
// 2^12 below their block's maximum, which lose low bits below 2^-16 of that
// maximum. The products run at the FP8 rate in the matrix unit and accumulate in
// fp32; the VALU only converts x, once per work-group. (Decoding FP4 on the VALU,
// where v_cvt_scalef32_pk_bf16_fp4 issues at half rate, cost about as many cycles
// per weight as the weight stream itself.)
//
// Instruction layout (pinned on the device): B lane L = column L % 16 (a weight
// row) with K = 32(L/16) + [0, 32), low nibble first; A lane L = row L % 16 with
// bytes 0-15 at K = 16(L/16) + [0, 16) and bytes 16-31 at K = 64 + 16(L/16) +
// [0, 16); the scale of lane (., g) on either side covers K-block g; output lane L
// register r = row 4(L/16) + r, column L % 16. With one token, the rows of A carry
// the terms of its split instead of tokens: row t holds term t with that term's
// scales, the rows past the last term are zero (scale code 0), and the token's
// result is the sum of output rows 0 .. terms-1 (lanes 0-15, registers 0 .. terms-1).
// One instruction thus multiplies every term by the weights; with a term per
// instruction the matrix unit's work (about 44 clocks per 16 x 128 weights on a
// SIMD) was a large share of the weight stream's time and did not all hide under it.
//
// Work: a work-group is (slot, 16 rows of the gate and of the up matrix). Its four
// waves take contiguous quarters of K (in 128-wide steps) and issue all their
// weight loads before anything else; their partial sums meet in LDS and are added
// in wave order.
#include <hip/hip_ext.h>

#include "moeq_device.h"
#include "moeq_kernels.h"

namespace moeq {

namespace {

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x2_t __attribute__((ext_vector_type(2)));

constexpr int MX_WAVES = 4;
constexpr int MX_STEPS = 8;                           // K steps of 128 per wave
constexpr int MX_KMAX = 128 * MX_WAVES * MX_STEPS;    // 4096
#ifndef MOEQ_MX_DEPTH
#define MOEQ_MX_DEPTH 8
#endif
// NVFP4 gate/up K steps in flight per wave for a single token (its six slots'
// work-groups fit the chip in one round): its steps carry the block-scale
// arithmetic, and loads interleaved with them measured faster (bs=1 NVFP4 + Q2_K
// layer: 22.41 us at 2, 22.51 at 3, 22.93 at 8, 23.3 at 1). Over several tokens
// (more work-groups than fit at once) all steps' loads first is faster (T = 16:
// 252 - 255 against 260 - 262 us at 2), as it is for MXFP4 at any T (bs=1: 19.5 us
// at 8, 20.05 - 20.27 at 2 - 6).
#ifndef MOEQ_NV_DEPTH
#define MOEQ_NV_DEPTH 2
#endif
#ifndef MOEQ_DM_DEPTH
#define MOEQ_DM_DEPTH 8
#endif
constexpr int MX_DEPTH = MOEQ_MX_DEPTH;  // gate/up K steps in flight per wave (MXFP4)
constexpr int DM_DEPTH = MOEQ_DM_DEPTH;  // down K steps in flight per wave

// e8m0 exponent of a 32-block with maximum a: the smallest 2^e with a / 2^e <= 448
// (e = p - 9 if the frexp mantissa of a is <= 0.875, else p - 8), clamped to the
// code range; zero or subnormal maxima give 0.
__device__ __forceinline__ uint32_t gu_mx_exponent(float amax) {
  const uint32_t ab = f2u(amax);
  if (ab < 0x00800000u) return 0u;
  const int p = (int)(ab >> 23) - 126;
  const uint32_t frac = ab & 0x007FFFFFu;
  const int e = (frac <= 0x00600000u) ? p - 9 : p - 8;
  const int E = e + 127;
  return (uint32_t)(E < 0 ? 0 : (E > 254 ? 254 : E));
}

struct MxStage {
  uint8_t code[2][MX_KMAX];  // E4M3 codes of hi and lo
  uint8_t sc[2][MX_KMAX / 32];
};

// NVFP4 (e2m1 codes, an E4M3 scale per 16 along K and an fp32 scale_2 per expert
// tensor: DeepSeek V4 Flash - REAP K180 Mixed NVFP4 card, section "NVFP4: lossless
// MXFP4->NVFP4 conversion") in the same
// instruction. Its block scale is not a power of two and its blocks are 16 wide,
// so it cannot be the instruction's B scale (B scale code 127, i.e. 1). Instead
// each row of A holds one term of x on one 16-block of the 128-wide step and zeros
// elsewhere: row m = 8 t + d is term t on block d (K = 32 (d & 3) + 16 (d >> 2) ...
// in the instruction's K order; see nv_row_piece). Output row m is then the
// unscaled dot of that 16-block alone, and the lane holding it multiplies it by the
// block's E4M3 scale before adding it up. Lane (column n, q) holds output rows
// 4q .. 4q + 3, i.e. blocks d = 4 (q & 1) + r of term q >> 1, whose four E4M3
// bytes are one 32-bit word of row n's scale plane. scale_2 multiplies the sum.
//
// A lane (row m, group g) holds step bytes 16g + [0, 16) (registers 0-3) and
// 64 + 16g + [0, 16) (registers 4-7); block d of the step is bytes 16d + [0, 16) of
// x's 128 values in the order the B operand uses (32g + [0, 32) per lane group,
// low nibble first), so row m's 16 bytes sit in lane group d & 3, low half if
// d < 4. (For MXFP4 the K-block of the scale is what matters and the rows are just
// the terms.)

template <int FMT, int DEPTH>  // DEPTH: K steps in flight per wave
__global__ __launch_bounds__(64 * MX_WAVES) void k_gu1_fp4(GemvParams P) {
  constexpr bool NV = FMT == FMT_NVFP4;
  __shared__ MxStage st;
  __shared__ float red[MX_WAVES][2][16];
  // NVFP4: the wave's scale runs, copied in once (see below)
  __shared__ __attribute__((aligned(16))) uint8_t scs[NV ? MX_WAVES : 1][2][NV ? 1024 : 16];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot = blockIdx.y;
  const int n0 = blockIdx.x * 16;
  const int K = P.cols;
  const int nsteps = K / 128;
  const int e = P.ids[slot];
  const bool ok = e >= 0 && e < P.n_experts;

  // The token's values first (the conversion below waits only for them), then every
  // weight load of the wave; steps past the wave's last re-read it and are not used.
  // Thread t converts values 16t .. 16t + 15 (two threads per 32-block; K <= 4096 =
  // 16 x 256); threads past K re-read the last 16.
  const int k0 = min(16 * (int)threadIdx.x, K - 16);
  // slot = pair t * top_k + k: token t's row of x
  const uint16_t* xr = reinterpret_cast<const uint16_t*>(P.act) + (size_t)(slot / P.top_k) * K + k0;
  const u32x4 v0 = ld16(xr), v1 = ld16(xr + 8);
  __builtin_amdgcn_sched_barrier(0);
  const int n = lane & 15, g = lane >> 4;
  const int rn = min(n0 + n, P.rows - 1);
  const int ec = ok ? e : 0;
  // NVFP4 scale_2 of both tensors now (uniform loads), not after the last barrier.
  const float s2g = NV ? P.w[0].scale2[ec] : 1.f, s2u = NV ? P.w[1].scale2[ec] : 1.f;
  const uint8_t* wd[2];
  const uint8_t* ws[2];
  constexpr int SPB = NV ? 8 : 4;  // scale bytes per 128-wide step
#pragma unroll
  for (int mt = 0; mt < 2; mt++) {
    wd[mt] = P.w[mt].data + (size_t)ec * P.w[mt].estride + (size_t)rn * (K / 2);
    ws[mt] = P.w[mt].scales + (size_t)ec * P.w[mt].sestride + (size_t)rn * (K / 128 * SPB);
  }
  // Wave w takes the contiguous K steps [w spw, (w + 1) spw): consecutive steps of
  // one wave complete each other's 128-byte lines.
  const int spw = 4 * ((nsteps + 4 * MX_WAVES - 1) / (4 * MX_WAVES));  // a multiple of 4 (aligned scale runs)
  const int s0 = wave * spw;
  const int my_steps = max(0, min(spw, nsteps - s0));  // uniform per wave
  u32x4 q[2][MX_STEPS];
  // Scale runs of row rn for the wave's steps, 16 bytes at a time: MXFP4 dword i =
  // step s0 + i (four e8m0 bytes); NVFP4 dwords 2i, 2i + 1 = step s0 + i (eight E4M3
  // bytes). Every valid run lies inside the row (my_steps is a multiple of 4).
  constexpr int NSB = MX_STEPS * SPB / 16;
  u32x4 sbv4[2][NSB];
  if constexpr (NV) {
    // NVFP4 (twice the scale bytes): the wave's 16 rows' runs are copied into LDS
    // once, lane l taking run l % NSB of row l / NSB (row r at bytes 16 NSB r), and
    // read back after the conversion of x. Loaded by each lane, every run came from
    // 16 rows' lines per instruction, four lanes per row asking for the same bytes
    // (bs=1 NVFP4 + Q2_K layer 22.41 against 21.82 us). For MXFP4 the copy and its
    // wait cost more than they save (19.53 against 20.00 us per layer).
    static_assert(16 * NSB <= 64, "a wave's scale runs fit one copy instruction per matrix");
    const int pr = min(lane / NSB, 15), pc = lane % NSB;
    const int r = min(n0 + pr, P.rows - 1);
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
      const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(P.w[mt].scales + (size_t)ec * P.w[mt].sestride), (short)0, 0x7FFFFFFF, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          sr, (__attribute__((address_space(3))) void*)&scs[wave][mt][0], 16,
          r * (K / 128 * SPB) + min(SPB * s0 + 16 * pc, SPB * nsteps - 16), 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);  // the copies before every weight load
  } else {
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
#pragma unroll
      for (int j = 0; j < NSB; j++)
        sbv4[mt][j] = ld16(ws[mt] + (size_t)min(SPB * s0 + 16 * j, SPB * nsteps - 16));
    }
  }
  // Step i's chunk of row rn (steps past the wave's last re-read that one).
  auto load_step = [&](int i) {
    const int s = min(s0 + min(i, max(my_steps - 1, 0)), nsteps - 1);
#pragma unroll
    for (int mt = 0; mt < 2; mt++) q[mt][i] = ld16(wd[mt] + (size_t)s * 64 + 16 * g);
  };
#pragma unroll
  for (int i = 0; i < DEPTH; i++) load_step(i);
  __builtin_amdgcn_sched_barrier(0);

  // x -> hi/lo E4M3 codes and per-32 scales in LDS.
  if (16 * (int)threadIdx.x < K) {
    float x[16];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      x[2 * j] = u2f(v0[j] << 16);
      x[2 * j + 1] = u2f(v0[j] & 0xFFFF0000u);
      x[8 + 2 * j] = u2f(v1[j] << 16);
      x[8 + 2 * j + 1] = u2f(v1[j] & 0xFFFF0000u);
    }
#pragma unroll
    for (int term = 0; term < 2; term++) {
      float amax = 0.f;
#pragma unroll
      for (int j = 0; j < 16; j++) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[j]));
      amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1, 64));  // the block's other half
      const uint32_t E = gu_mx_exponent(amax);
      // The conversions take the block scale 2^(E - 127) as their scale operand
      // (only its exponent field is read, as an e8m0 code): encoding divides by
      // it, decoding multiplies by it, bit for bit as scaling by ldexp around
      // unscaled conversions. x / 2^(E - 127) is at most 448: no clipping.
      const float scale = u2f(E << 23);
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const i16x2_t lo =
            __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(i16x2_t{0, 0}, x[4 * j], x[4 * j + 1], scale, false);
        const i16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, x[4 * j + 2], x[4 * j + 3], scale, true);
        w[j] = (amax == 0.f) ? 0u : __builtin_bit_cast(uint32_t, hi);
      }
      *reinterpret_cast<u32x4*>(&st.code[term][k0]) = u32x4{w[0], w[1], w[2], w[3]};
      if ((threadIdx.x & 1) == 0) st.sc[term][k0 / 32] = (uint8_t)E;
      if (term == 0) {
        // residual x - hi, exact in fp32
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[j], scale, false);
          const f32x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[j], scale, true);
          x[4 * j] -= a[0];
          x[4 * j + 1] -= a[1];
          x[4 * j + 2] -= b[0];
          x[4 * j + 3] -= b[1];
        }
      }
    }
  }
  __syncthreads();
  if constexpr (NV) {
    // the copies landed: only the DEPTH steps' weight loads issued after them may
    // still be in flight (the compiler does not track the copies' LDS writes)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * DEPTH) : "memory");
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
      for (int j = 0; j < NSB; j++) sbv4[mt][j] = *reinterpret_cast<const u32x4*>(&scs[wave][mt][16 * (NSB * n + j)]);
  }

  f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
  float accn[2] = {0.f, 0.f};  // NVFP4: this lane's scaled block sums
#pragma unroll
  for (int i = 0; i < MX_STEPS; i++) {
    if constexpr (DEPTH < MX_STEPS) {
      if (i + DEPTH < MX_STEPS) load_step(i + DEPTH);  // keep DEPTH steps in flight
      __builtin_amdgcn_sched_barrier(0);
    }
    if (i < my_steps) {
      const int s = s0 + i;
      u32x4 a0 = u32x4{0u, 0u, 0u, 0u}, a1 = a0;
      int sa = 0;
      if constexpr (!NV) {
        // A row n < 2 is term n of x (hi, lo); rows 2-15 are zero with scale code 0.
        if (n < 2) {
          a0 = *reinterpret_cast<const u32x4*>(&st.code[n][128 * s + 16 * g]);
          a1 = *reinterpret_cast<const u32x4*>(&st.code[n][128 * s + 64 + 16 * g]);
          sa = st.sc[n][4 * s + g];
        }
      } else {
        // nv_row_piece: row n = 8t + d carries term t on block d, whose 16 bytes are
        // lane group d & 3's low (d < 4) or high half; the scale is term t's e8m0
        // of the lane group's own K-block (it multiplies zeros elsewhere).
        const int t = n >> 3, d = n & 7;
        sa = st.sc[t][4 * s + g];
        if ((d & 3) == g) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(&st.code[t][128 * s + 16 * d]);
          if (d < 4) a0 = v;
          else a1 = v;
        }
      }
      const i32x8_t av = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int mt = 0; mt < 2; mt++) {
        // only the low four registers of an FP4 operand are read
        const i32x8_t bv =
            __builtin_bit_cast(i32x8_t, __builtin_shufflevector(q[mt][i], q[mt][i], 0, 1, 2, 3, -1, -1, -1, -1));
        if constexpr (!NV) {
          const int sbv = (int)(sbv4[mt][i >> 2][i & 3] >> (8 * g));  // this lane's chunk scale, low byte
          acc[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[mt], 0, 4, 0, sa, 0, sbv);
        } else {
          const f32x4_t c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              av, bv, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 4, 0, sa, 0, 127);
          // E4M3 scales of blocks 4 (q & 1) + r of step s: one word (q = g here)
          const uint32_t sw = sbv4[mt][i >> 1][2 * (i & 1) + (g & 1)];
          const f32x2_t s01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sw, 1.0f, false);
          const f32x2_t s23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sw, 1.0f, true);
          accn[mt] = __builtin_fmaf(s01[0], c[0], accn[mt]);
          accn[mt] = __builtin_fmaf(s01[1], c[1], accn[mt]);
          accn[mt] = __builtin_fmaf(s23[0], c[2], accn[mt]);
          accn[mt] = __builtin_fmaf(s23[1], c[3], accn[mt]);
        }
      }
    }
  }
  // Prefetches past the wave's last step are never used: let them land first.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if constexpr (!NV) {
    if (lane < 16) {  // output rows 0 and 1: the hi and lo products
      red[wave][0][lane] = acc[0][0] + acc[0][1];
      red[wave][1][lane] = acc[1][0] + acc[1][1];
    }
  } else {
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {  // the four lane groups of column n
      accn[mt] += __shfl_xor(accn[mt], 16, 64);
      accn[mt] += __shfl_xor(accn[mt], 32, 64);
    }
    if (lane < 16) {
      red[wave][0][lane] = accn[0];
      red[wave][1][lane] = accn[1];
    }
  }
  __syncthreads();
  if (threadIdx.x < 16) {
    float gs = 0.f, us = 0.f;
#pragma unroll
    for (int w = 0; w < MX_WAVES; w++) {
      gs += red[w][0][threadIdx.x];
      us += red[w][1][threadIdx.x];
    }
    gs *= s2g;  // 1 for MXFP4
    us *= s2u;
    const int r = n0 + (int)threadIdx.x;
    if (r < P.rows) P.out[(size_t)slot * P.rows + r] = ok ? silu_mul(gs, us) : 0.f;
    if (!ok && blockIdx.x == 0 && threadIdx.x == 0) atomicOr(P.err, 1u);
  }
}

// ---------------------------------------------------------------- down, one token
// The same instruction for the down projection of one token: y = sum over the
// routed slots k of w_k D_{e_k} h_k (a route-weighted sum of the routed experts'
// outputs). h is fp32, so it is split into three E4M3 terms (about 12 significant
// bits; each residual is exact in fp32, and the bits dropped lie below 2^-13 of the
// block maximum, well inside the projection tolerance). A work-group takes 16
// output rows for all slots: two waves per slot, each half of K; the partials are
// combined in LDS in slot order with the route weights.
constexpr int DM_TERMS = 3;
constexpr int DM_KPARTS = 2;
constexpr int DM_KMAX = 128 * DM_KPARTS * MX_STEPS;  // 2048
constexpr int DM_SLOTS = 8;

struct DmStage {
  uint8_t code[DM_TERMS][DM_SLOTS * DM_KMAX];
  uint8_t sc[DM_TERMS][DM_SLOTS * DM_KMAX / 32];
};

__global__ __launch_bounds__(64 * DM_KPARTS * DM_SLOTS) void k_down1_mx4(Down1Params P) {
  __shared__ DmStage st;
  __shared__ float red[DM_SLOTS * DM_KPARTS][16];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot = wave / DM_KPARTS, part = wave % DM_KPARTS;
  const int n0 = blockIdx.x * 16;
  const int K = P.cols;
  const int nsteps = K / 128;
  // Token blockIdx.y (one token per grid row: its slots' ids, route weights, h, y).
  const int32_t* ids = P.ids + (size_t)blockIdx.y * P.top_k;
  const float* rwt = P.rw + (size_t)blockIdx.y * P.top_k;
  const float* ht = P.h + (size_t)blockIdx.y * P.top_k * K;
  float* yt = P.y + (size_t)blockIdx.y * P.rows;
  const int e = ids[slot];
  const bool ok = e >= 0 && e < P.n_experts;

  // h first (the conversion waits only for it): thread t converts values 16t ..
  // 16t + 15 of the slots' concatenated h, [top_k][K] (two threads per 32-block;
  // the block size is 64 x 2 x top_k threads = top_k x K / 16 for K = 2048).
  const int total = P.top_k * K;
  const int v0i = min(16 * (int)threadIdx.x, total - 16);
  const float* hp = ht + v0i;
  // Route weights before anything else: lane k holds rw[k] for the combine at the
  // end, which would otherwise wait a memory round trip after the last barrier.
  const float rwv = rwt[min(lane, P.top_k - 1)];
  const u32x4 hv0 = ld16(hp), hv1 = ld16(hp + 4), hv2 = ld16(hp + 8), hv3 = ld16(hp + 12);
  __builtin_amdgcn_sched_barrier(0);

  // Weights: K steps [part spw, (part + 1) spw) of row n0 + n of expert e.
  const int n = lane & 15, g = lane >> 4;
  const int rn = min(n0 + n, P.rows - 1);
  const int ec = ok ? e : 0;
  const uint8_t* wd = P.w.data + (size_t)ec * P.w.estride + (size_t)rn * (K / 2);
  const uint8_t* ws = P.w.scales + (size_t)ec * P.w.sestride + (size_t)rn * (K / 32);
  const int spw = 4 * ((nsteps + 4 * DM_KPARTS - 1) / (4 * DM_KPARTS));  // a multiple of 4 (aligned scale runs)
  const int s0 = part * spw;
  const int my_steps = max(0, min(spw, nsteps - s0));
  u32x4 sbv4[MX_STEPS / 4];
#pragma unroll
  for (int j = 0; j < MX_STEPS / 4; j++) sbv4[j] = ld16(ws + (size_t)min(4 * (s0 + 4 * j), 4 * (nsteps - 4)));
  u32x4 q[MX_STEPS];
  auto load_step = [&](int i) { q[i] = ld16(wd + (size_t)min(s0 + min(i, max(my_steps - 1, 0)), nsteps - 1) * 64 + 16 * g); };
#pragma unroll
  for (int i = 0; i < DM_DEPTH; i++) load_step(i);
  __builtin_amdgcn_sched_barrier(0);

  // h -> three E4M3 terms with per-32 scales in LDS (one pass: K <= 2048).
  if (16 * (int)threadIdx.x < total) {
    const int v = v0i;
    float x[16];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      x[j] = u2f(hv0[j]);
      x[4 + j] = u2f(hv1[j]);
      x[8 + j] = u2f(hv2[j]);
      x[12 + j] = u2f(hv3[j]);
    }
#pragma unroll
    for (int term = 0; term < DM_TERMS; term++) {
      float amax = 0.f;
#pragma unroll
      for (int j = 0; j < 16; j++) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[j]));
      amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1, 64));  // the block's other half
      const uint32_t E = gu_mx_exponent(amax);
      const float scale = u2f(E << 23);  // the block scale as the conversions' scale operand
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const i16x2_t lo =
            __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(i16x2_t{0, 0}, x[4 * j], x[4 * j + 1], scale, false);
        const i16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, x[4 * j + 2], x[4 * j + 3], scale, true);
        w[j] = (amax == 0.f) ? 0u : __builtin_bit_cast(uint32_t, hi);
      }
      *reinterpret_cast<u32x4*>(&st.code[term][v]) = u32x4{w[0], w[1], w[2], w[3]};
      if ((threadIdx.x & 1) == 0) st.sc[term][v / 32] = (uint8_t)E;
      if (term + 1 < DM_TERMS) {
#pragma unroll
        for (int j = 0; j < 4; j++) {  // residual, exact in fp32
          const f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[j], scale, false);
          const f32x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[j], scale, true);
          x[4 * j] -= a[0];
          x[4 * j + 1] -= a[1];
          x[4 * j + 2] -= b[0];
          x[4 * j + 3] -= b[1];
        }
      }
    }
  }
  __syncthreads();

  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int hb = slot * K;  // this slot's h among the staged codes
#pragma unroll
  for (int i = 0; i < MX_STEPS; i++) {
    if (i + DM_DEPTH < MX_STEPS) load_step(i + DM_DEPTH);
    __builtin_amdgcn_sched_barrier(0);
    if (i < my_steps) {
      const int s = s0 + i;
      const i32x8_t bv = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(q[i], q[i], 0, 1, 2, 3, -1, -1, -1, -1));
      const int sbv = (int)(sbv4[i >> 2][i & 3] >> (8 * g));
      // A row n < DM_TERMS is term n of h; the other rows are zero with scale code 0.
      u32x4 a0 = u32x4{0u, 0u, 0u, 0u}, a1 = a0;
      int sa = 0;
      if (n < DM_TERMS) {
        a0 = *reinterpret_cast<const u32x4*>(&st.code[n][hb + 128 * s + 16 * g]);
        a1 = *reinterpret_cast<const u32x4*>(&st.code[n][hb + 128 * s + 64 + 16 * g]);
        sa = st.sc[n][(hb + 128 * s) / 32 + g];
      }
      const i32x8_t av = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0, 4, 0, sa, 0, sbv);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // unused prefetches land before the end
  static_assert(DM_TERMS == 3, "output rows 0-2 hold the terms' products");
  if (lane < 16) red[wave][lane] = ok ? acc[0] + acc[1] + acc[2] : 0.f;
  __syncthreads();
  if (threadIdx.x < 16) {
    float y = 0.f;
    for (int k = 0; k < P.top_k; k++) {
      float pk = 0.f;
#pragma unroll
      for (int h = 0; h < DM_KPARTS; h++) pk += red[k * DM_KPARTS + h][threadIdx.x];
      y += pk * u2f(__builtin_amdgcn_readlane(f2u(rwv), k));
    }
    const int r = n0 + (int)threadIdx.x;
    if (r < P.rows) yt[r] = y;
  }
  if (!ok && blockIdx.x == 0 && lane == 0 && part == 0) atomicOr(P.err, 1u);
}

}  // namespace

// K a multiple of 512: every wave's 16-byte runs of chunk scales stay inside the row.
bool gu1_mx4_fits(int rows, int cols) { return rows > 0 && cols > 0 && cols % 512 == 0 && cols <= MX_KMAX; }

// K a multiple of 512 up to 2048, at most 8 slots.
bool down1_mx4_fits(int rows, int cols, int top_k) {
  return rows > 0 && cols > 0 && cols % 512 == 0 && cols <= DM_KMAX && top_k >= 1 && top_k <= DM_SLOTS;
}

hipError_t launch_down1_mx4(const Down1Params& p, hipStream_t s) {
  if (!down1_mx4_fits(p.rows, p.cols, p.top_k)) return hipErrorInvalidValue;
  dim3 g((unsigned)((p.rows + 15) / 16), (unsigned)(p.T > 1 ? p.T : 1)), b((unsigned)(64 * DM_KPARTS * p.top_k));
  hipLaunchKernelGGL(k_down1_mx4, g, b, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_gu1_fp4(int fmt, const GemvParams& p, int n_slots, hipStream_t s, const LaunchEvents* ev) {
  if (!gu1_mx4_fits(p.rows, p.cols) || (fmt != FMT_MXFP4 && fmt != FMT_NVFP4)) return hipErrorInvalidValue;
  dim3 g((unsigned)((p.rows + 15) / 16), (unsigned)n_slots), b(64 * MX_WAVES);
  auto k = fmt == FMT_MXFP4 ? k_gu1_fp4<FMT_MXFP4, MX_DEPTH>
           : n_slots <= 8    ? k_gu1_fp4<FMT_NVFP4, MOEQ_NV_DEPTH>
                             : k_gu1_fp4<FMT_NVFP4, MX_DEPTH>;
  if (ev) hipExtLaunchKernelGGL(k, g, b, 0, s, ev->start, ev->stop, 0, p);
  else hipLaunchKernelGGL(k, g, b, 0, s, p);
  return hipGetLastError();
}

}  // namespace moeq
