// Token-grouped gate/up for IQ2_XXS experts on the bf16 matrix instruction
// v_mfma_f32_16x16x32_bf16, for batches (T > 1) routed through the grouping tables.
//
// The GEMV path decodes an expert's weights once per routed token; this kernel
// decodes them once per group of up to 16 tokens and lets the matrix instruction
// do the multiply-adds. IQ2_XXS decodes exactly into bf16: a codebook entry is
// eight small integers (at most 8 significant bits) and a sign per entry (IQ2_XXS
// + Q2_K + FP8 hybrid card, format table; the block layout of IQ2_XXS: sub-blocks
// of 32 weights, four 8-weight groups each, a 4-bit scale per sub-block and an
// fp16 d per 256). The sub-block scale multiplies the instruction's fp32 partial,
// so, as in the GEMV, only the fp32 accumulation rounds.
//
// Instruction operands: the weights are operand B (16 columns = 16 weight rows),
// the tokens operand A (16 rows = up to 16 tokens of the expert). One instruction
// covers one sub-block (K = 32) of 16 weight rows: lane (n = lane % 16, g = lane /
// 16) supplies group g of row n's sub-block (its 8 weights as four bf16 pairs) and,
// for operand A, the 8 activations of token n at the same K. Output lane L
// register r is token 4(L/16) + r, weight row L % 16: the lane that decoded row n
// also holds row n's outputs, so it scales them with the sub-block scale it
// decoded itself.
//
// Work: a work-group is (one routed expert, 64 weight rows); each of its four waves
// takes 16 rows of the gate and of the up matrix (SwiGLU is then lane-local).
// Superblocks (256 K) stream through two buffers (weight bytes in LDS, the rest in
// registers): the next superblock's loads are issued before the current one is
// computed. Each weight byte is loaded by one lane only (see sb_rows_issue); with
// four lanes per row loading the whole row the kernel was bound by those loads.
// Token lanes past the expert's last token read that token again (same
// addresses) and are not stored.
#include <hip/hip_runtime.h>

#include "moeq_device.h"
#include "moeq_kernels.h"

namespace moeq {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int GI_WAVES = 4;
constexpr int GI_ROWS = 16 * GI_WAVES;  // weight rows per work-group

// One superblock (256 K) of one wave: the fp16 d of row n for both matrices and
// the 16-token activation slices (8 bf16 per sub-block per lane) in registers; the
// 64 bytes of sub-block data of each row in LDS (below).
struct GiBuf {
  uint32_t d[2];
  u32x4 x[8];
};

// A superblock's weight bytes of a wave's 16 rows go through LDS. Every lane needs
// all 64 bytes of its row, but the four lanes of a row loading the same bytes made
// the kernel wait on its loads: four times the address work for the same lines
// (762 against 534 us per IQ2_XXS + Q2_K layer at T = 64, uniform routing). So lane
// (n, g) loads only bytes [16g, 16g + 16) of row n, straight into LDS, where the
// load puts lane l's 16 bytes at the wave's base + 16 l; each lane then reads the
// four pieces of its row back.
typedef __attribute__((address_space(3))) void gi_lds_t;
__device__ __forceinline__ void sb_rows_issue(__amdgpu_buffer_rsrc_t w, int piece_off, int sb, uint8_t* wl) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(w, (gi_lds_t*)wl, 16, piece_off, sb * 64, 0, 0);
}
__device__ __forceinline__ void sb_rows_read(const uint8_t* wl, int n, u32x4 (&w)[4]) {
#pragma unroll
  for (int q = 0; q < 4; q++) w[q] = *reinterpret_cast<const u32x4*>(wl + 16 * (n + 16 * q));
}

// Raw buffer loads: a uniform base (the expert's planes, the activations), a
// loop-invariant lane offset and a uniform superblock offset, so the loop needs no
// per-lane address registers (whose reuse made the compiler wait for loads still
// in flight).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gi_buffer(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFFF, 0x00020000);
}

struct GiStreams {
  __amdgpu_buffer_rsrc_t w[2], s[2], x;
  int w_off, s_off, x_off;  // lane byte offsets: row rn's data and d, token row + group g
};

// Loads of superblock sb: the weight pieces of both matrices into the wave's LDS
// buffer wl ([matrix][lane] 16 bytes), d and the token's activations at the same K
// into registers. GI_LOADS vector-memory instructions in all: the compute waits
// for a buffer by that count, since the compiler does not track the LDS writes.
constexpr int GI_LOADS = 12;
__device__ __forceinline__ void gi_issue(const GiStreams& st, int sb, int piece_off, uint8_t* wl, GiBuf& b) {
#pragma unroll
  for (int mt = 0; mt < 2; mt++) sb_rows_issue(st.w[mt], piece_off, sb, wl + 1024 * mt);
#pragma unroll
  for (int mt = 0; mt < 2; mt++) b.d[mt] = __builtin_amdgcn_raw_buffer_load_b16(st.s[mt], st.s_off, sb * 2, 0);
#pragma unroll
  for (int j = 0; j < 8; j++)
    b.x[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(st.x, st.x_off + 64 * j, sb * 512, 0));
}

// One superblock from buffer (b, wl), issued before the other buffer's GI_LOADS.
__device__ __forceinline__ void gi_compute(const GiBuf& b, const uint8_t* wl, int n, int g, const Iq2Lds* t,
                                           f32x4_t (&acc)[2]) {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(GI_LOADS) : "memory");
  u32x4 w[2][4];
#pragma unroll
  for (int mt = 0; mt < 2; mt++) sb_rows_read(wl + 1024 * mt, n, w[mt]);
  // operand B of sub-block j of matrix mt: the codebook entry with the signs applied
  auto operand = [&](int mt, int j) {
    const uint32_t a0 = w[mt][j >> 1][2 * (j & 1)], a1 = w[mt][j >> 1][2 * (j & 1) + 1];
    const uint32_t gi = (a0 >> (8 * g)) & 0xFFu;
    const uint32_t code = (a1 >> (7 * g)) & 0x7Fu;
    const u32x4 gw = *reinterpret_cast<const u32x4*>(&t->grid[gi * 4]);
    const u32x4 m = t->sgn[code];
    // sign bits of the codebook words are clear, so OR applies the signs
    return u32x4{gw[0] | m[0], gw[1] | m[1], gw[2] | m[2], gw[3] | m[3]};
  };
  auto product = [&](int mt, int j) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, b.x[j]),
                                                   __builtin_bit_cast(bf16x8_t, operand(mt, j)),
                                                   f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  };
  float d8[2];
#pragma unroll
  for (int mt = 0; mt < 2; mt++) d8[mt] = half_bits_f32(b.d[mt]) * 0.125f;
  auto scale_add = [&](int mt, int j, const f32x4_t& c) {
    const uint32_t a1 = w[mt][j >> 1][2 * (j & 1) + 1];
    const float db = d8[mt] * (float)(2u * (a1 >> 28) + 1u);  // exact: 11 x 5 bits
#pragma unroll
    for (int r = 0; r < 4; r++) acc[mt][r] = __builtin_fmaf(c[r], db, acc[mt][r]);
  };
  // Two sub-blocks in flight: the products of sub-block j are issued before the
  // scaled sums of sub-block j - 1, so only two sub-blocks' results are live (174
  // -> 152 VGPRs against all eight products of a matrix first; IQ2_XXS + Q2_K at
  // T = 64 491.5-493.5 -> 486-488 us). Each accumulator still adds its sub-blocks
  // in order.
  f32x4_t c[2][2];
#pragma unroll
  for (int j = 0; j <= 8; j++) {
    if (j < 8) {
#pragma unroll
      for (int mt = 0; mt < 2; mt++) c[j & 1][mt] = product(mt, j);
    }
    if (j > 0) {
#pragma unroll
      for (int mt = 0; mt < 2; mt++) scale_add(mt, j - 1, c[(j - 1) & 1][mt]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

__global__ __launch_bounds__(64 * GI_WAVES) __attribute__((amdgpu_waves_per_eu(2))) void k_gu_iq2(GemvParams P) {
  __shared__ Iq2Lds lds_tab[1];
  // the two weight buffers of each wave, as two arrays: the compiler then knows
  // that reading one need not wait for the loads still filling the other
  __shared__ __attribute__((aligned(16))) uint8_t wbuf0[GI_WAVES][2048];
  __shared__ __attribute__((aligned(16))) uint8_t wbuf1[GI_WAVES][2048];
  iq2_fill_lds(&lds_tab[0], P.grid, threadIdx.x, 64 * GI_WAVES);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  uint8_t* const wl0 = &wbuf0[wave][0];
  uint8_t* const wl1 = &wbuf1[wave][0];
  const int slot = blockIdx.y;
  if (slot >= P.route.n_slots()[0]) return;
  const int e = P.route.slots()[slot];
  const int pstart = P.route.offsets()[e];
  const int M = P.route.offsets()[e + 1] - pstart;
  const int n0 = blockIdx.x * GI_ROWS + wave * 16;
  if (n0 >= P.rows || M <= 0) return;

  if (e < 0 || e >= P.n_experts) {
    // Out-of-range expert id (its bucket): its pairs contribute nothing.
    for (int m = 0; m < M; m++) {
      const int pair = P.route.perm()[pstart + m];
      if (lane < 16 && n0 + lane < P.rows) P.out[(size_t)pair * P.rows + n0 + lane] = 0.f;
    }
    return;
  }

  const int nsb = P.cols / 256;
  const int rn = min(n0 + n, P.rows - 1);
  GiStreams st;
#pragma unroll
  for (int mt = 0; mt < 2; mt++) {
    st.w[mt] = gi_buffer(P.w[mt].data + (size_t)e * P.w[mt].estride);
    st.s[mt] = gi_buffer(P.w[mt].scales + (size_t)e * P.w[mt].sestride);
  }
  st.x = gi_buffer(P.act);
  st.w_off = rn * nsb * 64;
  st.s_off = rn * nsb * 2;

  for (int m0 = 0; m0 < M; m0 += 16) {
    // Token of operand-A row n (lanes past the last token repeat it).
    const int pa = P.route.perm()[pstart + min(m0 + n, M - 1)];
    st.x_off = (pa / P.top_k) * P.cols * 2 + 16 * g;
    f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
    const int poff = st.w_off + 16 * g;
    GiBuf A, B;
    gi_issue(st, 0, poff, wl0, A);
    // Two buffers in turn; the prefetch is unconditional (after the last
    // superblock it re-reads it, a cache hit), so no branch separates a prefetch
    // from the arithmetic after it. A buffer's LDS is refilled only after the
    // compute that read it, whose reads have returned (their values were used).
    for (int sb = 0;; sb += 2) {
      __builtin_amdgcn_sched_barrier(0);
      gi_issue(st, min(sb + 1, nsb - 1), poff, wl1, B);
      __builtin_amdgcn_sched_barrier(0);
      gi_compute(A, wl0, n, g, &lds_tab[0], acc);
      if (sb + 1 >= nsb) break;
      __builtin_amdgcn_sched_barrier(0);
      gi_issue(st, min(sb + 2, nsb - 1), poff, wl0, A);
      __builtin_amdgcn_sched_barrier(0);
      gi_compute(B, wl1, n, g, &lds_tab[0], acc);
      if (sb + 2 >= nsb) break;
    }
    // The final prefetch is never used: let it land before the registers are reused.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // Lane: weight row n0 + n, tokens m0 + 4g + r, whose pair lane 4g + r read for
    // operand A (taken while every lane is active; no loads after the arithmetic).
    int pr[4];
#pragma unroll
    for (int r = 0; r < 4; r++) pr[r] = __shfl(pa, 4 * g + r, 64);
    if (n0 + n < P.rows) {
#pragma unroll
      for (int r = 0; r < 4; r++)
        if (m0 + 4 * g + r < M) P.out[(size_t)pr[r] * P.rows + n0 + n] = silu_mul(acc[0][r], acc[1][r]);
    }
  }
}

// ---------------------------------------------------------------- many tokens per expert
// Prefill-sized batches: each sub-block is decoded once and applied to GW_NT
// 16-token tiles per pass, so the decode is shared by up to 16 GW_NT = 64 tokens
// instead of 16 (an expert with up to 64 pairs is decoded once). The pass's activations are staged once per superblock in LDS for
// the work-group's four waves (each wave reading its own copy from L2 had been
// half the kernel's time), in two buffers with one barrier per superblock, and the
// activation and weight loads run two superblocks ahead.
constexpr int GW_NT = 4;
constexpr int GW_RND = GW_NT / 2;  // staging rounds: 256 threads stage 32 tokens x 8 sub-blocks each

struct GwBuf {
  u32x4 w[2][4];
  uint32_t d[2];
};

__device__ __forceinline__ void gw_issue(const GiStreams& st, int sb, GwBuf& b) {
#pragma unroll
  for (int mt = 0; mt < 2; mt++) {
#pragma unroll
    for (int i = 0; i < 4; i++)
      b.w[mt][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(st.w[mt], st.w_off + 16 * i, sb * 64, 0));
    b.d[mt] = __builtin_amdgcn_raw_buffer_load_b16(st.s[mt], st.s_off, sb * 2, 0);
  }
}

// The pass's activations for one superblock, shared by the work-group's waves:
// [((tile * 8 + sub-block) * 16 + token) * 4 + group] = 8 bf16 at K = 32 j + 8 g.
struct GwStage {
  u32x4 x[GW_NT * 8 * 16 * 4];
};

// One superblock: each sub-block is decoded once (both matrices) and applied to
// the pass's tiles, whose activations come from LDS.
__device__ __forceinline__ void gw_compute(int nt, const GwBuf& b, const GwStage& xs, int n, int g, const Iq2Lds* t,
                                           f32x4_t (&acc)[GW_NT][2]) {
  float d8[2];
#pragma unroll
  for (int mt = 0; mt < 2; mt++) d8[mt] = half_bits_f32(b.d[mt]) * 0.125f;
#pragma unroll
  for (int j = 0; j < 8; j++) {
    u32x4 wv[2];
    float db[2];
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
      const uint32_t a0 = b.w[mt][j >> 1][2 * (j & 1)], a1 = b.w[mt][j >> 1][2 * (j & 1) + 1];
      const uint32_t gi = (a0 >> (8 * g)) & 0xFFu;
      const uint32_t code = (a1 >> (7 * g)) & 0x7Fu;
      const u32x4 gw = *reinterpret_cast<const u32x4*>(&t->grid[gi * 4]);
      const u32x4 m = t->sgn[code];
      wv[mt] = u32x4{gw[0] | m[0], gw[1] | m[1], gw[2] | m[2], gw[3] | m[3]};
      db[mt] = d8[mt] * (float)(2u * (a1 >> 28) + 1u);  // exact: 11 x 5 bits
    }
#pragma unroll
    for (int ti = 0; ti < GW_NT; ti++) {
      if (ti < nt) {
        const u32x4 xv = xs.x[((ti * 8 + j) * 16 + n) * 4 + g];
#pragma unroll
        for (int mt = 0; mt < 2; mt++) {
          const f32x4_t c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xv),
                                                                    __builtin_bit_cast(bf16x8_t, wv[mt]),
                                                                    f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; r++) acc[ti][mt][r] = __builtin_fmaf(c[r], db[mt], acc[ti][mt][r]);
        }
      }
    }
  }
}

__global__ __launch_bounds__(64 * GI_WAVES) __attribute__((amdgpu_waves_per_eu(2))) void k_gu_iq2_wide(GemvParams P) {
  __shared__ Iq2Lds lds_tab[1];
  __shared__ GwStage stg[2];
  __shared__ int s_pair[16 * GW_NT];
  iq2_fill_lds(&lds_tab[0], P.grid, threadIdx.x, 64 * GI_WAVES);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int slot = blockIdx.y;
  if (slot >= P.route.n_slots()[0]) return;
  const int e = P.route.slots()[slot];
  const int pstart = P.route.offsets()[e];
  const int M = P.route.offsets()[e + 1] - pstart;
  const int r0 = blockIdx.x * GI_ROWS;
  if (r0 >= P.rows || M <= 0) return;  // uniform per work-group: the barriers below are reached by all
  if (e < 0 || e >= P.n_experts) {
    for (int m = 0; m < M; m++) {
      const int pair = P.route.perm()[pstart + m];
      for (int i = threadIdx.x; i < GI_ROWS; i += 64 * GI_WAVES)
        if (r0 + i < P.rows) P.out[(size_t)pair * P.rows + r0 + i] = 0.f;
    }
    return;
  }

  const int nsb = P.cols / 256;
  const int n0 = r0 + wave * 16;
  const int rn = min(n0 + n, P.rows - 1);
  GiStreams st;
#pragma unroll
  for (int mt = 0; mt < 2; mt++) {
    st.w[mt] = gi_buffer(P.w[mt].data + (size_t)e * P.w[mt].estride);
    st.s[mt] = gi_buffer(P.w[mt].scales + (size_t)e * P.w[mt].sestride);
  }
  st.x = gi_buffer(P.act);
  st.w_off = rn * nsb * 64;
  st.s_off = rn * nsb * 2;
  // staging: in round u, thread = (pass token tt + 32 u, sub-block q); its 64
  // bytes are the four 8-value groups of that sub-block
  static_assert(64 * GI_WAVES == 256 && GW_NT % 2 == 0, "staging covers 32 tokens per round");
  const int tt = threadIdx.x >> 3, q = threadIdx.x & 7;

  for (int m0 = 0; m0 < M; m0 += 16 * GW_NT) {
    const int nt = min(GW_NT, (M - m0 + 15) / 16);  // uniform
    int x_off[GW_RND], sidx[GW_RND];
#pragma unroll
    for (int u = 0; u < GW_RND; u++) {
      const int tk = tt + 32 * u;
      const int pt = P.route.perm()[pstart + min(m0 + tk, M - 1)];  // tokens past the last repeat it
      if (q == 0) s_pair[tk] = pt;
      x_off[u] = (pt / P.top_k) * P.cols * 2 + 64 * q;
      sidx[u] = (((tk >> 4) * 8 + q) * 16 + (tk & 15)) * 4;
    }
    auto xload = [&](int sb, u32x4(&dst)[GW_RND][4]) {
#pragma unroll
      for (int u = 0; u < GW_RND; u++)
#pragma unroll
        for (int i = 0; i < 4; i++)
          dst[u][i] =
              __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(st.x, x_off[u] + 16 * i, sb * 512, 0));
    };
    // Two superblocks in flight: register set k holds superblocks k, k + 2, ...
    // (loads past the last superblock re-read it and are not used).
    u32x4 v[2][GW_RND][4];
    GwBuf W[2];
    xload(0, v[0]);
    gw_issue(st, 0, W[0]);
    xload(min(1, nsb - 1), v[1]);
    gw_issue(st, min(1, nsb - 1), W[1]);
    f32x4_t acc[GW_NT][2];
#pragma unroll
    for (int ti = 0; ti < GW_NT; ti++) acc[ti][0] = acc[ti][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int sb = 0; sb < nsb; sb += 2) {
#pragma unroll
      for (int k = 0; k < 2; k++) {
        if (sb + k < nsb) {  // uniform
#pragma unroll
          for (int u = 0; u < GW_RND; u++)
#pragma unroll
            for (int i = 0; i < 4; i++) stg[k].x[sidx[u] + i] = v[k][u][i];
          xload(min(sb + k + 2, nsb - 1), v[k]);
          __syncthreads();
          gw_compute(nt, W[k], stg[k], n, g, &lds_tab[0], acc);
          gw_issue(st, min(sb + k + 2, nsb - 1), W[k]);
        }
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (n0 + n < P.rows) {
#pragma unroll
      for (int ti = 0; ti < GW_NT; ti++)
#pragma unroll
        for (int r = 0; r < 4; r++)
          if (ti < nt && m0 + 16 * ti + 4 * g + r < M)
            P.out[(size_t)s_pair[16 * ti + 4 * g + r] * P.rows + n0 + n] = silu_mul(acc[ti][0][r], acc[ti][1][r]);
    }
    __syncthreads();  // the staging buffers and s_pair are rewritten by the next pass
  }
}

// ---------------------------------------------------------------- Q2_K down, token-grouped
// The down projection of Q2_K experts for batches (T > 1), on
// v_mfma_f32_16x16x16_bf16: the weights of a sub-block are decoded once per group
// of up to 16 of the expert's tokens instead of once per (token, expert) pair.
//
// Q2_K (IQ2_XXS + Q2_K + FP8 hybrid card, format table; block layout: 256 weights
// in 16 sub-blocks of 16, a 4-bit scale and a 4-bit min per sub-block, fp16 d and
// dmin per 256): w = d sc q - dmin m with a 2-bit code q. The sub-block is 16 wide,
// so one instruction (K = 16) covers exactly one sub-block and its fp32 partial can
// take the sub-block's scale in the lane that holds it.
//
// Operands, as in k_gu_iq2: the weights are operand B (16 columns = 16 weight rows),
// the tokens operand A (16 rows = up to 16 tokens); output lane L register r is
// token 4(L/16) + r, weight row L % 16. Lane (row n, group g) takes weights
// 4g .. 4g + 3 of every sub-block: in the device layout these are dword g of the
// sub-block's 16-byte chunk, at the sub-block's crumb position p. OR-ed into the
// mantissa of 1.0 a crumb gives the exact bf16 value 1 + q / F (F = 128, 32, 8, 4
// for p = 0 .. 3), two weights per register in the K order (0, 2), (1, 3). With C
// the instruction's result and H the token's sub-block sum of the same bf16 h
// values, C - H = (sum h q) / F, and the token's output gets
//   d sc F (C - H) - dmin m H
// per sub-block: every product is exact and only fp32 sums round.
//
// The work-group's four waves (64 weight rows) share the token tile: per
// superblock its h is staged once in LDS, already split into bf16 hi + lo pairs in
// the instructions' K order, with the sums H (one (token, sub-block) per thread),
// in two buffers with one barrier per superblock; the loads run two superblocks
// ahead. Outputs are route-weighted partials per (pair, row), added by the combine.
struct GqStage {
  u32x4 a[16 * 16 * 4];  // [(sub-block j * 16 + token m) * 4 + group g]: hi (K 0,2), hi (1,3), lo, lo
  float h[16 * 16];      // [sub-block j * 16 + token m]: sum of the 16 bf16 (hi + lo) values
};

struct GqW {
  uint32_t w[4];  // dword g of each 16-byte chunk of the superblock, row n
  u32x4 sc;       // the 16 sub-block scale/min bytes of row n
  uint32_t dd;    // d | dmin << 16
};

typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ s16x4_t gq_pair(uint32_t a, uint32_t b) { return __builtin_bit_cast(s16x4_t, u32x2{a, b}); }

__device__ __forceinline__ void gq_wload(__amdgpu_buffer_rsrc_t wr, __amdgpu_buffer_rsrc_t sr, int w_off, int s_off,
                                         int sb, GqW& b) {
#pragma unroll
  for (int c = 0; c < 4; c++) b.w[c] = __builtin_amdgcn_raw_buffer_load_b32(wr, w_off + 16 * c, sb * 64, 0);
  b.sc = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(sr, s_off, sb * 20, 0));
  b.dd = __builtin_amdgcn_raw_buffer_load_b32(sr, s_off + 16, sb * 20, 0);
}

// This thread's (token, sub-block): 16 fp32 h values -> LDS as bf16 hi/lo pairs and
// their sum.
__device__ __forceinline__ void gq_stage_write(const u32x4 (&v)[4], int tm, int tj, GqStage& s) {
  float hsum = 0.f;
#pragma unroll
  for (int g = 0; g < 4; g++) {
    uint32_t h0, l0, h1, l1;
    split_pair(u2f(v[g][0]), u2f(v[g][2]), h0, l0);
    split_pair(u2f(v[g][1]), u2f(v[g][3]), h1, l1);
    s.a[(tj * 16 + tm) * 4 + g] = u32x4{h0, h1, l0, l1};
    hsum += (u2f(h0 << 16) + u2f(l0 << 16)) + (u2f(h0 & 0xFFFF0000u) + u2f(l0 & 0xFFFF0000u)) +
            (u2f(h1 << 16) + u2f(l1 << 16)) + (u2f(h1 & 0xFFFF0000u) + u2f(l1 & 0xFFFF0000u));
  }
  s.h[tj * 16 + tm] = hsum;
}

__device__ __forceinline__ void gq_compute(const GqW& b, const GqStage& s, int n, int g, f32x4_t& acc) {
  const uint32_t ONE = 0x3F803F80u;
  const float d = half_bits_f32(b.dd), dmin = half_bits_f32(b.dd >> 16);
  // d F for the four crumb positions (F = 128, 32, 8, 4: exact powers of two)
  const float dF[4] = {d * 128.f, d * 32.f, d * 8.f, d * 4.f};
#pragma unroll
  for (int c = 0; c < 4; c++) {
    const uint32_t w = b.w[c], w8 = b.w[c] >> 8;
#pragma unroll
    for (int p = 0; p < 4; p++) {
      const int j = 8 * (c >> 1) + (c & 1) + 2 * p;  // the sub-block at chunk c, crumb p
      // B: 1 + q / F for weights (4g, 4g + 2) and (4g + 1, 4g + 3)
      uint32_t ba, bb;
      if (p < 3) {
        const uint32_t m = 0x00030003u << (2 * p);
        ba = (w & m) | ONE;
        bb = (w8 & m) | ONE;
      } else {
        ba = ((w >> 1) & 0x00600060u) | ONE;
        bb = ((w8 >> 1) & 0x00600060u) | ONE;
      }
      const s16x4_t bv = gq_pair(ba, bb);
      const u32x4 av = s.a[(j * 16 + n) * 4 + g];  // A row n = token n
      f32x4_t cq = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(gq_pair(av[0], av[1]), bv, f32x4_t{0.f, 0.f, 0.f, 0.f},
                                                              0, 0, 0);
      cq = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(gq_pair(av[2], av[3]), bv, cq, 0, 0, 0);
      const f32x4_t hs = *reinterpret_cast<const f32x4_t*>(&s.h[j * 16 + 4 * g]);  // tokens 4g .. 4g + 3
      const uint32_t byte = (b.sc[j >> 2] >> (8 * (j & 3))) & 0xFFu;
      const float cs = dF[p] * (float)(byte & 15u);  // d sc F: exact (11 x 4 bits, power of two)
      const float cm = dmin * (float)(byte >> 4);    // exact
      // cs (cq - hs) - cm hs = cs cq - (cs + cm) hs
      const float csm = cs + cm;
#pragma unroll
      for (int r = 0; r < 4; r++) acc[r] = __builtin_fmaf(-csm, hs[r], __builtin_fmaf(cs, cq[r], acc[r]));
    }
  }
}

__global__ __launch_bounds__(64 * GI_WAVES) void k_dn_q2k(GemvParams P) {
  __shared__ GqStage stg[2];
  __shared__ int s_pair[16];
  __shared__ float s_rw[16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int slot = blockIdx.y;
  if (slot >= P.route.n_slots()[0]) return;
  const int e = P.route.slots()[slot];
  const int pstart = P.route.offsets()[e];
  const int M = P.route.offsets()[e + 1] - pstart;
  const int r0 = blockIdx.x * GI_ROWS;
  if (r0 >= P.rows || M <= 0) return;  // uniform per work-group: the barriers below are reached by all

  if (e < 0 || e >= P.n_experts) {
    // Out-of-range expert id (its bucket): its pairs contribute nothing.
    for (int m = 0; m < M; m++) {
      const int pair = P.route.perm()[pstart + m];
      for (int i = threadIdx.x; i < GI_ROWS; i += 64 * GI_WAVES)
        if (r0 + i < P.rows) P.out[(size_t)pair * P.rows + r0 + i] = 0.f;
    }
    return;
  }

  const int nsb = P.cols / 256;
  const int n0 = r0 + wave * 16;
  const int rn = min(n0 + n, P.rows - 1);
  const __amdgpu_buffer_rsrc_t wr = gi_buffer(P.w[0].data + (size_t)e * P.w[0].estride);
  const __amdgpu_buffer_rsrc_t sr = gi_buffer(P.w[0].scales + (size_t)e * P.w[0].sestride);
  const __amdgpu_buffer_rsrc_t xr = gi_buffer(P.act);
  const int w_off = rn * nsb * 64 + 4 * g, s_off = rn * nsb * 20;
  // staging: thread = (token tm, sub-block tj)
  const int tm = threadIdx.x >> 4, tj = threadIdx.x & 15;

  for (int m0 = 0; m0 < M; m0 += 16) {
    const int pt = P.route.perm()[pstart + min(m0 + tm, M - 1)];  // tokens past the last repeat it
    if (tj == 0) {
      s_pair[tm] = pt;
      s_rw[tm] = P.rw[pt];
    }
    const int x_off = pt * P.cols * 4 + 64 * tj;
    // Two superblocks in flight: register set k holds superblocks k, k + 2, ...
    // (loads past the last superblock re-read it and are not used).
    u32x4 v[2][4];
    GqW W[2];
    auto xload = [&](int sb, u32x4(&dst)[4]) {
#pragma unroll
      for (int i = 0; i < 4; i++)
        dst[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, x_off + 16 * i, sb * 1024, 0));
    };
    xload(0, v[0]);
    gq_wload(wr, sr, w_off, s_off, 0, W[0]);
    xload(min(1, nsb - 1), v[1]);
    gq_wload(wr, sr, w_off, s_off, min(1, nsb - 1), W[1]);
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int sb = 0; sb < nsb; sb += 2) {
#pragma unroll
      for (int k = 0; k < 2; k++) {
        if (sb + k < nsb) {  // uniform
          gq_stage_write(v[k], tm, tj, stg[k]);
          xload(min(sb + k + 2, nsb - 1), v[k]);
          __syncthreads();
          gq_compute(W[k], stg[k], n, g, acc);
          gq_wload(wr, sr, w_off, s_off, min(sb + k + 2, nsb - 1), W[k]);
        }
      }
    }
    // The final prefetches are never used: let them land before the registers are reused.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // Lane: weight row n0 + n, tokens m0 + 4g + r.
    if (n0 + n < P.rows) {
#pragma unroll
      for (int r = 0; r < 4; r++)
        if (m0 + 4 * g + r < M) P.out[(size_t)s_pair[4 * g + r] * P.rows + n0 + n] = acc[r] * s_rw[4 * g + r];
    }
    __syncthreads();  // the staging buffers and s_pair / s_rw are rewritten by the next tile
  }
}

// ---------------------------------------------------------------- IQ2_XXS down, token-grouped
// The down projection of IQ2_XXS experts for batches (T > 1), on
// v_mfma_f32_16x16x32_bf16, for the layers of the mix whose down projection keeps
// the IQ2_XXS floor (DeepSeekv4 Flash for 1x Spark forum thread, first post: an
// IQ2_XXS floor on most experts). As in k_gu_iq2, one instruction covers one
// 32-weight sub-block of 16 weight rows (operand B, decoded exactly into bf16)
// and the sub-block scale multiplies the instruction's fp32 partial in the lane
// that decoded it; the tokens (operand A) are h as bf16 hi + lo pairs (16
// significant bits, the rounding of the split is the only one besides fp32
// sums), two instructions per sub-block. The work-group's four waves (64 weight
// rows) share each 16-token tile's h, staged once per superblock in LDS already in
// the instruction's operand order; two buffers, one barrier per superblock, loads
// two superblocks ahead. Outputs are route-weighted partials per (pair, row).
struct GdStage {
  u32x4 a[8 * 16 * 4 * 2];  // [((sub-block j * 16 + token m) * 4 + group g) * 2 + lo]: 8 bf16 at K = 32 j + 8 g
};

struct GdW {
  u32x4 w[4];  // the superblock's 64 data bytes of row n
  uint32_t d;  // its fp16 d
};

__device__ __forceinline__ void gd_wload(__amdgpu_buffer_rsrc_t wr, __amdgpu_buffer_rsrc_t sr, int w_off, int s_off,
                                         int sb, GdW& b) {
#pragma unroll
  for (int i = 0; i < 4; i++)
    b.w[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, w_off + 16 * i, sb * 64, 0));
  b.d = __builtin_amdgcn_raw_buffer_load_b16(sr, s_off, sb * 2, 0);
}

// This thread's (token tm, half hf of sub-block j): 16 fp32 h values (K = 32 j +
// 16 hf + [0, 16)) -> groups 2 hf and 2 hf + 1 as bf16 hi and lo octets.
__device__ __forceinline__ void gd_stage_write(const u32x4 (&v)[4], int tm, int j, int hf, GdStage& s) {
#pragma unroll
  for (int q = 0; q < 2; q++) {
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const u32x4 u = v[2 * q + i];
      split_pair(u2f(u[0]), u2f(u[1]), hi[2 * i], lo[2 * i]);
      split_pair(u2f(u[2]), u2f(u[3]), hi[2 * i + 1], lo[2 * i + 1]);
    }
    const int base = ((j * 16 + tm) * 4 + 2 * hf + q) * 2;
    s.a[base] = u32x4{hi[0], hi[1], hi[2], hi[3]};
    s.a[base + 1] = u32x4{lo[0], lo[1], lo[2], lo[3]};
  }
}

__device__ __forceinline__ void gd_compute(const GdW& b, const GdStage& s, int n, int g, const Iq2Lds* t,
                                           f32x4_t& acc) {
  const float d8 = half_bits_f32(b.d) * 0.125f;
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const uint32_t a0 = b.w[j >> 1][2 * (j & 1)], a1 = b.w[j >> 1][2 * (j & 1) + 1];
    const uint32_t gi = (a0 >> (8 * g)) & 0xFFu;
    const uint32_t code = (a1 >> (7 * g)) & 0x7Fu;
    const u32x4 gw = *reinterpret_cast<const u32x4*>(&t->grid[gi * 4]);
    // sign words in registers here (mixed-layer prefill at T = 2048: 2360 against
    // 2492 us with the LDS table, which the gate/up kernels keep)
    uint32_t m[4];
    iq2_sign_words(code, m);
    const u32x4 wv = u32x4{gw[0] | m[0], gw[1] | m[1], gw[2] | m[2], gw[3] | m[3]};
    const int base = ((j * 16 + n) * 4 + g) * 2;  // A row n = token n
    f32x4_t c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, s.a[base]),
                                                        __builtin_bit_cast(bf16x8_t, wv), f32x4_t{0.f, 0.f, 0.f, 0.f},
                                                        0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, s.a[base + 1]),
                                                __builtin_bit_cast(bf16x8_t, wv), c, 0, 0, 0);
    const float db = d8 * (float)(2u * (a1 >> 28) + 1u);  // exact: 11 x 5 bits
#pragma unroll
    for (int r = 0; r < 4; r++) acc[r] = __builtin_fmaf(c[r], db, acc[r]);
  }
}

__global__ __launch_bounds__(64 * GI_WAVES) void k_dn_iq2(GemvParams P) {
  __shared__ Iq2Lds lds_tab[1];
  __shared__ GdStage stg[2];
  __shared__ int s_pair[16];
  __shared__ float s_rw[16];
  iq2_fill_lds(&lds_tab[0], P.grid, threadIdx.x, 64 * GI_WAVES);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int slot = blockIdx.y;
  if (slot >= P.route.n_slots()[0]) return;
  const int e = P.route.slots()[slot];
  const int pstart = P.route.offsets()[e];
  const int M = P.route.offsets()[e + 1] - pstart;
  const int r0 = blockIdx.x * GI_ROWS;
  if (r0 >= P.rows || M <= 0) return;  // uniform per work-group: the barriers below are reached by all
  if (e < 0 || e >= P.n_experts) {
    for (int m = 0; m < M; m++) {
      const int pair = P.route.perm()[pstart + m];
      for (int i = threadIdx.x; i < GI_ROWS; i += 64 * GI_WAVES)
        if (r0 + i < P.rows) P.out[(size_t)pair * P.rows + r0 + i] = 0.f;
    }
    return;
  }

  const int nsb = P.cols / 256;
  const int n0 = r0 + wave * 16;
  const int rn = min(n0 + n, P.rows - 1);
  const __amdgpu_buffer_rsrc_t wr = gi_buffer(P.w[0].data + (size_t)e * P.w[0].estride);
  const __amdgpu_buffer_rsrc_t sr = gi_buffer(P.w[0].scales + (size_t)e * P.w[0].sestride);
  const __amdgpu_buffer_rsrc_t xr = gi_buffer(P.act);
  const int w_off = rn * nsb * 64, s_off = rn * nsb * 2;
  // staging: thread = (token tm, sub-block tj / 2, half tj % 2)
  const int tm = threadIdx.x >> 4, tj = threadIdx.x & 15;

  for (int m0 = 0; m0 < M; m0 += 16) {
    const int pt = P.route.perm()[pstart + min(m0 + tm, M - 1)];  // tokens past the last repeat it
    if (tj == 0) {
      s_pair[tm] = pt;
      s_rw[tm] = P.rw[pt];
    }
    const int x_off = pt * P.cols * 4 + 64 * tj;
    u32x4 v[2][4];
    GdW W[2];
    auto xload = [&](int sb, u32x4(&dst)[4]) {
#pragma unroll
      for (int i = 0; i < 4; i++)
        dst[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, x_off + 16 * i, sb * 1024, 0));
    };
    xload(0, v[0]);
    gd_wload(wr, sr, w_off, s_off, 0, W[0]);
    xload(min(1, nsb - 1), v[1]);
    gd_wload(wr, sr, w_off, s_off, min(1, nsb - 1), W[1]);
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int sb = 0; sb < nsb; sb += 2) {
#pragma unroll
      for (int k = 0; k < 2; k++) {
        if (sb + k < nsb) {  // uniform
          gd_stage_write(v[k], tm, tj >> 1, tj & 1, stg[k]);
          xload(min(sb + k + 2, nsb - 1), v[k]);
          __syncthreads();
          gd_compute(W[k], stg[k], n, g, &lds_tab[0], acc);
          gd_wload(wr, sr, w_off, s_off, min(sb + k + 2, nsb - 1), W[k]);
        }
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the final prefetches are never used
    if (n0 + n < P.rows) {
#pragma unroll
      for (int r = 0; r < 4; r++)
        if (m0 + 4 * g + r < M) P.out[(size_t)s_pair[4 * g + r] * P.rows + n0 + n] = acc[r] * s_rw[4 * g + r];
    }
    __syncthreads();  // the staging buffers and s_pair / s_rw are rewritten by the next tile
  }
}

}  // namespace

// Buffer offsets are 32-bit: an expert's data plane and the activations must stay
// under 2^31 bytes (T * cols * 2 is checked at launch).
bool gu_iq2_fits(int rows, int cols) {
  return rows > 0 && cols > 0 && cols % 256 == 0 && (long)rows * (cols / 256) * 64 < (1L << 31);
}

hipError_t launch_gu_iq2(const GemvParams& p, int n_slots, bool wide, hipStream_t s) {
  if (!gu_iq2_fits(p.rows, p.cols) || (long)p.T * p.cols * 2 >= (1L << 31)) return hipErrorInvalidValue;
  dim3 g((unsigned)((p.rows + GI_ROWS - 1) / GI_ROWS), (unsigned)n_slots);
  if (wide) hipLaunchKernelGGL(k_gu_iq2_wide, g, dim3(64 * GI_WAVES), 0, s, p);
  else hipLaunchKernelGGL(k_gu_iq2, g, dim3(64 * GI_WAVES), 0, s, p);
  return hipGetLastError();
}

// K a multiple of 256; the raw buffer offsets of an expert's planes and of the
// activations stay below 2^31.
bool dn_q2k_fits(int rows, int cols, long pairs) {
  return rows > 0 && cols > 0 && cols % 256 == 0 && (long)rows * (cols / 256) * 64 < (1L << 31) &&
         pairs * cols * 4 < (1L << 31);
}

hipError_t launch_dn_q2k(const GemvParams& p, int n_slots, hipStream_t s) {
  if (!dn_q2k_fits(p.rows, p.cols, (long)p.T * p.top_k)) return hipErrorInvalidValue;
  dim3 g((unsigned)((p.rows + GI_ROWS - 1) / GI_ROWS), (unsigned)n_slots);
  hipLaunchKernelGGL(k_dn_q2k, g, dim3(64 * GI_WAVES), 0, s, p);
  return hipGetLastError();
}

}  // namespace moeq

namespace moeq {

hipError_t launch_dn_iq2(const GemvParams& p, int n_slots, hipStream_t s) {
  if (!dn_q2k_fits(p.rows, p.cols, (long)p.T * p.top_k)) return hipErrorInvalidValue;
  dim3 g((unsigned)((p.rows + GI_ROWS - 1) / GI_ROWS), (unsigned)n_slots);
  hipLaunchKernelGGL(k_dn_iq2, g, dim3(64 * GI_WAVES), 0, s, p);
  return hipGetLastError();
}

}  // namespace moeq
