// Dense FP8 linear with power-of-two block scales on the block-scaled matrix
// instruction v_mfma_scale_f32_16x16x128_f8f6f4, E4M3 on both operands:
// y[t] = W x[t] for
//   * MXFP8 - E4M3 weights with one e8m0 scale per 32 along K, the format of the
//     checkpoint's attention, shared-expert and head weights (DeepSeekv4 Flash for
//     1x Spark forum thread, first post);
//   * MXFP8 pre-stored in the instruction's operand order (the same thread,
//     second post: the same bytes stored in the matrix engine's own layout, so
//     nothing is repacked at run time): each lane's 32 operand bytes and its scale
//     bytes are contiguous (see DecFp8 in moeq_device.h), so every load of the
//     weight stream is a 1 KB contiguous wave access;
//   * FP8 with one UE8M0 scale per 32 x 32 tile (DeepSeek-V4.1-Flash mixed-Q2 GGUF
//     card, Recipe): its scale is, for every row, a scale per 32 along K, i.e. an
//     MX block scale repeated over 32 rows.
// The block scale is the instruction's B scale, so no weight is decoded on the
// VALU. The bf16 tokens are operand A as two E4M3 terms each (hi + lo, one e8m0
// scale per 32 per term, the non-clipping exponent rule of the MXFP8 quantiser);
// A row m holds term m % 2 of token m / 2 of the pass, so one instruction serves
// eight tokens. A bf16 value is the sum of its two terms exactly unless it lies far
// below its block's maximum; the largest error of an element is 2^-21.8 of its
// block's maximum (the second term's scale is at most 2^-4 of the block maximum
// over 224, and its rounding error at most 2^-10 of that scale).
//
// Instruction layout (pinned on the device for E4M3 operand A; the B operand of
// the same type takes the same layout): lane L = n + 16g holds row (A) or column
// (B) n with bytes 0-15 at K = 16g + [0, 16) and bytes 16-31 at K = 64 + 16g +
// [0, 16) of the 128-wide step; the scale given by lane (., g) covers K-block g;
// output lane L register r = A row 4(L/16) + r, B column L % 16.
//
// Work: one work-group of eight waves per 16 weight rows; the waves take
// contiguous runs of K steps (a multiple of four steps each) and issue all their
// weight loads before any arithmetic; the tokens go through LDS eight (four at K
// above 4096) at a time, all of a pass's token loads issued before its
// conversion, which runs before the weight loads are issued in the first pass;
// the eight waves' partials are added in wave order. (Sixteen tokens per pass, two
// A tiles per step, needed 140 KB of LDS and 200+ registers: slower at every T.)
#include <hip/hip_runtime.h>

#include "moeq_device.h"
#include "moeq_kernels.h"

namespace moeq {

namespace {

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int M8_WAVES = 8;
constexpr int M8_TOK = 8;          // tokens per pass (A rows = token x term)
constexpr int M8_STAGE = 32768;    // staged x bytes per term per pass (tokens x K)

#ifndef MOEQ_MX8_XFIRST
#define MOEQ_MX8_XFIRST 1
#endif

template <int FMT, int STEPS>
__global__ __launch_bounds__(64 * M8_WAVES) void k_linear_mx8(Mx8Params P) {
  __shared__ uint8_t code[2][M8_STAGE];
  __shared__ uint8_t sc[2][M8_STAGE / 32];
  __shared__ float red[M8_WAVES][M8_TOK][16];
  constexpr bool TILED = FMT == FMT_MXFP8_TILED;
  constexpr int NT = 64 * M8_WAVES;
  constexpr int XC = M8_STAGE / 16 / NT;  // x chunks of 16 values per thread per pass, at most

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int r0 = blockIdx.x * 16;
  const int rn = r0 + n;  // rows is a multiple of 16
  const int K = P.cols;
  const int nsteps = K / 128;
  const int cpt = K / 16;                        // 16-value chunks per token
  const int tpp = min(M8_TOK, M8_STAGE / K);     // tokens per pass
  const int nxc = (tpp * cpt + NT - 1) / NT;     // chunk iterations per pass (uniform)
  const int spw = 4 * ((nsteps + 4 * M8_WAVES - 1) / (4 * M8_WAVES));
  const int s0 = wave * spw;
  const int my = max(0, min(spw, nsteps - s0));  // uniform per wave

  // Issue every x load of a pass, then convert: one memory round trip per pass.
  auto stage = [&](int t0) {
    const int tn = min(tpp, P.T - t0);
    u32x4 xa[XC], xb[XC];
#pragma unroll
    for (int j = 0; j < XC; j++) {
      xa[j] = u32x4{0u, 0u, 0u, 0u};
      xb[j] = xa[j];
      const int c = j * NT + (int)threadIdx.x;
      if (j < nxc && c < tn * cpt) {
        const uint16_t* xr = P.x + (size_t)(t0 + c / cpt) * K + (c % cpt) * 16;
        xa[j] = ld16(xr);
        xb[j] = ld16(xr + 8);
      }
    }
#pragma unroll
    for (int j = 0; j < XC; j++) {
      if (j < nxc) {  // uniform
        const int c = j * NT + (int)threadIdx.x;
        uint32_t w[2][4], E[2];
        bf16_terms(xa[j], xb[j], w, E);
        if (c < tn * cpt) {
          const int off = (c / cpt) * K + (c % cpt) * 16;
#pragma unroll
          for (int tm = 0; tm < 2; tm++) {
            *reinterpret_cast<u32x4*>(&code[tm][off]) = u32x4{w[tm][0], w[tm][1], w[tm][2], w[tm][3]};
            if ((c & 1) == 0) sc[tm][off / 32] = (uint8_t)E[tm];
          }
        }
      }
    }
  };

  // The first pass's tokens are converted before (MOEQ_MX8_XFIRST) or while the
  // weight loads go out.
  if (MOEQ_MX8_XFIRST) stage(0);
  __builtin_amdgcn_sched_barrier(0);

  // Every weight load of the wave (steps past its last re-read that one).
  u32x4 qa[STEPS], qb[STEPS];
  uint32_t sb[TILED ? (STEPS + 3) / 4 : STEPS];
#pragma unroll
  for (int i = 0; i < STEPS; i++) {
    const int s = min(s0 + min(i, max(my - 1, 0)), nsteps - 1);
    if constexpr (TILED) {
      const uint8_t* t = P.w + ((size_t)(r0 >> 4) * nsteps + s) * 2048 + 32 * lane;
      qa[i] = ld16(t);
      qb[i] = ld16(t + 16);
    } else {
      const uint8_t* t = P.w + (size_t)rn * K + 128 * s + 16 * g;
      qa[i] = ld16(t);
      qb[i] = ld16(t + 64);
    }
  }
#pragma unroll
  for (int i = 0; i < (TILED ? (STEPS + 3) / 4 : STEPS); i++) {
    if constexpr (TILED) {
      const int grp = min(s0 / 4 + i, nsteps / 4 - 1);
      sb[i] = *reinterpret_cast<const uint32_t*>(P.s + ((size_t)(r0 >> 4) * (K / 512) + grp) * 256 + 4 * lane);
    } else {
      const int s = min(s0 + min(i, max(my - 1, 0)), nsteps - 1);
      const int b = 4 * s + g;  // this lane's K-block
      size_t off;
      if constexpr (FMT == FMT_MXFP8) off = (size_t)rn * (K / 32) + b;
      else off = (size_t)(rn >> 5) * (K / 32) + b;  // FP8 block-32
      sb[i] = P.s[off];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if (!MOEQ_MX8_XFIRST) stage(0);

  const int tok = n >> 1, term = n & 1;  // this lane's A row
  for (int t0 = 0; t0 < P.T; t0 += tpp) {
    const int tn = min(tpp, P.T - t0);
    if (t0 > 0) {
      __syncthreads();  // the previous pass has read the staging
      stage(t0);
    }
    __syncthreads();

    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < STEPS; i++) {
      if (i < my) {
        const int s = s0 + i;
        u32x4 a0 = u32x4{0u, 0u, 0u, 0u}, a1 = a0;
        int sa = 0;
        if (tok < tn) {
          const int off = tok * K + 128 * s + 16 * g;
          a0 = *reinterpret_cast<const u32x4*>(&code[term][off]);
          a1 = *reinterpret_cast<const u32x4*>(&code[term][off + 64]);
          sa = sc[term][(tok * K) / 32 + 4 * s + g];
        }
        const i32x8_t av = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
        const i32x8_t bv = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(qa[i], qb[i], 0, 1, 2, 3, 4, 5, 6, 7));
        const int sbv = TILED ? (int)((sb[i >> 2] >> (8 * (i & 3))) & 255u) : (int)sb[i];
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0, 0, 0, sa, 0, sbv);
      }
    }
    // lane (column n, g): registers 0, 1 = token 2g (terms), 2, 3 = token 2g + 1
    red[wave][2 * g][n] = acc[0] + acc[1];
    red[wave][2 * g + 1][n] = acc[2] + acc[3];
    __syncthreads();
    if (threadIdx.x < 16 * M8_TOK) {
      const int tk = threadIdx.x >> 4, col = threadIdx.x & 15;
      if (tk < tn) {
        float v = 0.f;
#pragma unroll
        for (int wv = 0; wv < M8_WAVES; wv++) v += red[wv][tk][col];
        P.y[(size_t)(t0 + tk) * P.rows + r0 + col] = v;
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // unused weight re-reads land before the end
}

// Row-major MXFP8 -> the pre-stored operand order, for n tensors back to back.
__global__ __launch_bounds__(256) void k_mxfp8_tile(const uint8_t* data, const uint8_t* scales, int rows, int cols,
                                                    uint8_t* tdata, uint8_t* tscales) {
  const size_t plane = (size_t)rows * cols;
  data += blockIdx.y * plane;
  tdata += blockIdx.y * plane;
  scales += blockIdx.y * (plane / 32);
  tscales += blockIdx.y * (plane / 32);
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int L = (int)(idx & 63), n = L & 15, g = L >> 4;
  const size_t tiles = (size_t)(rows / 16) * (cols / 128);
  if (idx / 64 < tiles) {
    const size_t tile = idx / 64;
    const int rt = (int)(tile / (cols / 128)), kt = (int)(tile % (cols / 128));
    const uint8_t* src = data + (size_t)(16 * rt + n) * cols + 128 * kt + 16 * g;
    uint8_t* dst = tdata + tile * 2048 + 32 * L;
    *reinterpret_cast<u32x4*>(dst) = ld16(src);
    *reinterpret_cast<u32x4*>(dst + 16) = ld16(src + 64);
  }
  const size_t groups = (size_t)(rows / 16) * (cols / 512);
  if (idx / 64 < groups) {
    const size_t grp = idx / 64;
    const int rt = (int)(grp / (cols / 512)), kg = (int)(grp % (cols / 512));
    const uint8_t* src = scales + (size_t)(16 * rt + n) * (cols / 32) + 16 * kg + g;
    const uint32_t v = (uint32_t)src[0] | ((uint32_t)src[4] << 8) | ((uint32_t)src[8] << 16) | ((uint32_t)src[12] << 24);
    *reinterpret_cast<uint32_t*>(tscales + grp * 256 + 4 * L) = v;
  }
}

template <int FMT>
hipError_t go(const Mx8Params& p, hipStream_t s) {
  const dim3 g((unsigned)(p.rows / 16)), b(64 * M8_WAVES);
  if (p.cols <= 4096) hipLaunchKernelGGL((k_linear_mx8<FMT, 4>), g, b, 0, s, p);
  else hipLaunchKernelGGL((k_linear_mx8<FMT, 8>), g, b, 0, s, p);
  return hipGetLastError();
}

}  // namespace

bool linear_mx8_fits(int fmt, int rows, int cols) {
  if (rows <= 0 || cols <= 0 || rows % 16 || cols % 128 || cols > 8192) return false;
  if (fmt == FMT_MXFP8_TILED) return cols % 512 == 0;
  if (fmt == FMT_FP8_B32) return rows % 32 == 0;
  return fmt == FMT_MXFP8;
}

hipError_t launch_linear_mx8(int fmt, const Mx8Params& p, hipStream_t s) {
  if (!linear_mx8_fits(fmt, p.rows, p.cols) || p.T < 1) return hipErrorInvalidValue;
  switch (fmt) {
    case FMT_MXFP8: return go<FMT_MXFP8>(p, s);
    case FMT_MXFP8_TILED: return go<FMT_MXFP8_TILED>(p, s);
    case FMT_FP8_B32: return go<FMT_FP8_B32>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_mxfp8_tile(const uint8_t* data, const uint8_t* scales, int rows, int cols, int n, uint8_t* tdata,
                             uint8_t* tscales, hipStream_t s) {
  if (rows <= 0 || cols <= 0 || rows % 16 || cols % 512 || n <= 0) return hipErrorInvalidValue;
  const size_t threads = (size_t)(rows / 16) * (cols / 128) * 64;  // one per (tile, lane); covers the scale groups
  hipLaunchKernelGGL(k_mxfp8_tile, dim3((unsigned)((threads + 255) / 256), (unsigned)n), dim3(256), 0, s, data, scales,
                     rows, cols, tdata, tscales);
  return hipGetLastError();
}

}  // namespace moeq
