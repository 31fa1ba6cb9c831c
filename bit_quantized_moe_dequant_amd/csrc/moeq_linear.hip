// Dense FP8 block-128 linear for two or more tokens: y[t] = W x[t], with W given as
// E4M3 codes and one UE8M0 scale per 128x128 tile (IQ2_XXS + Q2_K + FP8 hybrid
// card, format table; DeepSeek-V4-Flash W4A16-FP8 card, FP8 128x128 blocks), x in
// bf16, y in fp32.
//
// A token batch turns the GEMV into a small dense contraction (rows x tokens x K),
// so it runs on the bf16 matrix instruction v_mfma_f32_16x16x32_bf16 with the
// weights as operand A (16 rows) and the tokens as operand B (16 columns). Every
// E4M3 code is exact in bf16, every product of two bf16 values is exact in fp32,
// and the block scale is a power of two applied to the fp32 partial of its
// 128-wide K tile, so the only roundings are those of the fp32 accumulation.
//
// Work: one work-group of 16 waves per 16 weight rows. K advances in steps of 256
// (two scale tiles); the 16 waves take the steps round robin, so each weight byte
// is read once, and the per-wave partials are summed in LDS in wave order (the
// result does not depend on timing). A lane (row lr = lane % 16, group g = lane /
// 16) reads the 32 contiguous bytes at K = 32g + [0, 32) of each 128-wide tile of
// its row; instruction j (j = 0..3) of a tile takes bytes 8j..8j+7 of that run.
// The contraction is a sum, so any order of K is the same product as long as both
// operands follow it: the token lane (t, g) reads the bf16 values at the same K.
// Output lane L register r of the instruction is row 4(L/16) + r, token L % 16.
#include <hip/hip_runtime.h>

#include "moeq_device.h"
#include "moeq_kernels.h"

namespace moeq {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

#ifndef MOEQ_LN_WAVES
#define MOEQ_LN_WAVES 16
#endif
constexpr int LN_WAVES = MOEQ_LN_WAVES;
static_assert(LN_WAVES % 4 == 0 && LN_WAVES <= 16, "whole 256-thread groups");
constexpr int LN_THREADS = 64 * LN_WAVES;
constexpr int LN_ROWS = 16;    // weight rows per work-group
constexpr int LN_KSTEP = 256;  // K per step (two 128-wide scale tiles)
constexpr int LN_TG = 4;       // token tiles of 16 per pass over the weights

// bf16 A fragment of instruction j: weight bytes 8(j%2)..8(j%2)+7 of the 16-byte
// load j/2, element i = byte i.
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint32_t d0, uint32_t d1) {
  bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false);
  bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true);
  bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false);
  bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true);
  return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__global__ __launch_bounds__(LN_THREADS) void k_linear_fp8(LinearParams P) {
  __shared__ float red[LN_WAVES][LN_TG][256];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lr = lane & 15;
  const int g = lane >> 4;
  const int r0 = blockIdx.x * LN_ROWS;
  const int nsteps = P.cols / LN_KSTEP;
  const uint8_t* wrow = P.w + (size_t)(r0 + lr) * P.cols + 32 * g;
  const uint8_t* srow = P.s + (size_t)(r0 >> 7) * (P.cols >> 7);
  const int ntiles = (P.T + 15) >> 4;

  for (int tg = 0; tg < ntiles; tg += LN_TG) {
    f32x4_t acc[LN_TG];
#pragma unroll
    for (int ti = 0; ti < LN_TG; ti++) acc[ti] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int s = wave; s < nsteps; s += LN_WAVES) {
      const int k0 = s * LN_KSTEP;
      u32x4 wq[2][2];
#pragma unroll
      for (int h = 0; h < 2; h++) {
        wq[h][0] = ld16(wrow + k0 + 128 * h);
        wq[h][1] = ld16(wrow + k0 + 128 * h + 16);
      }
      const float sc0 = e8m0_f32(srow[k0 >> 7]);
      const float sc1 = e8m0_f32(srow[(k0 >> 7) + 1]);
#pragma unroll
      for (int ti = 0; ti < LN_TG; ti++) {
        if (tg + ti < ntiles) {
          const int tok = min(((tg + ti) << 4) + lr, P.T - 1);
          const uint16_t* xr = P.x + (size_t)tok * P.cols + k0 + 32 * g;
          u32x4 xv[2][4];
#pragma unroll
          for (int h = 0; h < 2; h++)
#pragma unroll
            for (int j = 0; j < 4; j++) xv[h][j] = ld16(xr + 128 * h + 8 * j);
          f32x4_t c[2];
#pragma unroll
          for (int h = 0; h < 2; h++) {
            c[h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; j++) {
              const u32x4 q = wq[h][j >> 1];
              const int d = 2 * (j & 1);
              c[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(q[d], q[d + 1]),
                                                             __builtin_bit_cast(bf16x8_t, xv[h][j]), c[h], 0, 0, 0);
            }
          }
#pragma unroll
          for (int r = 0; r < 4; r++) acc[ti][r] = __builtin_fmaf(c[1][r], sc1, __builtin_fmaf(c[0][r], sc0, acc[ti][r]));
        }
      }
    }

    // Partials of this wave: lane L register r = row 4(L/16) + r, token L % 16,
    // stored token-major so that the sums below write 16 consecutive rows.
#pragma unroll
    for (int ti = 0; ti < LN_TG; ti++)
#pragma unroll
      for (int r = 0; r < 4; r++) red[wave][ti][lr * 16 + 4 * g + r] = acc[ti][r];
    __syncthreads();
    // 256 sums per token tile, one per thread (several tiles per thread when the
    // work-group has fewer than 256 LN_TG threads)
    for (int ti = (int)threadIdx.x >> 8; ti < LN_TG; ti += LN_THREADS / 256) {
      const int idx = threadIdx.x & 255;
      const int tok = ((tg + ti) << 4) + (idx >> 4);
      if (tg + ti < ntiles && tok < P.T) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < LN_WAVES; w++) v += red[w][ti][idx];
        P.y[(size_t)tok * P.rows + r0 + (idx & 15)] = v;
      }
    }
    __syncthreads();
  }
}

}  // namespace

bool linear_fp8_fits(int rows, int cols) {
  return rows > 0 && cols > 0 && rows % 128 == 0 && cols % LN_KSTEP == 0;
}

hipError_t launch_linear_fp8(const LinearParams& p, hipStream_t s) {
  if (!linear_fp8_fits(p.rows, p.cols) || p.T < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_linear_fp8, dim3((unsigned)(p.rows / LN_ROWS)), dim3(LN_THREADS), 0, s, p);
  return hipGetLastError();
}

}  // namespace moeq
