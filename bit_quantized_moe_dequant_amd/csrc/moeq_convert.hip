// Device versions of the lossless MXFP4 <-> NVFP4 scale re-encodes, one
// work-group per tensor (DeepSeek V4 Flash - REAP K180 Mixed NVFP4 card, section
// "NVFP4: lossless MXFP4->NVFP4 conversion" and "How It Was Built", step 3: the
// e2m1 nibbles are carried over unchanged and only the scales change).
//
// MXFP4 -> NVFP4: scale_2 = 2^(Emax - 135) with Emax the tensor's largest e8m0
// code, and both 16-halves of a block with code E get the e4m3 code of
// 2^(E - Emax + 8); exact when Emax - Emin <= 17 and no code is 255.
// NVFP4 -> MXFP4: exact when both halves of every 32-block carry the same e4m3
// scale and that scale times scale_2 is a power of two 2^k, -127 <= k <= 127
// (then E = k + 127). A tensor that cannot be carried exactly gets status 1 and
// its outputs are not written; the check runs over the whole tensor before any
// output is written.
#include <hip/hip_runtime.h>

#include "moeq_device.h"
#include "moeq_kernels.h"

namespace moeq {

namespace {

constexpr int CV_THREADS = 1024;

// e4m3 code of 2^k, -9 <= k <= 8
__device__ __forceinline__ uint32_t e4m3_pow2_code(int k) { return k >= -6 ? (uint32_t)(k + 7) << 3 : 1u << (k + 9); }

// Exponent k of a positive power-of-two e4m3 code, or a value outside [-9, 8]
// (the caller rejects it) for anything else.
__device__ __forceinline__ int e4m3_pow2_exponent(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  if (c & 0x80u) return 1000;                      // negative
  if (e != 0) return m == 0 ? (int)e - 7 : 1000;   // normal: mantissa must be zero
  if (m == 1) return -9;                           // subnormals 2^-9, 2^-8, 2^-7
  if (m == 2) return -8;
  if (m == 4) return -7;
  return 1000;                                     // zero or not a power of two
}

// Exponent of a positive finite fp32 power of two, or 1000.
__device__ __forceinline__ int f32_pow2_exponent(float f) {
  const uint32_t b = f2u(f);
  if (b & 0x80000000u) return 1000;
  const uint32_t e = (b >> 23) & 255u, m = b & 0x7FFFFFu;
  if (e == 255u) return 1000;
  if (e != 0) return m == 0 ? (int)e - 127 : 1000;
  if (m == 0 || (m & (m - 1))) return 1000;
  return (31 - __builtin_clz(m)) - 149;
}

__device__ void copy_plane(const uint8_t* src, uint8_t* dst, size_t bytes) {
  if (src == dst) return;
  for (size_t i = threadIdx.x; i < bytes / 16; i += CV_THREADS)
    reinterpret_cast<u32x4*>(dst)[i] = reinterpret_cast<const u32x4*>(src)[i];
}

__global__ __launch_bounds__(CV_THREADS) void k_mx4_to_nv4(const uint8_t* nib, const uint8_t* e8m0, int rows, int cols,
                                                           uint8_t* nib_out, uint8_t* e4m3_out, float* scale2_out,
                                                           uint32_t* status) {
  __shared__ int s_min, s_max, s_nan;
  const size_t nb = (size_t)rows * (cols / 32), nbytes = (size_t)rows * cols / 2;
  const int t = blockIdx.x;
  const uint8_t* e8 = e8m0 + t * nb;
  if (threadIdx.x == 0) {
    s_min = 255;
    s_max = 0;
    s_nan = 0;
  }
  __syncthreads();
  int lo = 255, hi = 0, nan = 0;
  for (size_t i = threadIdx.x; i < nb; i += CV_THREADS) {
    const int E = e8[i];
    nan |= E == 255;
    lo = min(lo, E);
    hi = max(hi, E);
  }
  atomicMin(&s_min, lo);
  atomicMax(&s_max, hi);
  if (nan) atomicOr(&s_nan, 1);
  __syncthreads();
  const int emax = s_max;
  const bool lossy = s_nan || emax - s_min > 17;
  if (threadIdx.x == 0) {
    status[t] = lossy ? 1u : 0u;
    if (!lossy) scale2_out[t] = __builtin_ldexpf(1.0f, emax - 135);
  }
  if (lossy) return;
  uint8_t* e4 = e4m3_out + t * 2 * nb;
  for (size_t i = threadIdx.x; i < nb; i += CV_THREADS) {
    const uint8_t c = (uint8_t)e4m3_pow2_code((int)e8[i] - emax + 8);
    e4[2 * i] = c;
    e4[2 * i + 1] = c;
  }
  copy_plane(nib + t * nbytes, nib_out + t * nbytes, nbytes);
}

__global__ __launch_bounds__(CV_THREADS) void k_nv4_to_mx4(const uint8_t* nib, const uint8_t* e4m3, const float* scale2,
                                                           int rows, int cols, uint8_t* nib_out, uint8_t* e8m0_out,
                                                           uint32_t* status) {
  __shared__ int s_bad;
  const size_t nb = (size_t)rows * (cols / 32), nbytes = (size_t)rows * cols / 2;
  const int t = blockIdx.x;
  const uint8_t* e4 = e4m3 + t * 2 * nb;
  const int k2 = f32_pow2_exponent(scale2[t]);
  if (threadIdx.x == 0) s_bad = k2 == 1000;
  __syncthreads();
  int bad = 0;
  for (size_t i = threadIdx.x; i < nb; i += CV_THREADS) {
    const uint32_t c0 = e4[2 * i], c1 = e4[2 * i + 1];
    const int k = e4m3_pow2_exponent(c0) + k2;
    bad |= (c0 != c1) || k < -127 || k > 127;
  }
  if (bad) atomicOr(&s_bad, 1);
  __syncthreads();
  const bool lossy = s_bad != 0;
  if (threadIdx.x == 0) status[t] = lossy ? 1u : 0u;
  if (lossy) return;
  uint8_t* e8 = e8m0_out + t * nb;
  for (size_t i = threadIdx.x; i < nb; i += CV_THREADS) e8[i] = (uint8_t)(e4m3_pow2_exponent(e4[2 * i]) + k2 + 127);
  copy_plane(nib + t * nbytes, nib_out + t * nbytes, nbytes);
}

}  // namespace

hipError_t launch_mx4_to_nv4(const uint8_t* nib, const uint8_t* e8m0, int rows, int cols, int n, uint8_t* nib_out,
                             uint8_t* e4m3_out, float* scale2_out, uint32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(k_mx4_to_nv4, dim3((unsigned)n), dim3(CV_THREADS), 0, s, nib, e8m0, rows, cols, nib_out, e4m3_out,
                     scale2_out, status);
  return hipGetLastError();
}

hipError_t launch_nv4_to_mx4(const uint8_t* nib, const uint8_t* e4m3, const float* scale2, int rows, int cols, int n,
                             uint8_t* nib_out, uint8_t* e8m0_out, uint32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(k_nv4_to_mx4, dim3((unsigned)n), dim3(CV_THREADS), 0, s, nib, e4m3, scale2, rows, cols, nib_out,
                     e8m0_out, status);
  return hipGetLastError();
}

}  // namespace moeq
