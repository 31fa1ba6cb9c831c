// Routing, combine, MXFP8 activation quantisation and ggml block repack kernels.
#include "moeq_device.h"
#include "moeq_kernels.h"

namespace moeq {

// ---------------------------------------------------------------- routing
// Counting sort of the T*K (token, slot) pairs by expert, in one work-group.
// Out-of-range ids go to an extra bucket E (and set the device error bit) so the
// GEMV kernels can zero their outputs. Within a bucket the order of pairs may vary
// from run to run; every pair's result is computed independently of its position,
// so outputs do not depend on it.
constexpr int ROUTE_MAX_E = 1024;

__device__ int block_exclusive_scan(int v, int* tmp) {
  // Exclusive prefix over blockDim.x (a multiple of 64, <= 1024) values: an
  // inclusive scan inside each wave by lane shuffles, then wave 0 scans the wave
  // totals; three barriers in all. tmp holds at least 128 ints.
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) tmp[w] = x;
  __syncthreads();
  if (t < 64) {
    int s = t < (int)(blockDim.x >> 6) ? tmp[t] : 0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(s, off, 64);
      if (t >= off) s += y;
    }
    tmp[64 + t] = s;  // inclusive prefix of the wave totals
  }
  __syncthreads();
  const int incl = (w > 0 ? tmp[64 + w - 1] : 0) + x;
  __syncthreads();  // tmp is reused by the next scan
  return incl - v;
}

__global__ __launch_bounds__(1024) void k_route(const int32_t* ids, int P, int E, RouteView rv, uint32_t* err) {
  __shared__ int cnt[ROUTE_MAX_E + 1];
  __shared__ int cur[ROUTE_MAX_E + 1];
  __shared__ int tmp[1024];
  __shared__ int total_valid_slots;
  const int t = threadIdx.x;
  for (int i = t; i <= E; i += blockDim.x) cnt[i] = 0;
  __syncthreads();
  // Both passes over the ids read eight per thread before using any, so the
  // loads overlap instead of each waiting a memory round trip.
  constexpr int RB = 8;
  bool any_bad = false;
  for (int p0 = t; p0 < P; p0 += RB * (int)blockDim.x) {
    int ev[RB];
#pragma unroll
    for (int j = 0; j < RB; j++) {
      const int p = p0 + j * (int)blockDim.x;
      ev[j] = p < P ? ids[p] : 0;
    }
#pragma unroll
    for (int j = 0; j < RB; j++) {
      if (p0 + j * (int)blockDim.x >= P) break;
      int e = ev[j];
      if (e < 0 || e >= E) {
        e = E;
        any_bad = true;
      }
      atomicAdd(&cnt[e], 1);
    }
  }
  if (any_bad) atomicOr(err, 1u);  // expert id out of range
  __syncthreads();
  // Buckets 0..E (E + 1 <= 1025 values); thread t owns buckets 2t, 2t + 1.
  int b0 = 2 * t, b1 = 2 * t + 1;
  int c0 = b0 <= E ? cnt[b0] : 0, c1 = b1 <= E ? cnt[b1] : 0;
  int f0 = (b0 < E && c0 > 0) ? 1 : 0, f1 = (b1 < E && c1 > 0) ? 1 : 0;
  int off = block_exclusive_scan(c0 + c1, tmp);
  int soff = block_exclusive_scan(f0 + f1, tmp);
  // prefill work items: ceil(count / MC) per bucket, in bucket order
  const int h0 = (c0 + PREFILL_MC - 1) / PREFILL_MC, h1 = (c1 + PREFILL_MC - 1) / PREFILL_MC;
  const int hoff = block_exclusive_scan(h0 + h1, tmp);
  for (int j = 0; j < h0; j++) {
    rv.chunk_e()[hoff + j] = b0;
    rv.chunk_m0()[hoff + j] = j * PREFILL_MC;
  }
  for (int j = 0; j < h1; j++) {
    rv.chunk_e()[hoff + h0 + j] = b1;
    rv.chunk_m0()[hoff + h0 + j] = j * PREFILL_MC;
  }
  if (t == (int)blockDim.x - 1) rv.n_chunks()[0] = hoff + h0 + h1;
  if (b0 <= E) {
    rv.offsets()[b0] = off;
    cur[b0] = off;
    if (f0) rv.slots()[soff] = b0;
  }
  if (b1 <= E) {
    rv.offsets()[b1] = off + c0;
    cur[b1] = off + c0;
    if (f1) rv.slots()[soff + f0] = b1;
  }
  if (t == (int)blockDim.x - 1) total_valid_slots = soff + f0 + f1;
  __syncthreads();
  if (t == 0) {
    rv.offsets()[E + 1] = P;
    int ns = total_valid_slots;
    if (cnt[E] > 0) rv.slots()[ns++] = E;
    rv.n_slots()[0] = ns;
  }
  __syncthreads();
  for (int p0 = t; p0 < P; p0 += RB * (int)blockDim.x) {
    int ev[RB];
#pragma unroll
    for (int j = 0; j < RB; j++) {
      const int p = p0 + j * (int)blockDim.x;
      ev[j] = p < P ? ids[p] : 0;
    }
#pragma unroll
    for (int j = 0; j < RB; j++) {
      const int p = p0 + j * (int)blockDim.x;
      if (p >= P) break;
      int e = ev[j];
      if (e < 0 || e >= E) e = E;
      const int pos = atomicAdd(&cur[e], 1);
      rv.perm()[pos] = p;
    }
  }
}

hipError_t launch_route(const int32_t* ids, int P, int E, RouteView rv, uint32_t* err, hipStream_t s) {
  if (E > ROUTE_MAX_E) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_route, dim3(1), dim3(1024), 0, s, ids, P, E, rv, err);
  return hipGetLastError();
}

// ---------------------------------------------------------------- combine
// y[t][r] = sum over k in slot order of partial[t*K + k][r]; four outputs per
// thread (H is a multiple of 4: every format's K-block is).
__global__ __launch_bounds__(256) void k_combine(const float* partial, int T, int K, int H, float* y) {
  const size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= (size_t)T * H) return;
  const size_t t = i / H, r = i % H;
  const float* p = partial + t * K * (size_t)H + r;
  float4 acc = *reinterpret_cast<const float4*>(p);
  for (int k = 1; k < K; k++) {
    const float4 v = *reinterpret_cast<const float4*>(p + (size_t)k * H);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  *reinterpret_cast<float4*>(y + i) = acc;
}

hipError_t launch_combine(const float* partial, int T, int K, int H, float* y, hipStream_t s) {
  const size_t n = (size_t)T * H / 4;
  hipLaunchKernelGGL(k_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, partial, T, K, H, y);
  return hipGetLastError();
}

// ---------------------------------------------------------------- MXFP8 quantisation
// Per 32 consecutive values: E = clamp(e + 127, 0, 254) with e chosen so the block
// maximum a = m 2^p (m in [0.5, 1)) maps to a / 2^e <= 448 without clipping
// (e = p - 9 if m <= 0.875 else p - 8); all-zero blocks get E = 0 and codes 0;
// elements are rounded to nearest even onto E4M3FN, saturating, sign kept.
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  uint32_t sign = (__builtin_bit_cast(uint32_t, v) >> 24) & 0x80u;
  float a = __builtin_fabsf(v);
  uint32_t code;
  if (!(a < 448.0f)) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {               // below 2^-6: subnormal steps of 2^-9
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    int e = (int)((__builtin_bit_cast(uint32_t, a) >> 23) & 0xFFu) - 127;
    uint32_t q = (uint32_t)__builtin_rintf(__builtin_ldexpf(a, 3 - e));  // 8..16
    if (q == 16u) {
      e += 1;
      q = 8u;
    }
    code = ((uint32_t)(e + 7) << 3) | (q - 8u);
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return code | sign;
}

template <int IN_F32>
__global__ __launch_bounds__(256) void k_quant_mxfp8(const void* x, int T, int K, uint8_t* q, uint8_t* es) {
  size_t b = (size_t)blockIdx.x * blockDim.x + threadIdx.x;  // block index
  const int nb = K / 32;
  if (b >= (size_t)T * nb) return;
  float v[32];
  if (IN_F32) {
    const float* p = reinterpret_cast<const float*>(x) + b * 32;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      u32x4 w = ld16(p + 4 * i);
      v[4 * i + 0] = u2f(w[0]);
      v[4 * i + 1] = u2f(w[1]);
      v[4 * i + 2] = u2f(w[2]);
      v[4 * i + 3] = u2f(w[3]);
    }
  } else {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(x) + b * 32;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      u32x4 w = ld16(p + 8 * i);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        v[8 * i + 2 * j] = u2f(w[j] << 16);
        v[8 * i + 2 * j + 1] = u2f(w[j] & 0xFFFF0000u);
      }
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; i++) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
  uint32_t ab = __builtin_bit_cast(uint32_t, amax);
  uint32_t E;
  if (ab < 0x00800000u) {
    E = 0u;  // zero or subnormal maximum: e + 127 < 0
  } else {
    int p = (int)(ab >> 23) - 126;                 // amax = m 2^p, m in [0.5, 1)
    uint32_t frac = ab & 0x007FFFFFu;              // m = (1 + frac / 2^23) / 2
    int e = (frac <= 0x00600000u) ? p - 9 : p - 8;  // m <= 0.875  <=>  frac <= 0.75 * 2^23
    int Ei = e + 127;
    E = (uint32_t)(Ei < 0 ? 0 : (Ei > 254 ? 254 : Ei));
  }
  // The hardware conversion with the block scale as its scale operand (the e8m0
  // code in a float's exponent field) divides by 2^(E - 127) and rounds to nearest
  // even onto E4M3FN, as e4m3_rne does for every finite value: under this exponent
  // rule a finite value never exceeds 448 after scaling. Infinities and NaNs, which
  // the conversion turns into NaN codes, saturate to 448 with their sign as in
  // e4m3_rne. Blocks whose maximum is below 2^-105 take e4m3_rne itself: only there
  // can an fp32 subnormal element scale into E4M3's range, and the conversion's
  // handling of subnormal inputs is not relied on.
  uint32_t out[8];
  if (ab < 0x0B000000u) {
    const int shift = 127 - (int)E;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      uint32_t w = 0;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const uint32_t c = (amax == 0.f) ? 0u : e4m3_rne(__builtin_ldexpf(v[4 * i + j], shift));
        w |= c << (8 * j);
      }
      out[i] = w;
    }
  } else {
    const float scale = u2f(E << 23);
#pragma unroll
    for (int i = 0; i < 8; i++) {
      typedef short i16x2_t __attribute__((ext_vector_type(2)));
      const i16x2_t lo =
          __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(i16x2_t{0, 0}, v[4 * i], v[4 * i + 1], scale, false);
      const i16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, v[4 * i + 2], v[4 * i + 3], scale, true);
      uint32_t w = __builtin_bit_cast(uint32_t, hi);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const float a = v[4 * i + j];
        if (!(__builtin_fabsf(a) <= 3.402823466e38f))
          w = (w & ~(0xFFu << (8 * j))) | ((0x7Eu | ((f2u(a) >> 24) & 0x80u)) << (8 * j));
      }
      out[i] = w;
    }
  }
  u32x4* qo = reinterpret_cast<u32x4*>(q + b * 32);
  qo[0] = u32x4{out[0], out[1], out[2], out[3]};
  qo[1] = u32x4{out[4], out[5], out[6], out[7]};
  es[b] = (uint8_t)E;
}

hipError_t launch_quant_mxfp8(int in_f32, const void* x, int T, int K, uint8_t* q, uint8_t* e, hipStream_t s) {
  size_t nb = (size_t)T * (K / 32);
  dim3 g((unsigned)((nb + 255) / 256)), b(256);
  if (in_f32) hipLaunchKernelGGL(k_quant_mxfp8<1>, g, b, 0, s, x, T, K, q, e);
  else hipLaunchKernelGGL(k_quant_mxfp8<0>, g, b, 0, s, x, T, K, q, e);
  return hipGetLastError();
}

// ---------------------------------------------------------------- ggml repack
// Q2_K block (84 B: scales[16] qs[64] d dmin) -> qs plane (64 B) + scale plane
// (20 B: scales[16] d dmin). IQ2_XXS block (66 B: d, 64 B) -> data (64 B) + d (2 B).
__global__ __launch_bounds__(256) void k_pack(int fmt, const uint8_t* blocks, size_t nblk, uint8_t* data,
                                              uint8_t* scales) {
  size_t b = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblk) return;
  if (fmt == FMT_Q2_K) {
    const uint8_t* s = blocks + b * 84;
    uint8_t* d = data + b * 64;
    uint8_t* c = scales + b * 20;
    for (int i = 0; i < 64; i++) d[i] = s[16 + i];
    for (int i = 0; i < 16; i++) c[i] = s[i];
    for (int i = 0; i < 4; i++) c[16 + i] = s[80 + i];
  } else {
    const uint8_t* s = blocks + b * 66;
    uint8_t* d = data + b * 64;
    uint8_t* c = scales + b * 2;
    for (int i = 0; i < 64; i++) d[i] = s[2 + i];
    c[0] = s[0];
    c[1] = s[1];
  }
}

hipError_t launch_pack(int fmt, const uint8_t* blocks, int rows, int cols, int n, uint8_t* data, uint8_t* scales,
                       hipStream_t s) {
  size_t nblk = (size_t)n * rows * (cols / 256);
  hipLaunchKernelGGL(k_pack, dim3((unsigned)((nblk + 255) / 256)), dim3(256), 0, s, fmt, blocks, nblk, data, scales);
  return hipGetLastError();
}

__global__ void k_clear_words(uint32_t* p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

hipError_t launch_clear_words(uint32_t* p, int n, hipStream_t s) {
  hipLaunchKernelGGL(k_clear_words, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace moeq
